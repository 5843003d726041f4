// Device building blocks shared by the MFMA kernels of the GMA forward (gfx950, wave64).
//
// Responsibility logits as a matrix-core contraction.  For a diagonal Gaussian the
// log joint of component k at routing vector x is, in log2 units and up to a term that is
// the same for every k of a row (and so cancels in the softmax over k),
//     l_k(x) = c_k + sum_d a_kd x_d^2 + b_kd x_d,
//     a_kd = -log2(e) / (2 var_kd),  b_kd = log2(e) mu_kd / var_kd,
//     c_k  = log2(e) (p_k - 1/2 sum_d (log var_kd + mu_kd^2 / var_kd)),
// with var = softplus(var_raw) + var_floor and p the prior logits (softmax priors; the
// normalising log-sum-exp of p is row-constant and dropped).  Logits reach hundreds to
// thousands in magnitude, but the softmax needs them to ~1e-3 absolute, far beyond one
// bf16 operand (8 significant bits).  So both operands are split into bf16 pieces whose
// products are exact in the fp32 accumulator:
//     x is bf16 already (exact); x^2 = x2h + x2l exactly (x^2 has <= 16 significant bits);
//     a = ah + al, b = bh + bl (each to ~2^-17 relative);
//     l = c + ah.x2h + al.x2h + ah.x2l + bh.x + bl.x   (the al.x2l term, ~2^-17 of a x^2,
//                                                      is dropped).
// That is five 32x32x16 MFMAs per 16-wide chunk of the routing dimension; c_k seeds the
// accumulator.
//
// MFMA 32x32x16 bf16 register layouts (checked on the device):
//   A (32 x 16):  lane l holds A[l % 32][8 (l / 32) + j], j = 0..7
//   B (16 x 32):  lane l holds B[8 (l / 32) + j][l % 32]
//   C (32 x 32):  lane l, register i holds C[8 (i / 4) + 4 (l / 32) + (i % 4)][l % 32]
// The logits are computed as C[k][t] (components on rows, tokens on columns), so one lane
// holds one token and 16 of every 32 components: the softmax over k is in-lane plus one
// exchange with lane l ^ 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gma_numeric.h"

namespace gma {
namespace mf {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileT = 32;                   // tokens per wave tile (MFMA N)
constexpr int kIterT = kTileT * kWaves;      // tokens per workgroup iteration
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA (fp32 accumulate), layouts:
//   A (16 x 32): lane l holds A[l % 16][8 (l / 16) + j];  B (32 x 16): lane l holds B[8 (l / 16) + j][l % 16];
//   C (16 x 16): lane l, register i holds C[4 (l / 16) + i][l % 16].
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Value held by lane l ^ 32 (the other half of the wave), for x uniform per half-lane pair.
__device__ __forceinline__ float max_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// fp32 -> bf16 round to nearest even (inputs here are finite or +-inf).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// B-operand pieces of one 16-wide chunk of routing dims for one token: this lane's 8 bf16
// values x (already in `x1`), and the exact split x^2 = x2h + x2l.
struct XFrag {
    bf16x8 x1, x2h, x2l;
};

__device__ __forceinline__ void split_square(XFrag& f) {
    const u32x4 xp = __builtin_bit_cast(u32x4, f.x1);
    u32x4 hp, lp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float x0 = bf16lo_to_f32(xp[j]), x1 = bf16hi_to_f32(xp[j]);
        const float s0 = x0 * x0, s1 = x1 * x1;  // exact: <= 16 significant bits
        const uint32_t h = pack_bf16(s0, s1);
        hp[j] = h;
        // residuals are exact in fp32 and have <= 8 significant bits: exact in bf16
        lp[j] = pack_bf16(s0 - bf16lo_to_f32(h), s1 - bf16hi_to_f32(h));
    }
    f.x2h = __builtin_bit_cast(bf16x8, hp);
    f.x2l = __builtin_bit_cast(bf16x8, lp);
}

// Load this lane's 8 routing values of chunk `c` of a token row: dims 16c + 8h .. 16c + 8h + 7,
// zero beyond d_r (d_r is a multiple of 8 on this path, so a chunk half is all in or all out).
__device__ __forceinline__ bf16x8 load_x8(const bf16_t* row, int c, int h, int dr) {
    bf16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    const int d0 = 16 * c + 8 * h;
    if (d0 < dr) v = *reinterpret_cast<const bf16x8*>(row + d0);
    return v;
}

// This lane's raw routing values of one token row, all NC chunks (issued together so the
// loads of the next tile can be in flight while the current tile computes).
template <int NC>
__device__ __forceinline__ void load_xrow(bf16x8 (&xr)[NC], const bf16_t* row, int dr) {
    const int h = lane_id() >> 5;
#pragma unroll
    for (int c = 0; c < NC; ++c) xr[c] = load_x8(row, c, h, dr);
}

// Logits of one 32-token tile against all MT*32 components:
//   acc[m] = C[k = 32m + row][t] (layout above), seeded with c_k.
// sW: coefficient rows in LDS, row k = [ah(Dp) | al(Dp) | bh(Dp) | bl(Dp)] bf16, Dp = 16 NC,
// row stride `wstride` bytes; sC: c_k (float).  Consecutive MFMAs go to different
// accumulators (the MT component tiles) so they do not wait on each other.
template <int MT, int NC>
__device__ __forceinline__ void tile_logits(f32x16 (&acc)[MT], const bf16x8* xr, const unsigned char* sW,
                                            int wstride, const float* sC, bool init = true) {
    const int l = lane_id();
    const int h = l >> 5;
    constexpr int Dp = 16 * NC;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (!init) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 cq = *reinterpret_cast<const float4*>(sC + 32 * m + 8 * q + 4 * h);
            acc[m][4 * q] = cq.x;
            acc[m][4 * q + 1] = cq.y;
            acc[m][4 * q + 2] = cq.z;
            acc[m][4 * q + 3] = cq.w;
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        XFrag f;
        f.x1 = xr[c];
        split_square(f);
        const unsigned char* wr = sW + (size_t)(l & 31) * wstride + (16 * c + 8 * h) * 2;
        // component tiles in groups of up to four: the group's 4 x 4 coefficient fragments
        // stay in registers while its 20 MFMAs cycle over 4 independent accumulators
        constexpr int MG = MT < 4 ? MT : 4;
#pragma unroll
        for (int g0 = 0; g0 < MT; g0 += MG) {
            bf16x8 ah[MG], al[MG], bh[MG], bl[MG];
#pragma unroll
            for (int m = 0; m < MG; ++m) {
                const unsigned char* wm = wr + (size_t)32 * (g0 + m) * wstride;
                ah[m] = *reinterpret_cast<const bf16x8*>(wm);
                al[m] = *reinterpret_cast<const bf16x8*>(wm + 2 * Dp);
                bh[m] = *reinterpret_cast<const bf16x8*>(wm + 4 * Dp);
                bl[m] = *reinterpret_cast<const bf16x8*>(wm + 6 * Dp);
            }
#pragma unroll
            for (int m = 0; m < MG; ++m) acc[g0 + m] = mfma(ah[m], f.x2h, acc[g0 + m]);
#pragma unroll
            for (int m = 0; m < MG; ++m) acc[g0 + m] = mfma(bh[m], f.x1, acc[g0 + m]);
#pragma unroll
            for (int m = 0; m < MG; ++m) acc[g0 + m] = mfma(al[m], f.x2h, acc[g0 + m]);
#pragma unroll
            for (int m = 0; m < MG; ++m) acc[g0 + m] = mfma(bl[m], f.x1, acc[g0 + m]);
#pragma unroll
            for (int m = 0; m < MG; ++m) acc[g0 + m] = mfma(ah[m], f.x2l, acc[g0 + m]);
            // keep later groups' coefficient loads from being hoisted here (registers)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Software-pipelined logits.  The contraction of one tile is cut into units (a 16-wide chunk
// of routing dims x a group of up to 4 component tiles: 16 coefficient fragments, 20 MFMAs).
// The fragments of unit u+1 are loaded while unit u's MFMAs run, and `work(u, U)` -- VALU
// work of another tile (its softmax, packing, stores) -- sits in the same scheduling region
// as unit u's MFMAs, so the two interleave on one SIMD.  Regions are closed by
// sched_barrier so nothing drifts across units (register pressure stays bounded).
template <int MG>
struct WFrag {
    bf16x8 ah[MG], al[MG], bh[MG], bl[MG];
};

template <int MG, int Dp>
__device__ __forceinline__ void load_wfrag(WFrag<MG>& f, const unsigned char* sW, int wstride, int c, int g0) {
    const int l = lane_id(), h = l >> 5;
    const unsigned char* wr = sW + (size_t)(l & 31) * wstride + (16 * c + 8 * h) * 2;
#pragma unroll
    for (int m = 0; m < MG; ++m) {
        const unsigned char* wm = wr + (size_t)32 * (g0 + m) * wstride;
        f.ah[m] = *reinterpret_cast<const bf16x8*>(wm);
        f.al[m] = *reinterpret_cast<const bf16x8*>(wm + 2 * Dp);
        f.bh[m] = *reinterpret_cast<const bf16x8*>(wm + 4 * Dp);
        f.bl[m] = *reinterpret_cast<const bf16x8*>(wm + 6 * Dp);
    }
}

template <int MT, int NC, bool INIT = true, int MGMAX = 2, typename Work>
__device__ __forceinline__ void tile_logits_overlap(f32x16 (&acc)[MT], const bf16x8* xr, const unsigned char* sW,
                                                    int wstride, const float* sC, Work&& work) {
    // MG accumulators alternate (up to MGMAX); the fragments of two units are in flight
    constexpr int MG = MT < MGMAX ? MT : MGMAX;
    constexpr int GPC = MT / MG;  // groups per chunk
    constexpr int U = NC * GPC;
    constexpr int Dp = 16 * NC;
    const int h = lane_id() >> 5;
#pragma unroll
    for (int m = 0; m < (INIT ? MT : 0); ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 cq = *reinterpret_cast<const float4*>(sC + 32 * m + 8 * q + 4 * h);
            acc[m][4 * q] = cq.x;
            acc[m][4 * q + 1] = cq.y;
            acc[m][4 * q + 2] = cq.z;
            acc[m][4 * q + 3] = cq.w;
        }
    WFrag<MG> cur;
    load_wfrag<MG, Dp>(cur, sW, wstride, 0, 0);
    XFrag f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = u / GPC, g0 = (u % GPC) * MG;
        WFrag<MG> nxt;
        if (u + 1 < U) load_wfrag<MG, Dp>(nxt, sW, wstride, (u + 1) / GPC, ((u + 1) % GPC) * MG);
        if (g0 == 0) {
            f.x1 = xr[c];
            split_square(f);
        }
#pragma unroll
        for (int m = 0; m < MG; ++m) acc[g0 + m] = mfma(cur.ah[m], f.x2h, acc[g0 + m]);
#pragma unroll
        for (int m = 0; m < MG; ++m) acc[g0 + m] = mfma(cur.bh[m], f.x1, acc[g0 + m]);
#pragma unroll
        for (int m = 0; m < MG; ++m) acc[g0 + m] = mfma(cur.al[m], f.x2h, acc[g0 + m]);
#pragma unroll
        for (int m = 0; m < MG; ++m) acc[g0 + m] = mfma(cur.bl[m], f.x1, acc[g0 + m]);
#pragma unroll
        for (int m = 0; m < MG; ++m) acc[g0 + m] = mfma(cur.ah[m], f.x2l, acc[g0 + m]);
        work(u, U);
        __builtin_amdgcn_sched_barrier(0);
        if (u + 1 < U) cur = nxt;
    }
}

// The softmax of a finished logits tile, cut into four stages so a pipelined loop can spread
// it over the units of the next tile's logits: 0 row max, 1 exponentials of the first half
// of the component tiles, 2 the second half, row sum and its reciprocal, 3 scale, pack to
// bf16 and store the token's row (components 32m + 8q + 4 half + 0..3 as 8 bytes) at `grow`.
template <int MT>
struct SoftmaxStages {
    float mx, s, inv;
    __device__ __forceinline__ void stage(int st, f32x16 (&a)[MT], bool valid, unsigned char* grow) {
        const int half = lane_id() >> 5;
        if (st == 0) {
            float m0 = -INFINITY;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 16; ++i) m0 = fmaxf(m0, a[m][i]);
            mx = max_halves(m0);
            s = 0.0f;
        } else if (st == 1 || st == 2) {
            constexpr int H1 = (MT + 1) / 2;
            const int lo = st == 1 ? 0 : H1, hi = st == 1 ? H1 : MT;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < lo || m >= hi) continue;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float e = fast_exp2(a[m][i] - mx);
                    a[m][i] = e;
                    s += e;
                }
            }
            if (st == 2) {
                // s >= 1 (the maximum contributes 2^0): the hardware reciprocal (~1 ulp) is
                // far below the bf16 rounding of the responsibilities it scales
                const float r = __builtin_amdgcn_rcpf(sum_halves(s));
                inv = valid ? r : 0.0f;
            }
        } else {
            // register group q of tile m holds components 32 m + 8 q + 4 half + 0..3; one swap
            // of the upper lanes of group 2 qp with the lower lanes of group 2 qp + 1 gives each
            // lane 8 contiguous components (one 16-byte LDS store)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int qp = 0; qp < 2; ++qp) {
                    const int i0 = 8 * qp;
                    auto sx = __builtin_amdgcn_permlane32_swap(pack_bf16(a[m][i0] * inv, a[m][i0 + 1] * inv),
                                                               pack_bf16(a[m][i0 + 4] * inv, a[m][i0 + 5] * inv),
                                                               false, false);
                    auto sy = __builtin_amdgcn_permlane32_swap(pack_bf16(a[m][i0 + 2] * inv, a[m][i0 + 3] * inv),
                                                               pack_bf16(a[m][i0 + 6] * inv, a[m][i0 + 7] * inv),
                                                               false, false);
                    *reinterpret_cast<uint4*>(grow + 2 * (32 * m + 16 * qp + 8 * half)) =
                        make_uint4(sx[0], sy[0], sx[1], sy[1]);
                }
        }
    }
};

// In-place softmax numerator: acc <- 2^(acc - max_k acc) for this lane's token; returns the
// row sum over all components (both lane halves).
template <int MT>
__device__ __forceinline__ float tile_exp(f32x16 (&acc)[MT]) {
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[m][i]);
    mx = max_halves(mx);
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float e = fast_exp2(acc[m][i] - mx);
            acc[m][i] = e;
            s += e;
        }
    return sum_halves(s);
}

// Transposed 4x16-bit LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane
// L supplies the address of 4 consecutive 16-bit elements; lane i receives element i % 4
// from the addresses of lanes 4e + i / 4, e = 0..3: with lane 4e + c pointing at row
// (r0 + e), columns (c0 + 4c .. c0 + 4c + 3) of a row-major matrix, lane i gets the
// column c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ s16x4 lds_read_tr(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Operand fragment (lane -> matrix column `col0 + l % 32`, 8 consecutive rows
// row0 + 8 (l / 32) .. + 7) of a row-major bf16 matrix in LDS, via two transposed reads.
__device__ __forceinline__ bf16x8 lds_frag_tr(const unsigned char* base, int stride, int row0, int col0) {
    const int l = lane_id();
    const int g = l >> 4, i = l & 15;
    const int hop = g >> 1;
    const int col = col0 + 16 * (g & 1) + 4 * (i & 3);
    const unsigned char* p0 = base + (size_t)(row0 + 8 * hop + (i >> 2)) * stride + col * 2;
    const s16x4 lo = lds_read_tr(p0);
    const s16x4 hi = lds_read_tr(p0 + 4 * (size_t)stride);
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// Operand fragment of a row-major bf16 matrix in LDS whose 8 contraction rows follow the
// C-register order of a 32x32 MFMA result: lane l gets column col0 + l % 32 of rows
// row0 + 4h + (0..3) and row0 + 8 + 4h + (0..3), h = l / 32.  Used where the other operand
// is a C tile converted in place (its contraction slot 8h + e holds row 8 (e / 4) + 4h + e % 4).
__device__ __forceinline__ bf16x8 lds_frag_tr_crows(const unsigned char* base, int stride, int row0, int col0) {
    const int l = lane_id();
    const int g = l >> 4, i = l & 15;
    const int hop = g >> 1;
    const int col = col0 + 16 * (g & 1) + 4 * (i & 3);
    const unsigned char* p0 = base + (size_t)(row0 + 4 * hop + (i >> 2)) * stride + col * 2;
    const s16x4 lo = lds_read_tr(p0);
    const s16x4 hi = lds_read_tr(p0 + 8 * (size_t)stride);
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// Workgroup barrier that orders LDS only: outstanding global loads (prefetches) stay in
// flight across it, unlike __syncthreads(), which also waits for them.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Pack 8 consecutive C registers (two bf16 per 32-bit word) into an MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int first, float scale) {
    u32x4 p;
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = pack_bf16(c[first + 2 * j] * scale, c[first + 2 * j + 1] * scale);
    return __builtin_bit_cast(bf16x8, p);
}

// Output tiles of Gamma_K^T [V | 1] owned by one wave: tile (m, n), n < NT a value tile,
// n == NT the ones tile whose every column accumulates z_k.  With MT >= 4 a wave owns MT/4
// component tiles and every n; with MT < 4 the 4/MT waves sharing a component tile split the
// n range (an index past NT is computed but never stored).  Compile-time counts, wave-uniform
// indices: the loops are branch-free, so the transposed LDS reads of a whole group batch up.
template <int MT, int NT>
struct UpdateTiles {
    static constexpr int MW = MT >= 4 ? MT / 4 : 1;
    static constexpr int WPM = MT >= 4 ? 1 : 4 / MT;
    static constexpr int NW = (NT + 1 + WPM - 1) / WPM;
    __device__ static int m_of(int w, int j) { return MT >= 4 ? w * MW + j : w / WPM; }
    __device__ static int n_of(int w, int j) { return MT >= 4 ? j : (w % WPM) * NW + j; }
};

// `work(ks)` runs once per 16-position step, between the step's LDS reads and its MFMAs
// (a hook for issuing other loads in the shadow of the matrix cores).
template <int MT, int NT, int MW, int NW, typename Work>
__device__ __forceinline__ void update_from_lds(f32x16 (&acc)[MW][NW], const unsigned char* sG, int gs,
                                                const unsigned char* sV, int vs, const bf16x8& ones, Work&& work) {
    using UT = UpdateTiles<MT, NT>;
    const int w = wave_id();
#pragma unroll
    for (int ks = 0; ks < kIterT / 16; ++ks) {
        bf16x8 a[UT::MW], b[UT::NW];
#pragma unroll
        for (int j = 0; j < UT::MW; ++j) a[j] = lds_frag_tr(sG, gs, 16 * ks, 32 * UT::m_of(w, j));
#pragma unroll
        for (int j = 0; j < UT::NW; ++j) {
            const int n = UT::n_of(w, j);
            const bf16x8 t = lds_frag_tr(sV, vs, 16 * ks, n < NT ? 32 * n : 0);
            b[j] = n < NT ? t : ones;
        }
        work(ks);
#pragma unroll
        for (int i = 0; i < UT::MW; ++i)
#pragma unroll
            for (int j = 0; j < UT::NW; ++j) acc[i][j] = mfma(a[i], b[j], acc[i][j]);
    }
}

template <int MT, int NT, int MW, int NW>
__device__ __forceinline__ void update_from_lds(f32x16 (&acc)[MW][NW], const unsigned char* sG, int gs,
                                                const unsigned char* sV, int vs, const bf16x8& ones) {
    update_from_lds<MT, NT, MW, NW>(acc, sG, gs, sV, vs, ones, [](int) {});
}

// Position of component k inside its 16-wide block so that the C registers 8s..8s+7 of a
// logits tile (k = 16s + 8(j/4) + 4h + j%4, j = 0..7, h = lane half) line up with
// contraction slots 8h + j of a k-contraction MFMA: swap bits 2 and 3 of k.
__host__ __device__ __forceinline__ int kperm(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

}  // namespace mf
}  // namespace gma
