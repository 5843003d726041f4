// MFMA family of the GMA forward for bf16 inputs (gfx950): parameter prep, the
// bidirectional write/read kernels and host-side dispatch.
//
// Method: Gaussian Mixture Attention (arXiv 2606.18283), "Core mechanism":
//   item 1 -- Gamma = GMM posterior responsibilities (diagonal Gaussians, softplus
//             variances, softmax priors; item 3);
//   item 2 -- write Vt = Gamma_K^T V, Z = Gamma_K^T 1; read O = Gamma_Q Vt / (Gamma_Q Z + eps).
// Kernels:
//   gma_prep          coefficients [ah|al|bh|bl] (bf16) and c_k of every head.
//   gma_bidir_write   Gamma_K tile by tile (logit MFMAs + in-lane softmax), staged in LDS,
//                     then Gamma_K^T [V | 1] on MFMAs; each workgroup owns one contiguous
//                     split of the sequence and writes a fp32 partial of [Vt | Z].  Small
//                     tiles (K <= 64, d_r, d_v <= 64) run two workgroups per CU over twice the
//                     splits.
//   gma_split_reduce  (after the two-per-CU write) the split partials of each head added in
//                     split order into the first split's slot, once, instead of by every
//                     read workgroup of the head.
//   gma_bidir_read    adds the split partials of its head in split order (deterministic), or
//                     takes the reduced one, stages Vt^T and Z in LDS, then
//                     Gamma_Q tile by tile, unnormalised (2^(l - max)); one MFMA chain gives
//                     Gamma_Q Vt, Gamma_Q Z and the row sum s together; O = num / (den + eps s).
// Gamma never leaves the chip in these kernels.
#include <math.h>

#include "gma_internal.h"
#include "gma_mfma_common.h"
#include "gma_mfma_geo.h"
#include "gma_numeric.h"

namespace gma {

using namespace mf;

namespace {

constexpr int kMaxSplits = 64;

// LDS row strides (bytes) of the token-major staging buffers, padded by 32 B.
inline int gstride(const Geo& g) { return 2 * g.Kp + 32; }
inline int vstride(const Geo& g) { return 2 * g.Dvp + 32; }
inline int vtstride(const Geo& g) { return 2 * g.Kp + 16; }

// + one 64-byte row of bf16 ones (the ones operand of the update MFMAs)
size_t write_lds_bytes(const Geo& g) {
    return (size_t)g.Kp * g.wstride + (size_t)g.Kp * 4 + (size_t)kIterT * gstride(g) + (size_t)kIterT * vstride(g) + 64;
}

// Write instances that run two workgroups per CU (at most 256 registers, LDS for two): small
// component and dim tiles.  Their launches use twice the splits, combined in pairs.
__host__ __device__ constexpr bool write_dual(int MT, int NT, int NC) { return MT <= 2 && NT <= 2 && NC <= 4; }
inline bool write_dual(const Geo& g) { return write_dual(g.MT, g.NT, g.NC) && 2 * write_lds_bytes(g) <= kLdsMax; }
// The read kernel keeps the memory operand of its output MFMAs (MT * 2 * (NT + 1) fragments of
// 4 registers) in registers when that leaves it within 256 registers (no spills).
__host__ __device__ constexpr bool read_regmem(int MT, int NT) { return MT * (NT + 1) <= 12; }

size_t read_lds_bytes(const Geo& g) {
    return (size_t)g.Kp * g.wstride + (size_t)g.Kp * 4 + (size_t)(g.Dvp + 32) * vtstride(g);
}

// Splits of the key sequence (length Nk) for the write kernel: about one workgroup per CU,
// two for the dual-occupancy instances.
int num_splits(const gma_desc& d, int Nk) {
    const int bh = d.B * d.H;
    const int iters = (Nk + kIterT - 1) / kIterT;
    const int target = write_dual(geometry(d)) ? 512 : 256;
    int s = (target + bh - 1) / bh;
    if (s > iters) s = iters;
    if (s > kMaxSplits) s = kMaxSplits;
    return s < 1 ? 1 : s;
}

struct MfmaLayout {
    size_t W, C, part_v, part_z, total;
};

MfmaLayout mfma_layout(const gma_desc& d, int Nk) {
    const Geo g = geometry(d);
    const size_t BH = (size_t)d.B * d.H;
    const int S = num_splits(d, Nk);
    MfmaLayout L;
    size_t off = 0;
    L.W = off;
    off += align_up((size_t)d.H * g.Kp * 4 * g.Dp * sizeof(bf16_t));
    L.C = off;
    off += align_up((size_t)d.H * g.Kp * sizeof(float));
    L.part_v = off;
    off += align_up(BH * S * g.Kp * g.Dvp * sizeof(float));
    L.part_z = off;
    off += align_up(BH * S * g.Kp * sizeof(float));
    L.total = off;
    return L;
}

// ---------------------------------------------------------------------------------- prep
// One wave per (h, k), lanes over the routing dims: the bf16 hi/lo coefficients and c_k.
// var = softplus(var_raw) + floor and log(var) in fp32 (relative error ~1e-7, far below the
// ~2^-17 of the hi/lo coefficient pairs); 1/var, the coefficients and the sum over d for
// c_k in double.
__global__ void __launch_bounds__(256) gma_prep(const float* __restrict__ mu, const float* __restrict__ var_raw,
                                                const float* __restrict__ prior, int H, int K, int dr, int Kp,
                                                int Dp, float var_floor, bf16_t* __restrict__ W,
                                                float* __restrict__ cvec) {
    const int gtid = blockIdx.x * blockDim.x + threadIdx.x;
    const int gw = gtid >> 6, lane = threadIdx.x & 63;
    if (gw >= H * Kp) return;
    const int h = gw / Kp, k = gw % Kp;
    bf16_t* row = W + (size_t)gw * 4 * Dp;
    const double L2E = 1.4426950408889634;
    double acc = 0.0;
    for (int dd = lane; dd < Dp; dd += 64) {
        double a = 0.0, b = 0.0;
        if (k < K && dd < dr) {
            const size_t i = ((size_t)h * K + k) * dr + dd;
            const float r = var_raw[i];
            const float var = fmaxf(r, 0.0f) + log1pf(expf(-fabsf(r))) + var_floor;
            const double lam = 1.0 / (double)var;
            const double m = mu[i];
            a = -0.5 * lam * L2E;
            b = lam * m * L2E;
            acc += (double)logf(var) + m * m * lam;
        }
        const bf16_t ah = f32_to_bf16((float)a);
        const bf16_t al = f32_to_bf16((float)(a - (double)bf16_to_f32(ah)));
        const bf16_t bh = f32_to_bf16((float)b);
        const bf16_t bl = f32_to_bf16((float)(b - (double)bf16_to_f32(bh)));
        row[dd] = ah;
        row[Dp + dd] = al;
        row[2 * Dp + dd] = bh;
        row[3 * Dp + dd] = bl;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0)
        cvec[gw] = (k < K) ? (float)(L2E * ((double)prior[(size_t)h * K + k] - 0.5 * acc))
                           : -INFINITY;  // padded component: 2^-inf = 0 responsibility
}

// ---------------------------------------------------------------------------------- write
// Raw V values of one token row for this lane: dims 8 half + 16 j, j < NT * 2 (zero-padded;
// d_v is a multiple of 8 on this path).  FULL (d_v = 32 NT): every load is whole, so the loads
// are unconditional and no register is zeroed first (a conditional load costs a move per
// register and splits the scheduling region).
template <int NT, bool FULL>
__device__ __forceinline__ void load_vrow(bf16x8 (&vr)[2 * NT], const bf16_t* row, int dv) {
    const int half = lane_id() >> 5;
#pragma unroll
    for (int j = 0; j < 2 * NT; ++j) {
        const int d0 = 16 * j + 8 * half;
        if (FULL) {
            vr[j] = *reinterpret_cast<const bf16x8*>(row + d0);
        } else {
            bf16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
            if (d0 < dv) x = *reinterpret_cast<const bf16x8*>(row + d0);
            vr[j] = x;
        }
    }
}

// Routing values of one token row for this lane (as load_xrow); FULL: d_r = 16 NC, no tail,
// unconditional loads.
template <int NC, bool FULL>
__device__ __forceinline__ void load_krow(bf16x8 (&xr)[NC], const bf16_t* row, int dr) {
    if (FULL) {
        const int h = lane_id() >> 5;
#pragma unroll
        for (int c = 0; c < NC; ++c) xr[c] = *reinterpret_cast<const bf16x8*>(row + 16 * c + 8 * h);
    } else {
        load_xrow<NC>(xr, row, dr);
    }
}

// Stage assignment of the four softmax stages over the U units of a pipelined logits tile.
__host__ __device__ constexpr int stage_unit(int st, int U) { return (st * U) / 4; }

// The update of the write kernel: wave-uniform tile indices, the ones operand read from a
// 64-byte LDS row of ones with a zero row stride (so value and ones tiles take the same code,
// no per-register select); a wave whose last tile index lies past the ones tile (component
// tiles shared by several waves) skips that tile.
template <int MT, int NT, int MW, int NW, int NJ>
__device__ __forceinline__ void write_update_n(f32x16 (&acc)[MW][NW], const unsigned char* sG, int gs,
                                               const unsigned char* sV, int vs, const unsigned char* sOnes, int w) {
    using UT = UpdateTiles<MT, NT>;
#pragma unroll
    for (int ks = 0; ks < kIterT / 16; ++ks) {
        bf16x8 a[MW], b[NJ];
#pragma unroll
        for (int j = 0; j < MW; ++j) a[j] = lds_frag_tr(sG, gs, 16 * ks, 32 * UT::m_of(w, j));
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int n = UT::n_of(w, j);
            const bool isv = n < NT;
            b[j] = lds_frag_tr(isv ? sV : sOnes, isv ? vs : 0, isv ? 16 * ks : 0, isv ? 32 * n : 0);
        }
#pragma unroll
        for (int i = 0; i < MW; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = mfma(a[i], b[j], acc[i][j]);
    }
}
template <int MT, int NT, int MW, int NW>
__device__ __forceinline__ void write_update(f32x16 (&acc)[MW][NW], const unsigned char* sG, int gs,
                                             const unsigned char* sV, int vs, const unsigned char* sOnes) {
    using UT = UpdateTiles<MT, NT>;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (MT < 4 && NW > 1 && UT::n_of(w, NW - 1) > NT)
        write_update_n<MT, NT, MW, NW, (NW > 1 ? NW - 1 : NW)>(acc, sG, gs, sV, vs, sOnes, w);
    else
        write_update_n<MT, NT, MW, NW, NW>(acc, sG, gs, sV, vs, sOnes, w);
}

template <int MT, int NT, int NC, bool FULL>
__global__ void __launch_bounds__(kThreads, write_dual(MT, NT, NC) ? 2 : 1)
    gma_bidir_write(const bf16_t* __restrict__ kr, const bf16_t* __restrict__ v, const bf16_t* __restrict__ W,
                    const float* __restrict__ cvec, float* __restrict__ part_v, float* __restrict__ part_z, int BH,
                    int H, int N, int dr, int dv, int S, int split_len) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int Kp = 32 * MT, Dvp = 32 * NT, Dp = 16 * NC;
    constexpr int wstride = 8 * Dp + 16;
    constexpr int gs = 2 * Kp + 32, vs = 2 * Dvp + 32;
    using UT = UpdateTiles<MT, NT>;
    unsigned char* sW = smem;
    float* sC = reinterpret_cast<float*>(sW + (size_t)Kp * wstride);
    unsigned char* sG = reinterpret_cast<unsigned char*>(sC + Kp);
    unsigned char* sV = sG + (size_t)kIterT * gs;
    unsigned char* sOnes = sV + (size_t)kIterT * vs;

    int bh, split;
    head_part(blockIdx.x, BH, S, bh, split);
    const int h = bh % H;
    const int l = lane_id(), w = wave_id(), half = l >> 5, col = l & 31;
    const int n_begin = split * split_len;
    const int n_end = min(N, n_begin + split_len);
    const int nit = n_end > n_begin ? (n_end - n_begin + kIterT - 1) / kIterT : 0;
    float* pv = part_v + ((size_t)bh * S + split) * Kp * Dvp;
    float* pz = part_z + ((size_t)bh * S + split) * Kp;
    if (N == 0) {  // empty key sequence (cross variant): a zero memory, no rows to read
        for (int i = threadIdx.x; i < Kp * Dvp; i += kThreads) pv[i] = 0.0f;
        for (int i = threadIdx.x; i < Kp; i += kThreads) pz[i] = 0.0f;
        return;
    }
    const bf16_t* kr_h = kr + (size_t)bh * N * dr;
    const bf16_t* v_h = v + (size_t)bh * N * dv;
    // rows past the split read a valid row of the head (their responsibilities are zeroed)
    auto krow = [&](int it) -> const bf16_t* {
        const int t = min(n_begin + it * kIterT + kTileT * w + col, N - 1);
        return kr_h + (size_t)t * dr;
    };
    auto vrow = [&](int it) -> const bf16_t* {
        const int t = min(n_begin + it * kIterT + kTileT * w + col, N - 1);
        return v_h + (size_t)t * dv;
    };

    f32x16 wacc[UT::MW][UT::NW];
#pragma unroll
    for (int i = 0; i < UT::MW; ++i)
#pragma unroll
        for (int j = 0; j < UT::NW; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) wacc[i][j][e] = 0.0f;
    // coefficients, k rows for steps 0 and 1 and v rows for step 0: all loads in flight together
    bf16x8 xa[NC], xb[NC], vcur[2 * NT];
    {
        CoefRegs<MT, NC, kThreads> cr;
        cr.load(W, cvec, h);
        load_krow<NC, FULL>(xa, krow(0), dr);
        load_krow<NC, FULL>(xb, krow(1), dr);
        load_vrow<NT, FULL>(vcur, vrow(0), dv);
        cr.store(sW, sC, wstride);
        if (threadIdx.x < 16) reinterpret_cast<uint32_t*>(sOnes)[threadIdx.x] = 0x3f803f80u;  // bf16 1.0
    }
    __syncthreads();

    f32x16 accA[MT], accB[MT];
    tile_logits_overlap<MT, NC>(accA, xa, sW, wstride, sC, [](int, int) {});
    load_krow<NC, FULL>(xa, krow(2), dr);

    // One pipeline step: finish tile `it` (softmax, stage Gamma_K and V rows in LDS) while the
    // logits of tile it+1 run, then the LDS-fed update over the 128 staged positions.
    auto step = [&](int it, f32x16 (&cur)[MT], f32x16 (&nxt)[MT], bf16x8 (&xnext)[NC], bf16x8 (&xfar)[NC]) {
        const int t = n_begin + it * kIterT + kTileT * w + col;
        const bool valid = t < n_end;
        bf16x8 vnext[2 * NT];
        load_vrow<NT, FULL>(vnext, vrow(it + 1), dv);
        SoftmaxStages<MT> sm;
        unsigned char* grow = sG + (size_t)(kTileT * w + col) * gs;
        unsigned char* vdst = sV + (size_t)(kTileT * w + col) * vs;
        tile_logits_overlap<MT, NC>(nxt, xnext, sW, wstride, sC, [&](int u, int U) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
                if (stage_unit(st, U) == u) sm.stage(st, cur, valid, grow);
            if (u == U - 1) {
#pragma unroll
                for (int j = 0; j < 2 * NT; ++j) *reinterpret_cast<bf16x8*>(vdst + 2 * (16 * j + 8 * half)) = vcur[j];
            }
        });
        load_krow<NC, FULL>(xfar, krow(it + 3), dr);
        lds_barrier();
        write_update<MT, NT, UT::MW, UT::NW>(wacc, sG, gs, sV, vs, sOnes);
        lds_barrier();
#pragma unroll
        for (int j = 0; j < 2 * NT; ++j) vcur[j] = vnext[j];
    };
    // The last step has no next tile: softmax and update only.
    auto last = [&](int it, f32x16 (&cur)[MT]) {
        const int t = n_begin + it * kIterT + kTileT * w + col;
        const bool valid = t < n_end;
        SoftmaxStages<MT> sm;
        unsigned char* grow = sG + (size_t)(kTileT * w + col) * gs;
        unsigned char* vdst = sV + (size_t)(kTileT * w + col) * vs;
#pragma unroll
        for (int st = 0; st < 4; ++st) sm.stage(st, cur, valid, grow);
#pragma unroll
        for (int j = 0; j < 2 * NT; ++j) *reinterpret_cast<bf16x8*>(vdst + 2 * (16 * j + 8 * half)) = vcur[j];
        lds_barrier();
        write_update<MT, NT, UT::MW, UT::NW>(wacc, sG, gs, sV, vs, sOnes);
    };
    // Steps run in pairs (an odd count gets one step past the split, all of whose rows are
    // zeroed), so the loop body has no branch: xa holds step it+2's rows when step `it` starts
    // with nxt rows in xb (and vice versa).
    const int nit2 = (nit + 1) & ~1;
    for (int it = 0; it + 2 < nit2; it += 2) {
        step(it, accA, accB, xb, xb);
        step(it + 1, accB, accA, xa, xa);
    }
    if (nit2 > 0) {
        step(nit2 - 2, accA, accB, xb, xb);
        last(nit2 - 1, accB);
    }

    // ---- partial of this split -> workspace (fp32)
#pragma unroll
    for (int i = 0; i < UT::MW; ++i)
#pragma unroll
        for (int j = 0; j < UT::NW; ++j) {
            const int m = UT::m_of(w, i), n = UT::n_of(w, j);
            if (n > NT) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int k = 32 * m + 8 * (e >> 2) + 4 * half + (e & 3);
                if (n < NT)
                    pv[(size_t)k * Dvp + 32 * n + col] = wacc[i][j][e];
                else if (col == 0)
                    pz[k] = wacc[i][j][e];
            }
        }

}

// ---------------------------------------------------------------------------------- read
constexpr int kReadWaves = 8;  // two waves per SIMD: one computes exponentials while the other
                               // runs its MFMAs

template <int MT, int NT, int NC>
__global__ void __launch_bounds__(64 * kReadWaves, 2)
    gma_bidir_read(const bf16_t* __restrict__ qr, const bf16_t* __restrict__ W, const float* __restrict__ cvec,
                   const float* __restrict__ part_v, const float* __restrict__ part_z, bf16_t* __restrict__ out,
                   float eps, int BH, int H, int N, int dr, int dv, int S, int sstep, int parts, int part_len) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int Kp = 32 * MT, Dvp = 32 * NT, Dp = 16 * NC;
    constexpr int wstride = 8 * Dp + 16;
    constexpr int ts = 2 * Kp + 16;
    unsigned char* sW = smem;
    float* sC = reinterpret_cast<float*>(sW + (size_t)Kp * wstride);
    unsigned char* sT = reinterpret_cast<unsigned char*>(sC + Kp);  // (Dvp + 32) rows x Kp

    int bh, part;
    head_part(blockIdx.x, BH, parts, bh, part);
    const int h = bh % H;
    const int l = lane_id(), w = wave_id(), half = l >> 5;
    const bf16_t* q_h = qr + (size_t)bh * N * dr;
    bf16_t* o_h = out + (size_t)bh * N * dv;
    const int n_begin = part * part_len;
    const int n_end = min(N, n_begin + part_len);
    constexpr int kStep = kTileT * kReadWaves;

    bf16x8 xr[NC];
    {
        const int t = n_begin + kTileT * w + (l & 31);
        load_xrow<NC>(xr, q_h + (size_t)min(t, N - 1) * dr, dr);
    }

    // the head's memory [Vt | Z] = sum of the split partials of the write kernel (slots
    // 0, sstep, 2 sstep, ... of the S: sstep = S where gma_split_reduce has already added
    // them into slot 0), in split order (every workgroup of the head forms the identical sum).  The coefficient
    // loads and the partial loads of up to SB splits are in flight together.  Vt^T goes to
    // LDS rows 0..Dvp-1 in the permuted component order of the logits tiles, then Z hi
    // (8 rows), Z lo (8 rows) and ones (16 rows).
    {
        constexpr int kThr = 64 * kReadWaves;
        constexpr int kVec = Kp * Dvp / 4;
        constexpr int P = (kVec + kThr - 1) / kThr;
        constexpr int SB = P <= 4 ? 4 : (P <= 8 ? 2 : 1);  // splits per batch of loads
        const float* pv0 = part_v + (size_t)bh * S * Kp * Dvp;
        const float* pz0 = part_z + (size_t)bh * S * Kp;
        float4 sum[P];
#pragma unroll
        for (int p = 0; p < P; ++p) sum[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        float zsum = 0.0f;
        CoefRegs<MT, NC, kThr> cr;
        cr.load(W, cvec, h);
        const int nslot = (S + sstep - 1) / sstep;
        for (int s0 = 0; s0 < nslot; s0 += SB) {
            float4 x[SB][P];
            float zx[SB];
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const bool ok = s0 + u < nslot;
                const int sp = ok ? (s0 + u) * sstep : 0;
                const float4* src = reinterpret_cast<const float4*>(pv0 + (size_t)sp * Kp * Dvp);
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const int i = threadIdx.x + p * kThr;
                    x[u][p] = (ok && i < kVec) ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
                zx[u] = (ok && (int)threadIdx.x < Kp) ? pz0[(size_t)sp * Kp + threadIdx.x] : 0.0f;
            }
            if (s0 == 0) cr.store(sW, sC, wstride);
#pragma unroll
            for (int u = 0; u < SB; ++u) {
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    sum[p].x += x[u][p].x;
                    sum[p].y += x[u][p].y;
                    sum[p].z += x[u][p].z;
                    sum[p].w += x[u][p].w;
                }
                zsum += zx[u];
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = threadIdx.x + p * kThr;
            if (i < kVec) {
                const int k = i / (Dvp / 4), d0 = 4 * (i % (Dvp / 4));
                const int pos = (k & ~15) + kperm(k & 15);
                *reinterpret_cast<bf16_t*>(sT + (size_t)(d0 + 0) * ts + 2 * pos) = f32_to_bf16(sum[p].x);
                *reinterpret_cast<bf16_t*>(sT + (size_t)(d0 + 1) * ts + 2 * pos) = f32_to_bf16(sum[p].y);
                *reinterpret_cast<bf16_t*>(sT + (size_t)(d0 + 2) * ts + 2 * pos) = f32_to_bf16(sum[p].z);
                *reinterpret_cast<bf16_t*>(sT + (size_t)(d0 + 3) * ts + 2 * pos) = f32_to_bf16(sum[p].w);
            }
        }
        // Z hi (8 rows), Z lo (8 rows), ones (16 rows) below Vt^T
        if ((int)threadIdx.x < Kp) {
            const int k = threadIdx.x;
            const bf16_t zh = f32_to_bf16(zsum);
            const bf16_t zl = f32_to_bf16(zsum - bf16_to_f32(zh));
            const int pos = (k & ~15) + kperm(k & 15);
#pragma unroll
            for (int r = 0; r < 32; ++r)
                *reinterpret_cast<bf16_t*>(sT + (size_t)(Dvp + r) * ts + 2 * pos) =
                    r < 8 ? zh : (r < 16 ? zl : (bf16_t)0x3f80);
        }
    }
    __syncthreads();

    // The memory operand of the output MFMAs (Vt^T, Z hi/lo, ones) stays in registers for the
    // whole kernel where it fits (read_regmem); larger memories are read from LDS per tile.
    constexpr bool kRegMem = read_regmem(MT, NT);
    bf16x8 aV[kRegMem ? MT : 1][2][NT + 1];
    auto mem_frag = [&](int m, int sh, int n) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(sT + (size_t)(32 * n + (l & 31)) * ts + 2 * (32 * m + 16 * sh + 8 * half));
    };
    if constexpr (kRegMem) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int sh = 0; sh < 2; ++sh)
#pragma unroll
                for (int n = 0; n <= NT; ++n) aV[m][sh][n] = mem_frag(m, sh, n);
    }

    for (int base = n_begin + kTileT * w; base < n_end; base += kStep) {
        const int t = base + (l & 31);
        const bool valid = t < n_end;
        f32x16 acc[MT];
        tile_logits<MT, NC>(acc, xr, sW, wstride, sC);
        // next tile's routing rows: in flight during the softmax and the read MFMAs
        const int tn = t + kStep;
        load_xrow<NC>(xr, q_h + (size_t)min(tn, N - 1) * dr, dr);
        (void)tile_exp<MT>(acc);  // unnormalised; the row sum comes out of the MFMAs below
        f32x16 o[NT + 1];
#pragma unroll
        for (int n = 0; n <= NT; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[n][i] = 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
                u32x4 bp;
#pragma unroll
                for (int j = 0; j < 4; ++j) bp[j] = pack_bf16(acc[m][8 * sh + 2 * j], acc[m][8 * sh + 2 * j + 1]);
                const bf16x8 b = __builtin_bit_cast(bf16x8, bp);
#pragma unroll
                for (int n = 0; n <= NT; ++n) {
                    if constexpr (kRegMem)
                        o[n] = mfma(aV[m][sh][n], b, o[n]);
                    else
                        o[n] = mfma(mem_frag(m, sh, n), b, o[n]);
                }
            }
        // o[NT]: rows 0-7 Gamma_Q Z_hi, 8-15 Gamma_Q Z_lo, 16-31 row sum s
        const float den = o[NT][0] + o[NT][4];
        const float s = o[NT][8];
        const float inv = 1.0f / (den + eps * s);
        // C register group q of o[n] holds value dims 32 n + 8 q + 4 half + 0..3 of this lane's
        // position; the wave halves trade groups so that each lane stores 8 contiguous dims (16
        // bytes): half the store instructions of 8-byte stores
        bf16_t* orow = o_h + (size_t)t * dv;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int qp = 0; qp < 2; ++qp) {
                uint2 p0, p1;  // groups q = 2 qp and 2 qp + 1 of this lane
                p0.x = pack_bf16(o[n][8 * qp] * inv, o[n][8 * qp + 1] * inv);
                p0.y = pack_bf16(o[n][8 * qp + 2] * inv, o[n][8 * qp + 3] * inv);
                p1.x = pack_bf16(o[n][8 * qp + 4] * inv, o[n][8 * qp + 5] * inv);
                p1.y = pack_bf16(o[n][8 * qp + 6] * inv, o[n][8 * qp + 7] * inv);
                // one swap of the upper lanes of p0 with the lower lanes of p1: the lower half then
                // holds group 2 qp of both halves (dims 16 qp + 0..7), the upper half group 2 qp + 1
                auto sx = __builtin_amdgcn_permlane32_swap(p0.x, p1.x, false, false);
                auto sy = __builtin_amdgcn_permlane32_swap(p0.y, p1.y, false, false);
                const uint4 v16 = make_uint4(sx[0], sy[0], sx[1], sy[1]);
                const int d0 = 32 * n + 16 * qp + 8 * half;
                if (valid && d0 < dv) *reinterpret_cast<uint4*>(orow + d0) = v16;
            }
    }
}

// ---------------------------------------------------------------------------------- split reduce
// The S split partials of every head added in split order into split 0's slot (in place:
// each element is read and written by one thread; the loads of 8 splits are issued together,
// then added in order).  Grid (ceil(Kp (Dvp + 1) / 256), min(B H, 65535)), heads strided by
// gridDim.y.
__global__ void __launch_bounds__(256)
    gma_split_reduce(float* __restrict__ part_v, float* __restrict__ part_z, int BH, int S, int Kp, int Dvp) {
    const int nv = Kp * Dvp;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nv + Kp) return;
    for (size_t bh = blockIdx.y; bh < (size_t)BH; bh += gridDim.y) {
        float* p = i < nv ? part_v + bh * S * nv + i : part_z + bh * S * Kp + (i - nv);
        const size_t stride = i < nv ? (size_t)nv : (size_t)Kp;
        float acc = p[0];
        for (int s0 = 1; s0 < S; s0 += 8) {
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = s0 + u < S ? p[(size_t)(s0 + u) * stride] : 0.0f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < S) acc += x[u];
        }
        p[0] = acc;
    }
}

// ---------------------------------------------------------------------------------- memory
// Causal memory from the split partials of the write kernel: for component k < K,
// state[bh][k][c] = sum_s part_v[bh][s][k][c] (c < d_v), state[bh][k][d_v] = sum_s part_z[bh][s][k],
// in split order.  Grid (ceil(K (d_v+1) / 256), min(B H, 65535)), heads strided by gridDim.y.
__global__ void __launch_bounds__(256)
    gma_memory_reduce(const float* __restrict__ part_v, const float* __restrict__ part_z, float* __restrict__ state,
                      int BH, int S, int K, int Kp, int dv, int Dvp) {
    const int W = dv + 1;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= K * W) return;
    const int k = i / W, c = i % W;
    for (size_t bh = blockIdx.y; bh < (size_t)BH; bh += gridDim.y) {
        float acc = 0.0f;
        for (int s = 0; s < S; ++s)
            acc += c < dv ? part_v[((bh * S + s) * Kp + k) * Dvp + c] : part_z[(bh * S + s) * Kp + k];
        state[bh * K * W + i] = acc;
    }
}

// ---------------------------------------------------------------------------------- host
typedef void (*WriteFn)(const bf16_t*, const bf16_t*, const bf16_t*, const float*, float*, float*, int, int, int,
                        int, int, int, int);
typedef void (*ReadFn)(const bf16_t*, const bf16_t*, const float*, const float*, const float*, bf16_t*, float, int,
                       int, int, int, int, int, int, int, int);

// The exact-fit write kernel is built where it does not spill registers (the largest tiles
// keep the general form).
constexpr bool write_full_ok(int MT, int NT, int NC) { return MT <= 4 && MT * NT * NC < 128 && !(MT == 4 && NC == 8); }

template <int MT, int NT, int NC>
bool pick(bool full, WriteFn& wf, ReadFn& rf) {
    if constexpr (write_full_ok(MT, NT, NC))
        wf = full ? gma_bidir_write<MT, NT, NC, true> : gma_bidir_write<MT, NT, NC, false>;
    else
        wf = gma_bidir_write<MT, NT, NC, false>;
    rf = gma_bidir_read<MT, NT, NC>;
    return true;
}

template <int MT, int NT>
bool select_nc(int NC, bool full, WriteFn& wf, ReadFn& rf) {
    switch (NC) {
        case 1: return pick<MT, NT, 1>(full, wf, rf);
        case 2: return pick<MT, NT, 2>(full, wf, rf);
        case 4: return pick<MT, NT, 4>(full, wf, rf);
        case 8: return pick<MT, NT, 8>(full, wf, rf);
    }
    return false;
}

template <int MT>
bool select_nt(int NT, int NC, bool full, WriteFn& wf, ReadFn& rf) {
    switch (NT) {
        case 1: return select_nc<MT, 1>(NC, full, wf, rf);
        case 2: return select_nc<MT, 2>(NC, full, wf, rf);
        case 4: return select_nc<MT, 4>(NC, full, wf, rf);
    }
    return false;
}

bool select(const Geo& g, const gma_desc& d, WriteFn& wf, ReadFn& rf) {
    // exact fit (d_r = Dp, d_v = Dvp): every row load of the write kernel is whole, no zero
    // tail (the read kernel measured no faster in that form)
    const bool full = d.d_r == g.Dp && d.d_v == g.Dvp;
    switch (g.MT) {
        case 1: return select_nt<1>(g.NT, g.NC, full, wf, rf);
        case 2: return select_nt<2>(g.NT, g.NC, full, wf, rf);
        case 4: return select_nt<4>(g.NT, g.NC, full, wf, rf);
        case 8: return select_nt<8>(g.NT, g.NC, full, wf, rf);
    }
    return false;
}

}  // namespace

hipError_t mf::launch_prep(const Args& a, const Geo& g, bf16_t* W, float* cvec) {
    const gma_desc& d = a.d;
    const long threads = (long)d.H * g.Kp * 64;
    rec_begin(a, "gma_prep");
    gma_prep<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, a.stream>>>(
        a.mu, a.var_raw, a.prior, d.H, d.K, d.d_r, g.Kp, g.Dp, d.var_floor, W, cvec);
    rec_end(a);
    return hipGetLastError();
}

bool mfma_supported(const gma_desc& d, int causal) {
    // bf16 rows loaded as 16-byte vectors: d_r and d_v multiples of 8
    if (d.dtype != GMA_BF16 || d.d_r % 8 != 0 || d.d_v % 8 != 0) return false;
    if (causal) return causal_supported(d);
    const Geo g = geometry(d);
    return write_lds_bytes(g) <= kLdsMax && read_lds_bytes(g) <= kLdsMax;
}

size_t mfma_workspace(const gma_desc& d, int causal, int Nk) {
    // + room for the float64 parameters of the optional gamma_out diagnostic
    if (causal) return causal_workspace(d) + simt_param_bytes(d);
    return mfma_layout(d, Nk).total + simt_param_bytes(d);
}

// Write over the Nk key rows (kr, v), read over the N query rows (qr, out).
static hipError_t bidir_forward(const Args& a) {
    const gma_desc& d = a.d;
    const Geo g = geometry(d);
    const int Nk = a.Nk;
    const MfmaLayout L = mfma_layout(d, Nk);
    bf16_t* W = reinterpret_cast<bf16_t*>(a.ws + L.W);
    float* cvec = reinterpret_cast<float*>(a.ws + L.C);
    float* part_v = reinterpret_cast<float*>(a.ws + L.part_v);
    float* part_z = reinterpret_cast<float*>(a.ws + L.part_z);
    const int BH = d.B * d.H;
    hipError_t e;

    WriteFn wf;
    ReadFn rf;
    if (!select(g, d, wf, rf)) return hipErrorNotSupported;

    if ((e = launch_prep(a, g, W, cvec)) != hipSuccess) return e;

    const int S = num_splits(d, Nk);

    const int split_len = ((Nk + S - 1) / S + kIterT - 1) / kIterT * kIterT;
    const size_t wl = write_lds_bytes(g);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(wf), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)wl)) != hipSuccess)
        return e;
    rec_begin(a, "gma_bidir_write");
    hipLaunchKernelGGL(wf, dim3(BH * S), dim3(kThreads), wl, a.stream, static_cast<const bf16_t*>(a.kr),
                       static_cast<const bf16_t*>(a.v), W, cvec, part_v, part_z, BH, d.H, Nk, d.d_r, d.d_v, S,
                       split_len);
    rec_end(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the two-per-CU write runs twice the splits: add them once here rather than in every
    // read workgroup's prologue
    const bool reduced = write_dual(g) && S > 1;
    if (reduced) {
        const int nv = g.Kp * (g.Dvp + 1);
        rec_begin(a, "gma_split_reduce");
        gma_split_reduce<<<dim3((unsigned)((nv + 255) / 256), (unsigned)(BH < 65535 ? BH : 65535)), dim3(256), 0,
                           a.stream>>>(part_v, part_z, BH, S, g.Kp, g.Dvp);
        rec_end(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // read: about one workgroup per CU, each a contiguous run of the sequence of one head
    const int step = kTileT * kReadWaves;
    int parts = (256 + BH - 1) / BH;
    const int max_parts = (d.N + step - 1) / step;
    if (parts > max_parts) parts = max_parts;
    if (parts < 1) parts = 1;
    const int part_len = ((d.N + parts - 1) / parts + step - 1) / step * step;
    parts = (d.N + part_len - 1) / part_len;
    const size_t rl = read_lds_bytes(g);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(rf), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)rl)) != hipSuccess)
        return e;
    rec_begin(a, "gma_bidir_read");
    hipLaunchKernelGGL(rf, dim3(BH * parts), dim3(64 * kReadWaves), rl, a.stream, static_cast<const bf16_t*>(a.qr),
                       W, cvec, part_v, part_z, static_cast<bf16_t*>(a.out), a.eps, BH, d.H, d.N, d.d_r, d.d_v, S,
                       reduced ? S : 1, parts, part_len);
    rec_end(a);
    return hipGetLastError();
}

// The fused write kernel when its coefficient block fits in LDS, else the two-pass form on
// the causal kernels (responsibilities to HBM, then sub-segment totals).
static bool memory_fused(const gma_desc& d) { return mfma_supported(d, 0); }

bool mfma_memory_supported(const gma_desc& d) {
    if (d.dtype != GMA_BF16 || d.d_r % 8 != 0 || d.d_v % 8 != 0) return false;
    return memory_fused(d) || causal_supported(d);
}

size_t mfma_memory_workspace(const gma_desc& d) {
    return memory_fused(d) ? mfma_layout(d, d.N).total : causal_memory_workspace(d);
}

// The write phase over the d.N positions of a.kr, a.v, then the split partials summed into
// a.state.
hipError_t mfma_memory(const Args& a) {
    const gma_desc& d = a.d;
    if (!memory_fused(d)) return causal_memory(a);
    const Geo g = geometry(d);
    const int N = d.N;
    const MfmaLayout L = mfma_layout(d, N);
    bf16_t* W = reinterpret_cast<bf16_t*>(a.ws + L.W);
    float* cvec = reinterpret_cast<float*>(a.ws + L.C);
    float* part_v = reinterpret_cast<float*>(a.ws + L.part_v);
    float* part_z = reinterpret_cast<float*>(a.ws + L.part_z);
    const int BH = d.B * d.H;
    hipError_t e;
    WriteFn wf;
    ReadFn rf;
    if (!select(g, d, wf, rf)) return hipErrorNotSupported;
    if ((e = launch_prep(a, g, W, cvec)) != hipSuccess) return e;
    const int S = num_splits(d, N);
    const int split_len = ((N + S - 1) / S + kIterT - 1) / kIterT * kIterT;
    const size_t wl = write_lds_bytes(g);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(wf), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)wl)) != hipSuccess)
        return e;
    rec_begin(a, "gma_bidir_write");
    hipLaunchKernelGGL(wf, dim3(BH * S), dim3(kThreads), wl, a.stream, static_cast<const bf16_t*>(a.kr),
                       static_cast<const bf16_t*>(a.v), W, cvec, part_v, part_z, BH, d.H, N, d.d_r, d.d_v, S,
                       split_len);
    rec_end(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int per = d.K * (d.d_v + 1);
    rec_begin(a, "gma_memory_reduce");
    gma_memory_reduce<<<dim3((unsigned)((per + 255) / 256), (unsigned)(BH < 65535 ? BH : 65535)), dim3(256), 0,
                        a.stream>>>(part_v, part_z, a.state, BH, S, d.K, g.Kp, d.d_v, g.Dvp);
    rec_end(a);
    return hipGetLastError();
}

hipError_t mfma_forward(const Args& a) {
    const gma_desc& d = a.d;
    hipError_t e = a.causal ? causal_forward(a) : bidir_forward(a);
    if (e != hipSuccess) return e;
    if (a.gamma_out) {
        // diagnostic responsibilities (float32), outside the fused path: for self-mixing
        // shapes the responsibilities kernel gives them from the same matrix-core logits (the
        // five-pass split contraction) as the fused kernels, so they show what the fused path
        // routes; the cross variant (two lengths) takes the SIMT kernel's double logits
        if (a.Nk == d.N && stats_supported(d)) {
            // both workspace layouts open with the coefficient block W, then c
            const Geo g = geometry(d);
            bf16_t* W = reinterpret_cast<bf16_t*>(a.ws);
            float* cvec = reinterpret_cast<float*>(a.ws + align_up((size_t)d.H * g.Kp * 4 * g.Dp * sizeof(bf16_t)));
            return resp_rows(a, W, cvec, a.gamma_out);
        }
        const size_t off = a.causal ? causal_workspace(d) : mfma_layout(d, a.Nk).total;
        double* lam = reinterpret_cast<double*>(a.ws + off);
        double* cst = reinterpret_cast<double*>(a.ws + off + align_up((size_t)d.H * d.K * d.d_r * sizeof(double)));
        if ((e = simt_params(a, lam, cst)) != hipSuccess) return e;
        if ((e = simt_gamma(a, a.gamma_out, lam, cst)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gma
