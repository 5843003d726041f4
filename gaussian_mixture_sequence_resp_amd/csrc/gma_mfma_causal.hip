// Causal GMA forward on MFMAs (bf16 inputs, gfx950).
//
// Method: Gaussian Mixture Attention (arXiv 2606.18283), "Core mechanism" item 3: the
// causal variant replaces the write/read of item 2 by prefix sums of the latent memory and
// of the normaliser, so that position i reads
//     O_i = gamma_Q,i . S_i / (gamma_Q,i . z_i + eps),
//     [S_i | z_i] = sum_{j <= i} gamma_K,j (x) [v_j | 1]        (inclusive of i).
// Chunked form used here, with a group of 128 positions (four 32-position chunks, one per
// wave) and the state [S | z] at the start of the group:
//     O_group = Gamma_Q [S | z]  +  tril(Gamma_Q Gamma_K^T) [V | 1]     (within the group)
//     [S | z] += Gamma_K^T [V | 1]                                      (after the group)
// The sequence of each head is cut into S contiguous segments that run in parallel; the
// state entering segment s is the sum of the totals Gamma_K^T [V | 1] of segments 0..s-1,
// added in segment order (deterministic).
//
// Kernels (all on the caller's stream, in this order):
//   gma_prep            (shared with the bidirectional path) coefficients and c_k
//   gma_causal_resp     Gamma_Q and Gamma_K (normalised, bf16) of every position, token-major,
//                       plus Gamma_K transposed (component-major) for the state update
//   gma_causal_totals   per-segment totals Gamma_K^T [V | 1] (segments 0..S-2)
//   gma_causal_carry    exclusive prefix of the totals over segments (in place)
//   gma_causal_scan     one workgroup per (head, segment): sequential groups of 128
//                       positions; fp32 state in MFMA accumulators split over the 4 waves by
//                       output tile, bf16 shadow of the full state in LDS for Gamma_Q [S | z];
//                       intra-group term from masked Gamma_Q Gamma_K^T MFMA tiles (zero-filled
//                       above the diagonal, so positions after i never reach O_i).
#include <math.h>

#include "gma_internal.h"
#include "gma_mfma_common.h"
#include "gma_mfma_geo.h"
#include "gma_numeric.h"

namespace gma {
namespace mf {
namespace {

constexpr int kGroup = kIterT;  // 128 positions per scan step (one 32-position chunk per wave)

struct CausalLayout {
    size_t W, C, gq, gk, gkt, carry, total;
    int S, seg_len, Np;
};

int causal_segments(const gma_desc& d) {
    const int bh = d.B * d.H;
    const int groups = (d.N + kGroup - 1) / kGroup;
    int s = (256 + bh - 1) / bh;
    if (s > groups) s = groups;
    if (s > 64) s = 64;
    return s < 1 ? 1 : s;
}

CausalLayout causal_layout(const gma_desc& d) {
    const Geo g = geometry(d);
    const size_t BH = (size_t)d.B * d.H;
    CausalLayout L;
    L.S = causal_segments(d);
    L.seg_len = ((d.N + L.S - 1) / L.S + kGroup - 1) / kGroup * kGroup;
    L.S = (d.N + L.seg_len - 1) / L.seg_len;
    if (L.S < 1) L.S = 1;
    L.Np = (d.N + kGroup - 1) / kGroup * kGroup;
    size_t off = 0;
    L.W = off;
    off += align_up((size_t)d.H * g.Kp * 4 * g.Dp * sizeof(bf16_t));
    L.C = off;
    off += align_up((size_t)d.H * g.Kp * sizeof(float));
    L.gq = off;
    off += align_up(BH * L.Np * g.Kp * sizeof(bf16_t));
    L.gk = off;
    off += align_up(BH * L.Np * g.Kp * sizeof(bf16_t));
    L.gkt = off;
    off += align_up(BH * L.Np * g.Kp * sizeof(bf16_t));
    L.carry = off;
    off += align_up(BH * L.S * g.Kp * (g.Dvp + 1) * sizeof(float));
    L.total = off;
    return L;
}

inline int cvstride(const Geo& g) { return 2 * g.Dvp + 32; }
inline int shstride(const Geo& g) { return 2 * g.Kp + 16; }
inline size_t totals_lds_bytes(const Geo& g) { return (size_t)kGroup * cvstride(g); }
inline size_t scan_lds_bytes(const Geo& g) {
    return (size_t)kGroup * cvstride(g) + (size_t)(g.Dvp + 32) * shstride(g);
}

// ----------------------------------------------------------------------------- responsibilities
// Columns [c0, c0 + ncp) of every 16-wide chunk block of the head's coefficient rows into
// LDS (rows [ah | al | bh | bl] of ncp chunks each, stride wstride bytes), and c_k.
__device__ __forceinline__ void stage_coefficient_chunks(unsigned char* sW, float* sC, const bf16_t* W,
                                                         const float* cvec, int h, int Kp, int Dp, int c0, int ncp,
                                                         int wstride) {
    const bf16_t* src = W + (size_t)h * Kp * 4 * Dp;
    const int vec_per_piece = 2 * ncp;  // 16-byte vectors per piece of a row
    const int per_row = 4 * vec_per_piece;
    const int total = Kp * per_row;
    for (int i0 = threadIdx.x; i0 < total; i0 += 8 * blockDim.x) {
        bf16x8 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * blockDim.x;
            if (i < total) {
                const int r = i / per_row, rem = i % per_row;
                const int piece = rem / vec_per_piece, vv = rem % vec_per_piece;
                v[u] = *reinterpret_cast<const bf16x8*>(src + (size_t)r * 4 * Dp + piece * Dp + 16 * c0 + 8 * vv);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * blockDim.x;
            if (i < total) {
                const int r = i / per_row, rem = i % per_row;
                *reinterpret_cast<bf16x8*>(sW + (size_t)r * wstride + 16 * rem) = v[u];
            }
        }
    }
    for (int i = threadIdx.x; i < Kp; i += blockDim.x) sC[i] = cvec[(size_t)h * Kp + i];
}

// Eight waves (two per SIMD, so one wave's exponentials overlap the other's MFMAs); each
// wave handles one 32-position tile per 256-position step (one side per block row,
// blockIdx.y: 0 queries, 1 keys): logits (MFMA), softmax over the components, normalised
// responsibilities stored token-major as bf16; positions in [N, Np) get zeros.  When the
// coefficient block of a head exceeds LDS it is staged in NPH phases of the routing dims,
// the logits accumulating across phases.  The key side also stores Gamma_K component-major:
// a 32x32 MFMA against a permutation matrix moves the components from registers to lanes.
constexpr int kRespWaves = 8;

template <int MT, int NC, int NPH>
__global__ void __launch_bounds__(64 * kRespWaves, 2)
    gma_causal_resp(const bf16_t* __restrict__ qr, const bf16_t* __restrict__ kr, const bf16_t* __restrict__ W,
                    const float* __restrict__ cvec, bf16_t* __restrict__ GQ, bf16_t* __restrict__ GK,
                    bf16_t* __restrict__ GKT, int BH, int H, int N, int Np, int dr, int parts, int part_len) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int Kp = 32 * MT, Dp = 16 * NC, NCP = NC / NPH;
    constexpr int wstride = 8 * (16 * NCP) + 16;
    constexpr int kStep = kTileT * kRespWaves;
    unsigned char* sW = smem;
    float* sC = reinterpret_cast<float*>(smem + (size_t)Kp * wstride);
    int bh, part;
    head_part(blockIdx.x, BH, parts, bh, part);
    const int h = bh % H;
    const int l = lane_id(), w = wave_id(), half = l >> 5, col = l & 31;
    const int side = blockIdx.y;
    const bf16_t* x = (side == 0 ? qr : kr) + (size_t)bh * N * dr;
    bf16_t* G = (side == 0 ? GQ : GK) + (size_t)bh * Np * Kp;
    bf16_t* gt = GKT + (size_t)bh * Kp * Np;
    // permutation operands: B_s[c][k'] = 1 iff k' == 16 s + kperm(c) (c = 8 half + e)
    bf16x8 perm[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) perm[s2][e] = (short)(col == 16 * s2 + kperm(8 * half + e) ? 0x3f80 : 0);

    const int n_begin = part * part_len;
    const int n_end = min(Np, n_begin + part_len);
    auto row = [&](int b0) -> const bf16_t* {
        const int t = b0 + kTileT * w + col;
        return (t < n_end && t < N) ? x + (size_t)t * dr : nullptr;
    };
    bf16x8 xr[NC];
    load_xrow<NC>(xr, row(n_begin), dr);
    if (NPH == 1) {
        stage_coefficient_chunks(sW, sC, W, cvec, h, Kp, Dp, 0, NC, wstride);
        __syncthreads();
    }
    for (int b0 = n_begin; b0 < n_end; b0 += kStep) {
        const int t0 = b0 + kTileT * w;  // this wave's tile
        const int t = t0 + col;
        const bool valid = t < N;
        f32x16 acc[MT];
        if (NPH == 1) {
            tile_logits_overlap<MT, NCP, true>(acc, xr, sW, wstride, sC, [](int, int) {});
        } else {
#pragma unroll
            for (int ph = 0; ph < NPH; ++ph) {
                lds_barrier();
                stage_coefficient_chunks(sW, sC, W, cvec, h, Kp, Dp, ph * NCP, NCP, wstride);
                __syncthreads();
                if (ph == 0)
                    tile_logits_overlap<MT, NCP, true>(acc, xr, sW, wstride, sC, [](int, int) {});
                else
                    tile_logits_overlap<MT, NCP, false>(acc, xr + ph * NCP, sW, wstride, sC, [](int, int) {});
            }
        }
        load_xrow<NC>(xr, row(b0 + kStep), dr);  // next step's rows, in flight during the softmax
        const float s = tile_exp<MT>(acc);
        const float inv = valid ? 1.0f / s : 0.0f;
        if (t0 < n_end) {
            bf16_t* grow = G + (size_t)t * Kp;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const bf16x8 g0 = pack8(acc[m], 0, inv), g1 = pack8(acc[m], 8, inv);
                const u32x4 p0 = __builtin_bit_cast(u32x4, g0), p1 = __builtin_bit_cast(u32x4, g1);
                // registers 4q..4q+3 hold components 32m + 8q + 4 half + (0..3)
                *reinterpret_cast<uint2*>(grow + 32 * m + 0 + 4 * half) = make_uint2(p0[0], p0[1]);
                *reinterpret_cast<uint2*>(grow + 32 * m + 8 + 4 * half) = make_uint2(p0[2], p0[3]);
                *reinterpret_cast<uint2*>(grow + 32 * m + 16 + 4 * half) = make_uint2(p1[0], p1[1]);
                *reinterpret_cast<uint2*>(grow + 32 * m + 24 + 4 * half) = make_uint2(p1[2], p1[3]);
                if (side == 1) {
                    // D[t][k'] = sum_c G[t][c] B[c][k']: rows = positions, lanes = components
                    f32x16 tr;
#pragma unroll
                    for (int i = 0; i < 16; ++i) tr[i] = 0.0f;
                    tr = mfma(g0, perm[0], tr);
                    tr = mfma(g1, perm[1], tr);
                    bf16_t* trow = gt + (size_t)(32 * m + col) * Np + t0;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint2*>(trow + 8 * q + 4 * half) = make_uint2(
                            pack_bf16(tr[4 * q], tr[4 * q + 1]), pack_bf16(tr[4 * q + 2], tr[4 * q + 3]));
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------- state update
// V rows [base, base + 128) into sV (zero past n_end), each wave its 32 rows.
template <int NT>
__device__ __forceinline__ void stage_v(unsigned char* sV, int vs, const bf16_t* v_h, int base, int n_end, int dv) {
    const int l = lane_id(), w = wave_id(), half = l >> 5;
    const int t = base + kTileT * w + (l & 31);
    const bf16_t* row = t < n_end ? v_h + (size_t)t * dv : nullptr;
    unsigned char* dst = sV + (size_t)(kTileT * w + (l & 31)) * vs;
#pragma unroll
    for (int j = 0; j < 2 * NT; ++j) {
        const int d0 = 16 * j + 8 * half;
        bf16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
        if (row) {
            if ((dv & 7) == 0) {
                if (d0 < dv) x = *reinterpret_cast<const bf16x8*>(row + d0);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (d0 + e < dv) x[e] = (short)row[d0 + e];
            }
        }
        *reinterpret_cast<bf16x8*>(dst + 2 * d0) = x;
    }
}

// acc(tile m, n) += Gamma_K^T [k-tile m, 128 staged positions] x [V | 1][positions, d-tile n]
// for this wave's output tiles (tiles dealt in contiguous m-major runs; n == NT is the ones
// tile whose every column accumulates z_k).
template <int MT, int NT, int PW>
__device__ __forceinline__ void update_group(f32x16 (&acc)[PW], const bf16_t* gkt_h, int Np, int base,
                                             const unsigned char* sV, int vs) {
    constexpr int Tiles = MT * (NT + 1);
    const int l = lane_id(), w = wave_id(), half = l >> 5;
    bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (short)0x3f80;
#pragma unroll
    for (int ks = 0; ks < kGroup / 16; ++ks) {
        int last_m = -1;
        bf16x8 a;
#pragma unroll
        for (int j = 0; j < PW; ++j) {
            const int tile = w * PW + j;
            if (tile < Tiles) {
                const int m = tile / (NT + 1), n = tile % (NT + 1);
                if (m != last_m) {
                    a = *reinterpret_cast<const bf16x8*>(gkt_h + (size_t)(32 * m + (l & 31)) * Np + base + 16 * ks +
                                                         8 * half);
                    last_m = m;
                }
                const bf16x8 b = (n < NT) ? lds_frag_tr(sV, vs, 16 * ks, 32 * n) : ones;
                acc[j] = mfma(a, b, acc[j]);
            }
        }
    }
}

template <int MT, int NT>
__global__ void __launch_bounds__(kThreads, 1)
    gma_causal_totals(const bf16_t* __restrict__ GKT, const bf16_t* __restrict__ v, float* __restrict__ carry,
                      int BH, int N, int Np, int dv, int S, int seg_len) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int Kp = 32 * MT, Dvp = 32 * NT;
    constexpr int vs = 2 * Dvp + 32;
    constexpr int Tiles = MT * (NT + 1);
    constexpr int PW = (Tiles + kWaves - 1) / kWaves;
    int bh, seg;
    head_part(blockIdx.x, BH, S - 1, bh, seg);
    const int l = lane_id(), w = wave_id(), half = l >> 5;
    const int n_begin = seg * seg_len, n_end = min(N, n_begin + seg_len);
    f32x16 acc[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
    const bf16_t* gkt_h = GKT + (size_t)bh * Kp * Np;
    const bf16_t* v_h = v + (size_t)bh * N * dv;
    for (int base = n_begin; base < n_end; base += kGroup) {
        stage_v<NT>(smem, vs, v_h, base, n_end, dv);
        lds_barrier();
        update_group<MT, NT, PW>(acc, gkt_h, Np, base, smem, vs);
        lds_barrier();
    }
    float* T = carry + ((size_t)bh * S + seg) * Kp * (Dvp + 1);
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int tile = w * PW + j;
        if (tile < Tiles) {
            const int m = tile / (NT + 1), n = tile % (NT + 1);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int k = 32 * m + 8 * (i >> 2) + 4 * half + (i & 3);
                if (n < NT)
                    T[(size_t)k * (Dvp + 1) + 32 * n + (l & 31)] = acc[j][i];
                else if ((l & 31) == 0)
                    T[(size_t)k * (Dvp + 1) + Dvp] = acc[j][i];
            }
        }
    }
}

// In place: slot s <- sum of the totals of segments 0..s-1 (slot 0 <- 0), in segment order.
__global__ void __launch_bounds__(256) gma_causal_carry(float* __restrict__ carry, int BH, int S, int per) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)BH * per) return;
    const size_t bh = idx / per, e = idx % per;
    float* c = carry + bh * S * per + e;
    float run = 0.0f;
    for (int s0 = 0; s0 < S; s0 += 16) {
        float t[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) t[u] = (s0 + u < S - 1) ? c[(size_t)(s0 + u) * per] : 0.0f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (s0 + u < S) c[(size_t)(s0 + u) * per] = run;
            run += t[u];
        }
    }
}

// ----------------------------------------------------------------------------- scan
// Shadow (bf16, LDS) of the state, rows: S^T (Dvp rows, d), then z hi (8 rows), z lo (8 rows)
// and 16 rows of ones; columns = components in natural order.  Written from this wave's
// accumulator tiles.
template <int MT, int NT, int PW>
__device__ __forceinline__ void write_shadow(unsigned char* sS, int ss, const f32x16 (&acc)[PW]) {
    constexpr int Tiles = MT * (NT + 1);
    constexpr int Dvp = 32 * NT;
    const int l = lane_id(), w = wave_id(), half = l >> 5, col = l & 31;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int tile = w * PW + j;
        if (tile < Tiles) {
            const int m = tile / (NT + 1), n = tile % (NT + 1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k0 = 32 * m + 8 * q + 4 * half;
                const float v0 = acc[j][4 * q], v1 = acc[j][4 * q + 1], v2 = acc[j][4 * q + 2],
                            v3 = acc[j][4 * q + 3];
                if (n < NT) {
                    uint2 p;
                    p.x = pack_bf16(v0, v1);
                    p.y = pack_bf16(v2, v3);
                    *reinterpret_cast<uint2*>(sS + (size_t)(32 * n + col) * ss + 2 * k0) = p;
                } else if (col < 16) {
                    // z: rows Dvp..Dvp+7 hi part, Dvp+8..Dvp+15 lo part
                    uint2 hi, lo;
                    hi.x = pack_bf16(v0, v1);
                    hi.y = pack_bf16(v2, v3);
                    lo.x = pack_bf16(v0 - bf16lo_to_f32(hi.x), v1 - bf16hi_to_f32(hi.x));
                    lo.y = pack_bf16(v2 - bf16lo_to_f32(hi.y), v3 - bf16hi_to_f32(hi.y));
                    *reinterpret_cast<uint2*>(sS + (size_t)(Dvp + col) * ss + 2 * k0) = col < 8 ? hi : lo;
                }
            }
        }
    }
}

template <int MT, int NT>
__global__ void __launch_bounds__(kThreads, 1)
    gma_causal_scan(const bf16_t* __restrict__ GQ, const bf16_t* __restrict__ GK, const bf16_t* __restrict__ GKT,
                    const bf16_t* __restrict__ v, const float* __restrict__ carry, bf16_t* __restrict__ out,
                    float eps, int BH, int N, int Np, int dv, int S, int seg_len) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int Kp = 32 * MT, Dvp = 32 * NT;
    constexpr int vs = 2 * Dvp + 32, ss = 2 * Kp + 16;
    constexpr int Tiles = MT * (NT + 1);
    constexpr int PW = (Tiles + kWaves - 1) / kWaves;
    constexpr int KS = Kp / 16;  // 16-wide contraction steps over the components
    unsigned char* sV = smem;
    unsigned char* sS = smem + (size_t)kGroup * vs;

    int bh, seg;
    head_part(blockIdx.x, BH, S, bh, seg);
    const int l = lane_id(), w = wave_id(), half = l >> 5, col = l & 31;
    const int n_begin = seg * seg_len, n_end = min(N, n_begin + seg_len);

    // state entering this segment (fp32, this wave's output tiles)
    f32x16 st[PW];
    const float* cin = carry + ((size_t)bh * S + seg) * Kp * (Dvp + 1);
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int tile = w * PW + j;
        const int m = tile / (NT + 1), n = tile % (NT + 1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = 32 * m + 8 * (i >> 2) + 4 * half + (i & 3);
            st[j][i] = (tile < Tiles) ? cin[(size_t)k * (Dvp + 1) + (n < NT ? 32 * n + col : Dvp)] : 0.0f;
        }
    }
    // constant rows of the shadow: ones (den tile rows 16..31)
    for (int i = threadIdx.x; i < 16 * Kp; i += blockDim.x)
        *reinterpret_cast<bf16_t*>(sS + (size_t)(Dvp + 16 + i / Kp) * ss + 2 * (i % Kp)) = (bf16_t)0x3f80;
    write_shadow<MT, NT, PW>(sS, ss, st);

    const bf16_t* gq_h = GQ + (size_t)bh * Np * Kp;
    const bf16_t* gk_h = GK + (size_t)bh * Np * Kp;
    const bf16_t* gkt_h = GKT + (size_t)bh * Kp * Np;
    const bf16_t* v_h = v + (size_t)bh * N * dv;
    bf16_t* o_h = out + (size_t)bh * N * dv;
    // den-tile operand for the intra term: ones in rows 0..7 (they add to the z-hi rows)
    bf16x8 den_ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) den_ones[j] = (short)(col < 8 ? 0x3f80 : 0);

    for (int base = n_begin; base < n_end; base += kGroup) {
        stage_v<NT>(sV, vs, v_h, base, n_end, dv);
        lds_barrier();
        // ---- outputs of chunk w: positions base + 32w + col
        {
            const int i0 = base + kTileT * w;
            const int t = i0 + col;
            bf16x8 qf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ks] = *reinterpret_cast<const bf16x8*>(gq_h + (size_t)t * Kp + 16 * ks + 8 * half);
            f32x16 o[NT + 1];
#pragma unroll
            for (int n = 0; n <= NT; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[n][i] = 0.0f;
            // inter-group: Gamma_Q [S | z] from the shadow
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int n = 0; n <= NT; ++n) {
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8*>(sS + (size_t)(32 * n + col) * ss + 2 * (16 * ks + 8 * half));
                    o[n] = mfma(a, qf[ks], o[n]);
                }
            // intra-group: chunks c <= w; A[j', i] = gamma_K,j' . gamma_Q,i, zero for j' > i
            for (int c = 0; c <= w; ++c) {
                f32x16 aff;
#pragma unroll
                for (int i = 0; i < 16; ++i) aff[i] = 0.0f;
                const bf16_t* krow = gk_h + (size_t)(base + kTileT * c + col) * Kp;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    aff = mfma(*reinterpret_cast<const bf16x8*>(krow + 16 * ks + 8 * half), qf[ks], aff);
                if (c == w) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int jrow = 8 * (i >> 2) + 4 * half + (i & 3);
                        aff[i] = (jrow <= col) ? aff[i] : 0.0f;
                    }
                }
#pragma unroll
                for (int sh = 0; sh < 2; ++sh) {
                    const bf16x8 b = pack8(aff, 8 * sh, 1.0f);
#pragma unroll
                    for (int n = 0; n < NT; ++n)
                        o[n] = mfma(lds_frag_tr_crows(sV, vs, kTileT * c + 16 * sh, 32 * n), b, o[n]);
                    o[NT] = mfma(den_ones, b, o[NT]);
                }
            }
            const float den = o[NT][0] + o[NT][4];
            const float inv = 1.0f / (den + eps);
            if (t < n_end) {
                bf16_t* orow = o_h + (size_t)t * dv;
#pragma unroll
                for (int n = 0; n < NT; ++n)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int d0 = 32 * n + 8 * q + 4 * half;
                        if ((dv & 3) == 0) {
                            if (d0 < dv) {
                                uint2 p;
                                p.x = pack_bf16(o[n][4 * q] * inv, o[n][4 * q + 1] * inv);
                                p.y = pack_bf16(o[n][4 * q + 2] * inv, o[n][4 * q + 3] * inv);
                                *reinterpret_cast<uint2*>(orow + d0) = p;
                            }
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (d0 + r < dv) orow[d0 + r] = (bf16_t)bf16_bits_rne(o[n][4 * q + r] * inv);
                        }
                    }
            }
        }
        // ---- state += Gamma_K^T [V | 1] over the group (this wave's tiles)
        update_group<MT, NT, PW>(st, gkt_h, Np, base, sV, vs);
        lds_barrier();  // every wave is done reading sV and the old shadow
        write_shadow<MT, NT, PW>(sS, ss, st);
    }
}

// ----------------------------------------------------------------------------- dispatch
typedef void (*RespFn)(const bf16_t*, const bf16_t*, const bf16_t*, const float*, bf16_t*, bf16_t*, bf16_t*, int, int,
                       int, int, int, int, int);
typedef void (*TotFn)(const bf16_t*, const bf16_t*, float*, int, int, int, int, int, int);
typedef void (*ScanFn)(const bf16_t*, const bf16_t*, const bf16_t*, const bf16_t*, const float*, bf16_t*, float, int,
                       int, int, int, int, int);

template <int MT, int NC>
RespFn resp_fn(int nph) {
    if (nph == 1) return gma_causal_resp<MT, NC, 1>;
    if (nph == 2 && NC % 2 == 0) return gma_causal_resp<MT, NC, (NC % 2 == 0 ? 2 : 1)>;
    if (nph == 4 && NC % 4 == 0) return gma_causal_resp<MT, NC, (NC % 4 == 0 ? 4 : 1)>;
    return nullptr;
}
template <int MT>
RespFn resp_fn_nc(int NC, int nph) {
    switch (NC) {
        case 1: return resp_fn<MT, 1>(nph);
        case 2: return resp_fn<MT, 2>(nph);
        case 4: return resp_fn<MT, 4>(nph);
        case 8: return resp_fn<MT, 8>(nph);
    }
    return nullptr;
}
RespFn select_resp(const Geo& g, int nph) {
    switch (g.MT) {
        case 1: return resp_fn_nc<1>(g.NC, nph);
        case 2: return resp_fn_nc<2>(g.NC, nph);
        case 4: return resp_fn_nc<4>(g.NC, nph);
        case 8: return resp_fn_nc<8>(g.NC, nph);
    }
    return nullptr;
}
// LDS of the responsibilities kernel with the routing dims staged in nph phases.
size_t resp_lds(const Geo& g, int nph) {
    return (size_t)g.Kp * (8 * 16 * (g.NC / nph) + 16) + (size_t)g.Kp * 4;
}
int resp_phases(const Geo& g) {
    for (int nph = 1; nph <= g.NC && nph <= 4; nph *= 2)
        if (resp_lds(g, nph) <= kLdsMax) return nph;
    return 0;
}
template <int MT>
bool select_scan_nt(int NT, TotFn& tf, ScanFn& sf) {
    switch (NT) {
        case 1: tf = gma_causal_totals<MT, 1>; sf = gma_causal_scan<MT, 1>; return true;
        case 2: tf = gma_causal_totals<MT, 2>; sf = gma_causal_scan<MT, 2>; return true;
        case 4: tf = gma_causal_totals<MT, 4>; sf = gma_causal_scan<MT, 4>; return true;
    }
    return false;
}
bool select_scan(const Geo& g, TotFn& tf, ScanFn& sf) {
    switch (g.MT) {
        case 1: return select_scan_nt<1>(g.NT, tf, sf);
        case 2: return select_scan_nt<2>(g.NT, tf, sf);
        case 4: return select_scan_nt<4>(g.NT, tf, sf);
        case 8: return select_scan_nt<8>(g.NT, tf, sf);
    }
    return false;
}

hipError_t set_lds(const void* f, size_t bytes) {
    return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

bool causal_supported(const gma_desc& d) {
    const Geo g = geometry(d);
    return scan_lds_bytes(g) <= kLdsMax && totals_lds_bytes(g) <= kLdsMax && resp_phases(g) > 0;
}

size_t causal_workspace(const gma_desc& d) { return causal_layout(d).total; }

hipError_t causal_forward(const Args& a) {
    const gma_desc& d = a.d;
    const Geo g = geometry(d);
    const CausalLayout L = causal_layout(d);
    bf16_t* W = reinterpret_cast<bf16_t*>(a.ws + L.W);
    float* cvec = reinterpret_cast<float*>(a.ws + L.C);
    bf16_t* GQ = reinterpret_cast<bf16_t*>(a.ws + L.gq);
    bf16_t* GK = reinterpret_cast<bf16_t*>(a.ws + L.gk);
    bf16_t* GKT = reinterpret_cast<bf16_t*>(a.ws + L.gkt);
    float* carry = reinterpret_cast<float*>(a.ws + L.carry);
    const int BH = d.B * d.H;
    hipError_t e;

    const int nph = resp_phases(g);
    RespFn rf = nph ? select_resp(g, nph) : nullptr;
    TotFn tf;
    ScanFn sf;
    if (!rf || !select_scan(g, tf, sf)) return hipErrorNotSupported;

    if ((e = launch_prep(a, g, W, cvec)) != hipSuccess) return e;

    // responsibilities of both sides, ~one workgroup per CU per side
    const int rstep = kTileT * kRespWaves;
    int parts = (256 + BH - 1) / BH;
    const int max_parts = (L.Np + rstep - 1) / rstep;
    if (parts > max_parts) parts = max_parts;
    if (parts < 1) parts = 1;
    const int part_len = ((L.Np + parts - 1) / parts + rstep - 1) / rstep * rstep;
    parts = (L.Np + part_len - 1) / part_len;
    const size_t rl = resp_lds(g, nph);
    if ((e = set_lds(reinterpret_cast<const void*>(rf), rl)) != hipSuccess) return e;
    rec_begin(a, "gma_causal_resp");
    hipLaunchKernelGGL(rf, dim3(BH * parts, 2), dim3(64 * kRespWaves), rl, a.stream, static_cast<const bf16_t*>(a.qr),
                       static_cast<const bf16_t*>(a.kr), W, cvec, GQ, GK, GKT, BH, d.H, d.N, L.Np, d.d_r, parts,
                       part_len);
    rec_end(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const int per = g.Kp * (g.Dvp + 1);
    if (L.S > 1) {
        const size_t tl = totals_lds_bytes(g);
        if ((e = set_lds(reinterpret_cast<const void*>(tf), tl)) != hipSuccess) return e;
        rec_begin(a, "gma_causal_totals");
        hipLaunchKernelGGL(tf, dim3(BH * (L.S - 1)), dim3(kThreads), tl, a.stream, GKT,
                           static_cast<const bf16_t*>(a.v), carry, BH, d.N, L.Np, d.d_v, L.S, L.seg_len);
        rec_end(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    rec_begin(a, "gma_causal_carry");
    gma_causal_carry<<<dim3((unsigned)(((size_t)BH * per + 255) / 256)), dim3(256), 0, a.stream>>>(carry, BH, L.S,
                                                                                                   per);
    rec_end(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const size_t sl = scan_lds_bytes(g);
    if ((e = set_lds(reinterpret_cast<const void*>(sf), sl)) != hipSuccess) return e;
    rec_begin(a, "gma_causal_scan");
    hipLaunchKernelGGL(sf, dim3(BH * L.S), dim3(kThreads), sl, a.stream, GQ, GK, GKT, static_cast<const bf16_t*>(a.v),
                       carry, static_cast<bf16_t*>(a.out), a.eps, BH, d.N, L.Np, d.d_v, L.S, L.seg_len);
    rec_end(a);
    return hipGetLastError();
}

}  // namespace mf
}  // namespace gma
