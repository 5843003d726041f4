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
// state entering segment s is the sum of the totals Gamma_K^T [V | 1] of the positions
// before it, added in a fixed order (deterministic).  Value dims are processed in slices of
// at most 64 (one workgroup per slice; each slice carries its own copy of z).
//
// Responsibilities in memory.  Gamma_Q and Gamma_K (normalised, bf16) are stored in MFMA
// operand order: for every 32-position tile and every 16-wide block ks of components, the
// 64 lanes' 16-byte fragments lie contiguously (lane l = position l % 32 of the tile, holding
// slots 8 (l / 32) .. + 7 of the block).  Every store of the producer and every load of the
// consumers is then one contiguous 1 KB access per wave.  The slot order inside a block is
// the C-register order of the logits tile, i.e. slot s holds component 16 ks + kperm(s); all
// consumers index components by slot, so the state [S | z] is kept in the same order.
//
// Kernels (all on the caller's stream, in this order):
//   gma_prep            (shared with the bidirectional path) coefficients and c_k
//   gma_causal_resp     Gamma_Q and Gamma_K of every position (logit MFMAs + softmax)
//   gma_causal_totals   Gamma_K^T [V | 1] of fixed-length sub-segments before the last
//                       segment (only when S > 1)
//   gma_causal_scan     one workgroup per (head, segment, value slice); its prologue forms
//                       the state entering the segment as the ordered sum of the sub-segment
//                       totals before it; then sequential groups of
//                       128 positions; fp32 state in MFMA accumulators split over the 4 waves
//                       by output tile, bf16 shadow of the full state in LDS for
//                       Gamma_Q [S | z]; Gamma_K rows of the group staged in LDS for the
//                       masked intra-group tiles (zero-filled above the diagonal, so
//                       positions after i never reach O_i) and the state update.  The next
//                       group's Gamma_K, Gamma_Q and V are loaded into registers while the
//                       current group computes.
#include <math.h>

#include "gma_internal.h"
#include "gma_mfma_common.h"
#include "gma_mfma_geo.h"
#include "gma_numeric.h"

namespace gma {
namespace mf {
namespace {

constexpr int kGroup = kIterT;  // 128 positions per scan step (one 32-position chunk per wave)
constexpr int kSliceV = 64;     // value dims per scan workgroup
constexpr int kFrag = 64 * 8;   // bf16 elements of one operand fragment block (64 lanes x 8)

struct CausalLayout {
    size_t W, C, gq, gk, tpart, total;
    int S, seg_len, Np;     // segments, their length (multiple of kGroup), padded sequence
    int NS, Dvs;            // value slices and their width (padded)
    int TS, nsub, sub_len;  // totals: sub-segments per segment, their count and length
};

CausalLayout causal_layout(const gma_desc& d) {
    const Geo g = geometry(d);
    const int BH = d.B * d.H;
    CausalLayout L;
    L.Dvs = g.Dvp < kSliceV ? g.Dvp : kSliceV;
    L.NS = g.Dvp / L.Dvs;
    const int groups = (d.N + kGroup - 1) / kGroup;
    int s = (256 + BH * L.NS - 1) / (BH * L.NS);
    if (s > groups) s = groups;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    L.seg_len = ((d.N + s - 1) / s + kGroup - 1) / kGroup * kGroup;
    L.S = (d.N + L.seg_len - 1) / L.seg_len;
    if (L.S < 1) L.S = 1;
    L.Np = groups * kGroup;
    // totals: split every segment before the last into TS equal sub-segments so that about
    // 256 workgroups run; TS divides the segment's group count
    const int seg_groups = L.seg_len / kGroup;
    L.TS = 1;
    if (L.S > 1) {
        const int want = (256 + BH * (L.S - 1) * L.NS - 1) / (BH * (L.S - 1) * L.NS);
        for (int t = 1; t <= seg_groups && t <= want; ++t)
            if (seg_groups % t == 0) L.TS = t;
    }
    L.sub_len = L.seg_len / L.TS;
    L.nsub = (L.S - 1) * L.TS;
    const size_t per = (size_t)g.Kp * (L.Dvs + 1);
    size_t off = 0;
    L.W = off;
    off += align_up((size_t)d.H * g.Kp * 4 * g.Dp * sizeof(bf16_t));
    L.C = off;
    off += align_up((size_t)d.H * g.Kp * sizeof(float));
    L.gq = off;
    off += align_up((size_t)BH * L.Np * g.Kp * sizeof(bf16_t));
    L.gk = off;
    off += align_up((size_t)BH * L.Np * g.Kp * sizeof(bf16_t));
    L.tpart = off;
    off += align_up((size_t)BH * L.nsub * L.NS * per * sizeof(float));
    L.total = off;
    return L;
}

inline int gstride(int Kp) { return 2 * Kp + 32; }
inline int vstride(int Dvs) { return 2 * Dvs + 32; }
inline int shstride(int Kp) { return 2 * Kp + 16; }
inline size_t totals_lds_bytes(const Geo& g, int Dvs) {
    return (size_t)kGroup * gstride(g.Kp) + (size_t)kGroup * vstride(Dvs);
}
inline size_t scan_lds_bytes(const Geo& g, int Dvs) {
    return totals_lds_bytes(g, Dvs) + (size_t)(Dvs + 32) * shstride(g.Kp);
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

// ---- soft usage inside the responsibilities kernel (statistics mode)
// Sum over the 32 tokens of a tile (lanes l % 32 of each half) of every component, as a
// reduce-scatter: five exchange stages, each pairing lane l with a partner that differs in
// one lane bit (l ^ 16: lane swap; l ^ 8: DPP row rotate by 8; 7 - l mod 8: DPP half-row
// mirror; l ^ 2, l ^ 1: DPP quad permutes).  At each stage a lane keeps the lower or the
// upper half of its values (by that bit) and adds the partner's copy of that half, so the
// 16 MT values of a lane end as MT / 2 sums (tokens added in a fixed pairing order) of the
// flattened indices (MT / 2) (l % 32) .. + MT / 2 - 1; for MT = 1 the last stage adds the
// pair's single values instead (both lanes of the pair then hold the same sum).
template <int STAGE>
__device__ __forceinline__ float rs_partner(float x) {
    if constexpr (STAGE == 0) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float((lane_id() >> 4) & 1 ? r[0] : r[1]);
    } else {
        constexpr int ctrl = STAGE == 1 ? 0x128 : STAGE == 2 ? 0x141 : STAGE == 3 ? 0x4E : 0xB1;
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xf, 0xf, false));
    }
}
template <int STAGE, int N>
__device__ __forceinline__ void rs_stage(const float (&v)[N], float (&o)[N / 2]) {
    const bool bit = (lane_id() >> (4 - STAGE)) & 1;
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const float keep = bit ? v[j + N / 2] : v[j];
        const float send = bit ? v[j] : v[j + N / 2];
        o[j] = keep + rs_partner<STAGE>(send);
    }
}
// v: the tile's values (16 MT, flattened 16 m + e); out: this lane's F = max(1, MT / 2) sums.
template <int MT>
__device__ __forceinline__ void tile_token_sums(const float (&v)[16 * MT], float (&out)[MT >= 2 ? MT / 2 : 1]) {
    float a[8 * MT], b[4 * MT], c[2 * MT], d[MT];
    rs_stage<0>(v, a);
    rs_stage<1>(a, b);
    rs_stage<2>(b, c);
    rs_stage<3>(c, d);
    if constexpr (MT >= 2) {
        rs_stage<4>(d, out);
    } else {
        out[0] = d[0] + rs_partner<4>(d[0]);
    }
}

// Eight waves (two per SIMD, so one wave's exponentials overlap the other's MFMAs); each
// wave handles one 32-position tile per 256-position step (one side per block row,
// blockIdx.y: 0 queries, 1 keys): logits (MFMA), softmax over the components, normalised
// responsibilities stored as bf16 operand fragments; positions in [N, Np) get zeros.  When
// the coefficient block of a head exceeds LDS it is staged in NPH phases of the routing
// dims, the logits accumulating across phases.  MODE kRespStats: instead of fragments, the
// hard assignment of every position of side 0, argmax of its fp32 logits (lowest component
// among equal maxima), into hard [BH][N], and the workgroup's soft usage (its positions'
// float32 responsibilities summed per component: per tile across the tokens, per lane
// across tiles, then across the waves in wave order) as float32 [BH parts][Kp] into GK
// reinterpreted as float (natural component order).  MODE kRespRows: instead of fragments, the normalised
// responsibilities as float32 rows [BH][N][K] (components < K) into GQ / GK reinterpreted
// as float (the backward's layout).
constexpr int kRespWaves = 8;
constexpr int kRespFrag = 0, kRespStats = 1, kRespRows = 2;

template <int MT, int NC, int NPH, int MODE>
__global__ void __launch_bounds__(64 * kRespWaves, 2)
    gma_causal_resp(const bf16_t* __restrict__ qr, const bf16_t* __restrict__ kr, const bf16_t* __restrict__ W,
                    const float* __restrict__ cvec, bf16_t* __restrict__ GQ, bf16_t* __restrict__ GK,
                    int* __restrict__ hard, int BH, int H, int N, int Np, int dr, int parts, int part_len, int K) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int Kp = 32 * MT, Dp = 16 * NC, NCP = NC / NPH, KS = Kp / 16;
    constexpr int wstride = 8 * (16 * NCP) + 16;
    constexpr int kStep = kTileT * kRespWaves;
    unsigned char* sW = smem;
    float* sC = reinterpret_cast<float*>(smem + (size_t)Kp * wstride);
    int bh, part;
    head_part(blockIdx.x, BH, parts, bh, part);
    const int h = bh % H;
    const int l = lane_id(), w = wave_id(), col = l & 31;
    const int side = blockIdx.y;
    const bf16_t* x = (side == 0 ? qr : kr) + (size_t)bh * N * dr;
    bf16_t* G = (side == 0 ? GQ : GK) + (size_t)bh * Np * Kp + 8 * l;

    const int n_begin = part * part_len;
    const int n_end = min(Np, n_begin + part_len);
    // positions past the sequence read its last row (their responsibilities are zeroed)
    auto row = [&](int b0) -> const bf16_t* { return x + (size_t)min(b0 + kTileT * w + col, N - 1) * dr; };
    bf16x8 xr[NC];
    load_xrow<NC>(xr, row(n_begin), dr);
    if (NPH == 1) {
        stage_coefficient_chunks(sW, sC, W, cvec, h, Kp, Dp, 0, NC, wstride);
        __syncthreads();
    }
    constexpr int UF = MT >= 2 ? MT / 2 : 1;  // usage sums per lane (statistics mode)
    float us[UF];
#pragma unroll
    for (int i = 0; i < UF; ++i) us[i] = 0.0f;
    for (int b0 = n_begin; b0 < n_end; b0 += kStep) {
        const int t0 = b0 + kTileT * w;  // this wave's tile
        const bool valid = t0 + col < N;
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
        if constexpr (MODE == kRespStats) {
            // register e of tile m holds component 32 m + 8 (e / 4) + 4 half + e % 4 of token
            // col: increasing in (m, e), so a strict > keeps the lowest of equal maxima
            const int half = l >> 5;
            float bv = -INFINITY;
            int bk = 0;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float xv = acc[m][e];
                    if (xv > bv) {
                        bv = xv;
                        bk = 32 * m + 8 * (e >> 2) + 4 * half + (e & 3);
                    }
                }
            const float ov = __shfl_xor(bv, 32, 64);
            const int ok = __shfl_xor(bk, 32, 64);
            if (ov > bv || (ov == bv && ok < bk)) bk = ok;
            if (half == 0 && valid && t0 < n_end) hard[(size_t)bh * N + t0 + col] = bk;
        }
        const float s = tile_exp<MT>(acc);
        const float inv = valid ? 1.0f / s : 0.0f;
        if constexpr (MODE == kRespRows) {
            // register e of tile m: component 32 m + 8 (e / 4) + 4 half + e % 4 of row t0 + col
            float* gr = reinterpret_cast<float*>(side == 0 ? GQ : GK) + ((size_t)bh * N + t0 + col) * K;
            const int half = l >> 5;
            if (valid) {
                // registers 4 q .. 4 q + 3 are 4 consecutive components: one 16-byte store when
                // K is a multiple of 4 (rows then start on 16-byte boundaries)
                const bool vec = (K & 3) == 0;
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int kc = 32 * m + 8 * q + 4 * half;
                        if (vec && kc < K) {
                            *reinterpret_cast<float4*>(gr + kc) = make_float4(
                                acc[m][4 * q] * inv, acc[m][4 * q + 1] * inv, acc[m][4 * q + 2] * inv,
                                acc[m][4 * q + 3] * inv);
                        } else {
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                if (kc + j < K) gr[kc + j] = acc[m][4 * q + j] * inv;
                        }
                    }
            }
        } else if constexpr (MODE == kRespStats) {
            const float sc = t0 < n_end ? inv : 0.0f;
            float v[16 * MT];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int e = 0; e < 16; ++e) v[16 * m + e] = acc[m][e] * sc;
            float r[UF];
            tile_token_sums<MT>(v, r);
#pragma unroll
            for (int i = 0; i < UF; ++i) us[i] += r[i];
        } else if (t0 < n_end) {
            // registers 8 sh .. 8 sh + 7 of tile m are slots 8 half + 0..7 of block 2m + sh
            bf16_t* gt = G + (size_t)(t0 / kTileT) * KS * kFrag;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                *reinterpret_cast<bf16x8*>(gt + (size_t)(2 * m) * kFrag) = pack8(acc[m], 0, inv);
                *reinterpret_cast<bf16x8*>(gt + (size_t)(2 * m + 1) * kFrag) = pack8(acc[m], 8, inv);
            }
        }
    }
    if constexpr (MODE == kRespStats) {
        // lane (half, c) holds flattened indices UF c + i (UF (c >> 1) for MT = 1, where the
        // odd lanes repeat their even neighbour): index 16 m + e is component
        // 32 m + 8 (e / 4) + 4 half + e % 4.  Per-wave sums to LDS, then over the waves.
        float* su = reinterpret_cast<float*>(smem);
        __syncthreads();  // the coefficient block is no longer read
        const int half = l >> 5;
#pragma unroll
        for (int i = 0; i < UF; ++i) {
            const int idx = MT >= 2 ? UF * col + i : (col >> 1);
            const int m = idx >> 4, e = idx & 15;
            const int k = 32 * m + 8 * (e >> 2) + 4 * half + (e & 3);
            if (MT >= 2 || (col & 1) == 0) su[w * Kp + k] = us[i];
        }
        __syncthreads();
        float* up = reinterpret_cast<float*>(GK) + ((size_t)bh * parts + part) * Kp;
        for (int k = threadIdx.x; k < Kp; k += blockDim.x) {
            float t = 0.0f;
#pragma unroll
            for (int ww = 0; ww < kRespWaves; ++ww) t += su[ww * Kp + k];
            up[k] = t;
        }
    }
}

// Component-parallel responsibilities, for a coefficient block too large for LDS (256
// components of 128 routing dims: 266 KB of split coefficients, which gma_causal_resp would
// restage from L2 in phases at every step).  Each of the eight waves owns 32 components and
// keeps their split coefficients in registers for the whole launch; the workgroup walks its
// positions in steps of kCpTiles 32-position tiles.  Per step the raw routing rows are split
// once by the whole workgroup (x and the exact x^2 = x2h + x2l) into an LDS buffer (two
// buffers: the next step's rows are loaded while the current step's products run and split
// after them), and every wave forms its components' logits of all tiles of the step (the
// same five products per 16-dim chunk as gma_causal_resp).  The softmax over all components is
// assembled from per-wave statistics: each wave's per-position maximum m_w over its components
// and the sum s_w of 2^(logit - m_w) go through LDS, and after one barrier each wave scales its
// exponentials by 2^(m_w - M) / sum_w' s_w' 2^(m_w' - M), M the maximum over the waves.  The
// output is the fragment layout of gma_causal_resp (wave w writes blocks 2w and 2w + 1), zero
// past N.
constexpr int kCpTiles = 2;
template <int NC>
struct CpLds {
    static constexpr int Dp = 16 * NC;
    static constexpr int xs = 2 * Dp + 16;                                  // bytes per staged row
    static constexpr int piece = kTileT * kCpTiles * xs;                    // x, x2h or x2l of a step
    static constexpr int buf = 3 * piece;
    static constexpr int xch = 2 * kRespWaves * kTileT * kCpTiles * 8;    // two buffers of (m, s)
    static constexpr size_t total = 2 * (size_t)buf + xch + 32 * kRespWaves * 4;
};

template <int NC>
__global__ void __launch_bounds__(64 * kRespWaves, 1)
    gma_causal_resp_cp(const bf16_t* __restrict__ qr, const bf16_t* __restrict__ kr, const bf16_t* __restrict__ W,
                       const float* __restrict__ cvec, bf16_t* __restrict__ GQ, bf16_t* __restrict__ GK,
                       int* __restrict__ hard, int BH, int H, int N, int Np, int dr, int parts, int part_len, int K) {
    extern __shared__ __align__(16) unsigned char smem[];
    using L = CpLds<NC>;
    constexpr int Kp = 32 * kRespWaves, Dp = L::Dp, KS = Kp / 16;
    constexpr int kStep = kTileT * kCpTiles;
    constexpr int kNT = 64 * kRespWaves;
    constexpr int VPR = Dp / 8;                // 16-byte vectors per staged row
    constexpr int XV = kStep * VPR / kNT;      // raw vectors per thread per step
    static_assert(XV >= 1 && kStep * VPR % kNT == 0, "step rows must split evenly over the threads");
    unsigned char* sX = smem;
    float2* sM = reinterpret_cast<float2*>(smem + 2 * L::buf);
    float* sC = reinterpret_cast<float*>(smem + 2 * L::buf + L::xch);
    int bh, part;
    head_part(blockIdx.x, BH, parts, bh, part);
    const int h = bh % H;
    const int l = lane_id(), w = wave_id(), col = l & 31, half = l >> 5;
    const int side = blockIdx.y;
    const bf16_t* x = (side == 0 ? qr : kr) + (size_t)bh * N * dr;
    bf16_t* G = (side == 0 ? GQ : GK) + (size_t)bh * Np * Kp + 8 * l;
    const int n_begin = part * part_len;
    const int n_end = min(Np, n_begin + part_len);
    if (n_begin >= n_end) return;  // uniform over the workgroup

    // this wave's coefficient fragments: component 32 w + col, dims 16 c + 8 half .. + 7
    bf16x8 ca[NC], cal[NC], cb[NC], cbl[NC];
    {
        const bf16_t* wr = W + ((size_t)h * Kp + 32 * w + col) * 4 * Dp + 8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            ca[c] = *reinterpret_cast<const bf16x8*>(wr + 16 * c);
            cal[c] = *reinterpret_cast<const bf16x8*>(wr + Dp + 16 * c);
            cb[c] = *reinterpret_cast<const bf16x8*>(wr + 2 * Dp + 16 * c);
            cbl[c] = *reinterpret_cast<const bf16x8*>(wr + 3 * Dp + 16 * c);
        }
    }
    for (int i = threadIdx.x; i < Kp; i += kNT) sC[i] = cvec[(size_t)h * Kp + i];

    // raw rows of a step: vector v = thread + kNT u is position v / VPR, dims 8 (v % VPR);
    // positions past the sequence read its last row (their responsibilities are zeroed)
    bf16x8 xraw[XV];
    auto load_raw = [&](int b0) {
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const int v = threadIdx.x + kNT * u;
            const int t = min(b0 + v / VPR, N - 1), d0 = 8 * (v % VPR);
            bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
            if (d0 < dr) z = *reinterpret_cast<const bf16x8*>(x + (size_t)t * dr + d0);
            xraw[u] = z;
        }
    };
    auto store_split = [&](int b) {
        unsigned char* base = sX + (size_t)b * L::buf;
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const int v = threadIdx.x + kNT * u;
            const int off = (v / VPR) * L::xs + 16 * (v % VPR);
            XFrag f;
            f.x1 = xraw[u];
            split_square(f);
            *reinterpret_cast<bf16x8*>(base + off) = f.x1;
            *reinterpret_cast<bf16x8*>(base + L::piece + off) = f.x2h;
            *reinterpret_cast<bf16x8*>(base + 2 * L::piece + off) = f.x2l;
        }
    };
    load_raw(n_begin);
    store_split(0);
    __syncthreads();

    int it = 0;
    for (int b0 = n_begin; b0 < n_end; b0 += kStep, ++it) {
        const int b = it & 1;
        const bool more = b0 + kStep < n_end;
        if (more) load_raw(b0 + kStep);
        // register i of acc[j]: component 32 w + 8 (i / 4) + 4 half + i % 4, position 32 j + col
        f32x16 acc[kCpTiles];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 cq = *reinterpret_cast<const float4*>(sC + 32 * w + 8 * q + 4 * half);
#pragma unroll
            for (int j = 0; j < kCpTiles; ++j) {
                acc[j][4 * q] = cq.x;
                acc[j][4 * q + 1] = cq.y;
                acc[j][4 * q + 2] = cq.z;
                acc[j][4 * q + 3] = cq.w;
            }
        }
        const unsigned char* xb = sX + (size_t)b * L::buf + (size_t)col * L::xs + 16 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            bf16x8 p1[kCpTiles], p2h[kCpTiles], p2l[kCpTiles];
#pragma unroll
            for (int j = 0; j < kCpTiles; ++j) {
                const unsigned char* pj = xb + (size_t)kTileT * j * L::xs + 32 * c;
                p1[j] = *reinterpret_cast<const bf16x8*>(pj);
                p2h[j] = *reinterpret_cast<const bf16x8*>(pj + L::piece);
                p2l[j] = *reinterpret_cast<const bf16x8*>(pj + 2 * L::piece);
            }
#pragma unroll
            for (int j = 0; j < kCpTiles; ++j) acc[j] = mfma(ca[c], p2h[j], acc[j]);
#pragma unroll
            for (int j = 0; j < kCpTiles; ++j) acc[j] = mfma(cb[c], p1[j], acc[j]);
#pragma unroll
            for (int j = 0; j < kCpTiles; ++j) acc[j] = mfma(cal[c], p2h[j], acc[j]);
#pragma unroll
            for (int j = 0; j < kCpTiles; ++j) acc[j] = mfma(cbl[c], p1[j], acc[j]);
#pragma unroll
            for (int j = 0; j < kCpTiles; ++j) acc[j] = mfma(ca[c], p2l[j], acc[j]);
        }
        // per-wave statistics of every position of the step
        float mloc[kCpTiles];
#pragma unroll
        for (int j = 0; j < kCpTiles; ++j) {
            float m0 = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) m0 = fmaxf(m0, acc[j][i]);
            // a wave whose components are all padding (logits -inf) keeps a finite maximum, so
            // its exponentials and sum are 0 rather than 2^(-inf + inf)
            m0 = fmaxf(max_halves(m0), -__FLT_MAX__);
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float e = fast_exp2(acc[j][i] - m0);
                acc[j][i] = e;
                s += e;
            }
            s = sum_halves(s);
            mloc[j] = m0;
            if (half == 0) sM[(b * kRespWaves + w) * kStep + kTileT * j + col] = make_float2(m0, s);
        }
        if (more) store_split(b ^ 1);  // the buffer read one step ago: every wave is past that
        lds_barrier();
#pragma unroll
        for (int j = 0; j < kCpTiles; ++j) {
            const int t0 = b0 + kTileT * j;
            // lanes l and l + 32 hold the same position: each half takes four waves' terms,
            // then the halves exchange (maximum, then the two partial sums in half order)
            constexpr int WH = kRespWaves / 2;
            float2 st[WH];
            float M = -INFINITY;
#pragma unroll
            for (int u = 0; u < WH; ++u) {
                st[u] = sM[(b * kRespWaves + WH * half + u) * kStep + kTileT * j + col];
                M = fmaxf(M, st[u].x);
            }
            M = max_halves(M);
            float S = 0.0f;
#pragma unroll
            for (int u = 0; u < WH; ++u) S += st[u].y * fast_exp2(st[u].x - M);
            S = sum_halves(S);
            // S >= 1 (the wave holding the maximum contributes at least 2^0)
            const float inv = t0 + col < N ? fast_exp2(mloc[j] - M) * __builtin_amdgcn_rcpf(S) : 0.0f;
            if (t0 < n_end) {
                bf16_t* gt = G + (size_t)(t0 / kTileT) * KS * kFrag;
                *reinterpret_cast<bf16x8*>(gt + (size_t)(2 * w) * kFrag) = pack8(acc[j], 0, inv);
                *reinterpret_cast<bf16x8*>(gt + (size_t)(2 * w + 1) * kFrag) = pack8(acc[j], 8, inv);
            }
        }
    }
}

// ----------------------------------------------------------------------------- group staging
// Register prefetch of one group: this thread's share of the Gamma_K fragments (the group's
// four tiles are one contiguous block of 16 Kp 16-byte chunks; thread i takes chunks
// i + 256 u) and of the value slice rows (chunk c = row c / PPR, 8 dims at 8 (c % PPR)).
template <int MT, int NTS>
struct GroupRegs {
    static constexpr int KS = 2 * MT;    // 16-wide component blocks
    static constexpr int Dvs = 32 * NTS;
    static constexpr int PPR = Dvs / 8;  // 16-byte pieces per value row
    static constexpr int VU = kGroup * PPR / kThreads;
    bf16x8 g[KS];
    bf16x8 v[VU];

    __device__ __forceinline__ void load_g(int u, const bf16_t* gk_group) {
        g[u] = *reinterpret_cast<const bf16x8*>(gk_group + 8 * ((size_t)threadIdx.x + kThreads * u));
    }
    // rows past n_end read a valid row: positions there have zero Gamma_K (past the sequence)
    // or are masked out of every output that could see them
    __device__ __forceinline__ void load_v(int u, const bf16_t* v_h, int base, int n_end, int dv, int dv0) {
        const int c = threadIdx.x + kThreads * u;
        const int t = min(base + c / PPR, n_end - 1), d0 = dv0 + 8 * (c % PPR);
        bf16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
        if (d0 < dv) x = *reinterpret_cast<const bf16x8*>(v_h + (size_t)t * dv + d0);
        v[u] = x;
    }
    __device__ __forceinline__ void load(const bf16_t* gk_group, const bf16_t* v_h, int base, int n_end, int dv,
                                         int dv0) {
#pragma unroll
        for (int u = 0; u < KS; ++u) load_g(u, gk_group);
#pragma unroll
        for (int u = 0; u < VU; ++u) load_v(u, v_h, base, n_end, dv, dv0);
    }
    // The share of step s (of 8) of the loads above: indices u with u % 8 == s.
    __device__ __forceinline__ void load_step(int s, const bf16_t* gk_group, const bf16_t* v_h, int base, int n_end,
                                              int dv, int dv0) {
#pragma unroll
        for (int u = s; u < KS; u += 8) load_g(u, gk_group);
#pragma unroll
        for (int u = s; u < VU; u += 8) load_v(u, v_h, base, n_end, dv, dv0);
    }
    // sG: row j = position j of the group, column = slot (Kp bf16, stride gs bytes);
    // sV: row j = position, columns = the slice's value dims (stride vs bytes).
    __device__ __forceinline__ void store(unsigned char* sG, int gs, unsigned char* sV, int vs) const {
        const int l = lane_id(), w = wave_id();
#pragma unroll
        for (int u = 0; u < KS; ++u) {
            const int blk = kWaves * u + w;  // = chunk / 64
            const int tile = blk / KS, ks = blk % KS;
            *reinterpret_cast<bf16x8*>(sG + (size_t)(kTileT * tile + (l & 31)) * gs + 2 * (16 * ks + 8 * (l >> 5))) =
                g[u];
        }
#pragma unroll
        for (int u = 0; u < VU; ++u) {
            const int c = threadIdx.x + kThreads * u;
            *reinterpret_cast<bf16x8*>(sV + (size_t)(c / PPR) * vs + 16 * (c % PPR)) = v[u];
        }
    }
};

// ----------------------------------------------------------------------------- totals
// [S | z] contribution Gamma_K^T [V | 1] of one sub-segment and one value slice, written as
// fp32 rows k (slot order) of Dvs + 1 columns (the value dims, then z).
template <int MT, int NTS>
__global__ void __launch_bounds__(kThreads, 1)
    gma_causal_totals(const bf16_t* __restrict__ GK, const bf16_t* __restrict__ v, float* __restrict__ tpart, int BH,
                      int N, int Np, int dv, int NS, int nsub, int sub_len) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int Kp = 32 * MT, Dvs = 32 * NTS;
    constexpr int gs = 2 * Kp + 32, vs = 2 * Dvs + 32;
    using UT = UpdateTiles<MT, NTS>;
    using GR = GroupRegs<MT, NTS>;
    unsigned char* sG = smem;
    unsigned char* sV = smem + (size_t)kGroup * gs;
    int bh, sub;
    head_part(blockIdx.x, BH, nsub, bh, sub);
    const int y = blockIdx.y, dv0 = Dvs * y;
    const int l = lane_id(), w = wave_id(), half = l >> 5, col = l & 31;
    const int n_begin = sub * sub_len, n_end = min(N, n_begin + sub_len);
    const bf16_t* gk_h = GK + (size_t)bh * Np * Kp;
    const bf16_t* v_h = v + (size_t)bh * N * dv;

    f32x16 acc[UT::MW][UT::NW];
#pragma unroll
    for (int i = 0; i < UT::MW; ++i)
#pragma unroll
        for (int j = 0; j < UT::NW; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (short)0x3f80;

    // the next group's loads are issued between the MFMAs of the current group's update
    GR r;
    r.load(gk_h + (size_t)n_begin * Kp, v_h, n_begin, n_end, dv, dv0);
    for (int base = n_begin; base < n_end; base += kGroup) {
        r.store(sG, gs, sV, vs);
        lds_barrier();
        const int nb = base + kGroup;
        const bool more = nb < n_end;
        const bf16_t* gnext = gk_h + (size_t)nb * Kp;
        update_from_lds<MT, NTS, UT::MW, UT::NW>(acc, sG, gs, sV, vs, ones, [&](int s8) {
            if (more) r.load_step(s8, gnext, v_h, nb, n_end, dv, dv0);
        });
        lds_barrier();
    }

    float* T = tpart + ((size_t)(bh * nsub + sub) * NS + y) * Kp * (Dvs + 1);
#pragma unroll
    for (int i = 0; i < UT::MW; ++i)
#pragma unroll
        for (int j = 0; j < UT::NW; ++j) {
            const int m = UT::m_of(w, i), n = UT::n_of(w, j);
            if (n > NTS) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int k = 32 * m + 8 * (e >> 2) + 4 * half + (e & 3);
                if (n < NTS)
                    T[(size_t)k * (Dvs + 1) + 32 * n + col] = acc[i][j][e];
                else if (col == 0)
                    T[(size_t)k * (Dvs + 1) + Dvs] = acc[i][j][e];
            }
        }
}

// ----------------------------------------------------------------------------- scan
// Shadow (bf16, LDS) of the state, rows: S^T (Dvs rows, value dims of the slice), then z hi
// (8 rows), z lo (8 rows) and 16 rows of ones; columns = slots.  Written from this wave's
// accumulator tiles.
template <int MT, int NTS, int MW, int NW>
__device__ __forceinline__ void write_shadow(unsigned char* sS, int ss, const f32x16 (&acc)[MW][NW]) {
    using UT = UpdateTiles<MT, NTS>;
    constexpr int Dvs = 32 * NTS;
    const int l = lane_id(), w = wave_id(), half = l >> 5, col = l & 31;
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            const int m = UT::m_of(w, i), n = UT::n_of(w, j);
            if (n > NTS) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k0 = 32 * m + 8 * q + 4 * half;
                const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1], v2 = acc[i][j][4 * q + 2],
                            v3 = acc[i][j][4 * q + 3];
                if (n < NTS) {
                    uint2 p;
                    p.x = pack_bf16(v0, v1);
                    p.y = pack_bf16(v2, v3);
                    *reinterpret_cast<uint2*>(sS + (size_t)(32 * n + col) * ss + 2 * k0) = p;
                } else if (col < 16) {
                    // z: rows Dvs..Dvs+7 hi part, Dvs+8..Dvs+15 lo part
                    uint2 hi, lo;
                    hi.x = pack_bf16(v0, v1);
                    hi.y = pack_bf16(v2, v3);
                    lo.x = pack_bf16(v0 - bf16lo_to_f32(hi.x), v1 - bf16hi_to_f32(hi.x));
                    lo.y = pack_bf16(v2 - bf16lo_to_f32(hi.y), v3 - bf16hi_to_f32(hi.y));
                    *reinterpret_cast<uint2*>(sS + (size_t)(Dvs + col) * ss + 2 * k0) = col < 8 ? hi : lo;
                }
            }
        }
}

template <int MT, int NTS>
__global__ void __launch_bounds__(kThreads, 1)
    gma_causal_scan(const bf16_t* __restrict__ GQ, const bf16_t* __restrict__ GK, const bf16_t* __restrict__ v,
                    const float* __restrict__ tpart, bf16_t* __restrict__ out, float eps, int BH, int N, int Np,
                    int dv, int S, int NS, int seg_len, int TS) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int Kp = 32 * MT, Dvs = 32 * NTS;
    constexpr int gs = 2 * Kp + 32, vs = 2 * Dvs + 32, ss = 2 * Kp + 16;
    constexpr int KS = Kp / 16;  // 16-wide contraction steps over the components
    using UT = UpdateTiles<MT, NTS>;
    using GR = GroupRegs<MT, NTS>;
    unsigned char* sG = smem;
    unsigned char* sV = sG + (size_t)kGroup * gs;
    unsigned char* sS = sV + (size_t)kGroup * vs;

    int bh, seg;
    head_part(blockIdx.x, BH, S, bh, seg);
    const int y = blockIdx.y, dv0 = Dvs * y;
    const int l = lane_id(), w = wave_id(), half = l >> 5, col = l & 31;
    const int n_begin = seg * seg_len, n_end = min(N, n_begin + seg_len);

    // state entering this segment (fp32, this wave's output tiles): the totals of the
    // sub-segments before it, added in sub-segment order (a fixed order: every run gives the
    // same bits); segment 0 starts from zero
    f32x16 st[UT::MW][UT::NW];
#pragma unroll
    for (int i = 0; i < UT::MW; ++i)
#pragma unroll
        for (int j = 0; j < UT::NW; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) st[i][j][e] = 0.0f;
    {
        const int nsub = (S - 1) * TS, nprev = seg * TS;
        const size_t per = (size_t)Kp * (Dvs + 1);
        const float* src = tpart + ((size_t)bh * nsub * NS + y) * per;
        for (int u0 = 0; u0 < nprev; u0 += 2) {
            float x0[UT::MW][UT::NW][16], x1[UT::MW][UT::NW][16];
            const bool ok1 = u0 + 1 < nprev;
            const float* p0 = src + (size_t)u0 * NS * per;
            const float* p1 = src + (size_t)(ok1 ? u0 + 1 : u0) * NS * per;
#pragma unroll
            for (int i = 0; i < UT::MW; ++i)
#pragma unroll
                for (int j = 0; j < UT::NW; ++j) {
                    const int m = UT::m_of(w, i), n = UT::n_of(w, j);
                    const int cc = n < NTS ? 32 * n + col : Dvs;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const size_t off = (size_t)(32 * m + 8 * (e >> 2) + 4 * half + (e & 3)) * (Dvs + 1) + cc;
                        x0[i][j][e] = p0[off];
                        x1[i][j][e] = p1[off];
                    }
                }
#pragma unroll
            for (int i = 0; i < UT::MW; ++i)
#pragma unroll
                for (int j = 0; j < UT::NW; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        st[i][j][e] += x0[i][j][e];
                        if (ok1) st[i][j][e] += x1[i][j][e];
                    }
        }
#pragma unroll
        for (int i = 0; i < UT::MW; ++i)
#pragma unroll
            for (int j = 0; j < UT::NW; ++j)
                if (UT::n_of(w, j) > NTS)
#pragma unroll
                    for (int e = 0; e < 16; ++e) st[i][j][e] = 0.0f;
    }
    // constant rows of the shadow: ones (den tile rows 16..31)
    for (int i = threadIdx.x; i < 2 * Kp; i += blockDim.x) {
        bf16x8 o8;
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] = (short)0x3f80;
        *reinterpret_cast<bf16x8*>(sS + (size_t)(Dvs + 16 + i / (Kp / 8)) * ss + 16 * (i % (Kp / 8))) = o8;
    }
    write_shadow<MT, NTS, UT::MW, UT::NW>(sS, ss, st);

    const bf16_t* gq_h = GQ + (size_t)bh * Np * Kp + 8 * l;
    const bf16_t* gk_h = GK + (size_t)bh * Np * Kp;
    const bf16_t* v_h = v + (size_t)bh * N * dv;
    bf16_t* o_h = out + (size_t)bh * N * dv;
    bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (short)0x3f80;
    // den-tile operand for the intra term: ones in rows 0..7 (they add to the z-hi rows)
    bf16x8 den_ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) den_ones[j] = (short)(col < 8 ? 0x3f80 : 0);

    // Group prefetch into registers: Gamma_K and V rows (stored to LDS at the top of the
    // group) and this wave's Gamma_Q fragments, all loaded during the previous group's state
    // update (qf is dead from the end of the intra term on).
    GR r;
    bf16x8 qf[KS];
    r.load(gk_h + (size_t)n_begin * Kp, v_h, n_begin, n_end, dv, dv0);
    {
        const bf16_t* src = gq_h + (size_t)(n_begin / kTileT + w) * KS * kFrag;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + (size_t)ks * kFrag);
    }

    for (int base = n_begin; base < n_end; base += kGroup) {
        r.store(sG, gs, sV, vs);
        lds_barrier();
        // ---- outputs of chunk w: positions base + 32w + col
        {
            const int t = base + kTileT * w + col;
            f32x16 o[NTS + 1];
#pragma unroll
            for (int n = 0; n <= NTS; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[n][i] = 0.0f;
            // inter-group: Gamma_Q [S | z] from the shadow (A fragments read one step ahead)
            {
                constexpr int NI = KS * (NTS + 1);
                const unsigned char* srow = sS + (size_t)col * ss + 16 * half;
                bf16x8 an = *reinterpret_cast<const bf16x8*>(srow);
#pragma unroll
                for (int idx = 0; idx < NI; ++idx) {
                    const int ks = idx / (NTS + 1), n = idx % (NTS + 1);
                    const bf16x8 a = an;
                    if (idx + 1 < NI) {
                        const int ks2 = (idx + 1) / (NTS + 1), n2 = (idx + 1) % (NTS + 1);
                        an = *reinterpret_cast<const bf16x8*>(srow + (size_t)32 * n2 * ss + 32 * ks2);
                    }
                    o[n] = mfma(a, qf[ks], o[n]);
                }
            }
            // intra-group: chunks c <= w; A[j', i] = gamma_K,j' . gamma_Q,i, zero for j' > i
            for (int c = 0; c <= w; ++c) {
                f32x16 aff;
#pragma unroll
                for (int i = 0; i < 16; ++i) aff[i] = 0.0f;
                const unsigned char* grow = sG + (size_t)(kTileT * c + col) * gs + 16 * half;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    aff = mfma(*reinterpret_cast<const bf16x8*>(grow + 32 * ks), qf[ks], aff);
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
                    for (int n = 0; n < NTS; ++n)
                        o[n] = mfma(lds_frag_tr_crows(sV, vs, kTileT * c + 16 * sh, 32 * n), b, o[n]);
                    o[NTS] = mfma(den_ones, b, o[NTS]);
                }
            }
            const float den = o[NTS][0] + o[NTS][4];
            const float inv = 1.0f / (den + eps);
            // register group q of o[n] holds dims 32 n + 8 q + 4 half + 0..3 of this lane's
            // position; one swap per group pair gives each lane 8 contiguous dims (one 16-byte
            // store): the lower half takes group 2 qp of both halves, the upper half 2 qp + 1
            bf16_t* orow = o_h + (size_t)t * dv;
#pragma unroll
            for (int n = 0; n < NTS; ++n)
#pragma unroll
                for (int qp = 0; qp < 2; ++qp) {
                    uint2 p0, p1;
                    p0.x = pack_bf16(o[n][8 * qp] * inv, o[n][8 * qp + 1] * inv);
                    p0.y = pack_bf16(o[n][8 * qp + 2] * inv, o[n][8 * qp + 3] * inv);
                    p1.x = pack_bf16(o[n][8 * qp + 4] * inv, o[n][8 * qp + 5] * inv);
                    p1.y = pack_bf16(o[n][8 * qp + 6] * inv, o[n][8 * qp + 7] * inv);
                    auto sx = __builtin_amdgcn_permlane32_swap(p0.x, p1.x, false, false);
                    auto sy = __builtin_amdgcn_permlane32_swap(p0.y, p1.y, false, false);
                    const int d0 = dv0 + 32 * n + 16 * qp + 8 * half;
                    if (t < n_end && d0 < dv)
                        *reinterpret_cast<uint4*>(orow + d0) = make_uint4(sx[0], sy[0], sx[1], sy[1]);
                }
        }
        // ---- state += Gamma_K^T [V | 1] over the group (this wave's tiles); the next group's
        // loads go out between its MFMAs
        const int nb = base + kGroup;
        const bool more = nb < n_end;
        const bf16_t* gnext = gk_h + (size_t)nb * Kp;
        const bf16_t* qnext = gq_h + (size_t)(nb / kTileT + w) * KS * kFrag;
        update_from_lds<MT, NTS, UT::MW, UT::NW>(st, sG, gs, sV, vs, ones, [&](int s8) {
            if (more) {
                r.load_step(s8, gnext, v_h, nb, n_end, dv, dv0);
#pragma unroll
                for (int ks = s8; ks < KS; ks += 8) qf[ks] = *reinterpret_cast<const bf16x8*>(qnext + (size_t)ks * kFrag);
            }
        });
        lds_barrier();  // every wave is done reading sG, sV and the old shadow
        write_shadow<MT, NTS, UT::MW, UT::NW>(sS, ss, st);
    }
}

// ----------------------------------------------------------------------------- dispatch
typedef void (*RespFn)(const bf16_t*, const bf16_t*, const bf16_t*, const float*, bf16_t*, bf16_t*, int*, int, int, int,
                       int, int, int, int, int);
typedef void (*TotFn)(const bf16_t*, const bf16_t*, float*, int, int, int, int, int, int, int);
typedef void (*ScanFn)(const bf16_t*, const bf16_t*, const bf16_t*, const float*, bf16_t*, float, int, int, int, int,
                       int, int, int, int);

template <int MT, int NC, int MODE>
RespFn resp_fn(int nph) {
    if (nph == 1) return gma_causal_resp<MT, NC, 1, MODE>;
    if (nph == 2 && NC % 2 == 0) return gma_causal_resp<MT, NC, (NC % 2 == 0 ? 2 : 1), MODE>;
    if (nph == 4 && NC % 4 == 0) return gma_causal_resp<MT, NC, (NC % 4 == 0 ? 4 : 1), MODE>;
    return nullptr;
}
template <int MT, int MODE>
RespFn resp_fn_nc(int NC, int nph) {
    switch (NC) {
        case 1: return resp_fn<MT, 1, MODE>(nph);
        case 2: return resp_fn<MT, 2, MODE>(nph);
        case 4: return resp_fn<MT, 4, MODE>(nph);
        case 8: return resp_fn<MT, 8, MODE>(nph);
    }
    return nullptr;
}
template <int MODE>
RespFn select_resp_t(const Geo& g, int nph) {
    switch (g.MT) {
        case 1: return resp_fn_nc<1, MODE>(g.NC, nph);
        case 2: return resp_fn_nc<2, MODE>(g.NC, nph);
        case 4: return resp_fn_nc<4, MODE>(g.NC, nph);
        case 8: return resp_fn_nc<8, MODE>(g.NC, nph);
    }
    return nullptr;
}
// Component-parallel form: eight 32-component tiles whose coefficients (in registers) would
// otherwise be restaged in phases.
bool resp_cp(const Geo& g, int nph, int mode) { return mode == kRespFrag && nph > 1 && g.MT == 8 && g.NC == 8; }
RespFn select_resp(const Geo& g, int nph, int mode = kRespFrag) {
    if (mode == kRespStats) return select_resp_t<kRespStats>(g, nph);
    if (mode == kRespRows) return select_resp_t<kRespRows>(g, nph);
    if (resp_cp(g, nph, mode)) return gma_causal_resp_cp<8>;
    return select_resp_t<kRespFrag>(g, nph);
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
bool select_scan_nt(int NTS, TotFn& tf, ScanFn& sf) {
    switch (NTS) {
        case 1: tf = gma_causal_totals<MT, 1>; sf = gma_causal_scan<MT, 1>; return true;
        case 2: tf = gma_causal_totals<MT, 2>; sf = gma_causal_scan<MT, 2>; return true;
    }
    return false;
}
bool select_scan(const Geo& g, int NTS, TotFn& tf, ScanFn& sf) {
    switch (g.MT) {
        case 1: return select_scan_nt<1>(NTS, tf, sf);
        case 2: return select_scan_nt<2>(NTS, tf, sf);
        case 4: return select_scan_nt<4>(NTS, tf, sf);
        case 8: return select_scan_nt<8>(NTS, tf, sf);
    }
    return false;
}

hipError_t set_lds(const void* f, size_t bytes) {
    return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

// Position parts per (b, h) of the responsibilities kernel: about one workgroup per CU over
// all (b, h), each part a multiple of the workgroup's 256-position step.
int resp_parts(int BH, int Np, int* part_len) {
    const int rstep = kTileT * kRespWaves;
    int parts = (256 + BH - 1) / BH;
    const int max_parts = (Np + rstep - 1) / rstep;
    if (parts > max_parts) parts = max_parts;
    if (parts < 1) parts = 1;
    const int len = ((Np + parts - 1) / parts + rstep - 1) / rstep * rstep;
    if (part_len) *part_len = len;
    return (Np + len - 1) / len;
}

namespace {

// Responsibilities of `sides` sides (2: Gamma_Q into GQ and Gamma_K into GK; 1: Gamma_K
// only, into GK), about one workgroup per CU per side.
hipError_t launch_resp(const Args& a, const Geo& g, RespFn rf, int nph, int Np, int sides, const bf16_t* W,
                       const float* cvec, bf16_t* GQ, bf16_t* GK, int* hard = nullptr) {
    const gma_desc& d = a.d;
    const int BH = d.B * d.H;
    int part_len = 0;
    const int parts = resp_parts(BH, Np, &part_len);
    const bool cp = rf == static_cast<RespFn>(gma_causal_resp_cp<8>);
    const size_t rl = cp ? CpLds<8>::total : resp_lds(g, nph);
    hipError_t e;
    if ((e = set_lds(reinterpret_cast<const void*>(rf), rl)) != hipSuccess) return e;
    const bf16_t* kr = static_cast<const bf16_t*>(a.kr);
    const bf16_t* qr = sides == 2 ? static_cast<const bf16_t*>(a.qr) : kr;
    rec_begin(a, "gma_causal_resp");
    hipLaunchKernelGGL(rf, dim3(BH * parts, sides), dim3(64 * kRespWaves), rl, a.stream, qr, kr, W, cvec,
                       sides == 2 ? GQ : GK, GK, hard, BH, d.H, d.N, Np, d.d_r, parts, part_len, d.K);
    rec_end(a);
    return hipGetLastError();
}

// Ordered sum over the nsub sub-segment totals of each head into the causal memory
// [B,H,K,d_v+1] (natural component order; totals rows are slots, slot kperm(k) holds k).
__global__ void __launch_bounds__(256)
    gma_causal_memory_reduce(const float* __restrict__ tpart, float* __restrict__ state, int BH, int nsub, int NS,
                             int K, int Kp, int dv, int Dvs) {
    const int W = dv + 1;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= K * W) return;
    const int k = i / W, c = i % W;
    const int y = c < dv ? c / Dvs : 0, col = c < dv ? c % Dvs : Dvs;
    const size_t tile = (size_t)Kp * (Dvs + 1);
    for (size_t bh = blockIdx.y; bh < (size_t)BH; bh += gridDim.y) {
        const float* p = tpart + (bh * nsub * NS + y) * tile + (size_t)kperm(k) * (Dvs + 1) + col;
        float acc = 0.0f;
        for (int s = 0; s < nsub; ++s) acc += p[(size_t)s * NS * tile];
        state[bh * K * W + i] = acc;
    }
}

}  // namespace

bool causal_supported(const gma_desc& d) {
    if (fused_causal_supported(d)) return true;
    const Geo g = geometry(d);
    const int Dvs = g.Dvp < kSliceV ? g.Dvp : kSliceV;
    return scan_lds_bytes(g, Dvs) <= kLdsMax && resp_phases(g) > 0;
}

size_t causal_workspace(const gma_desc& d) {
    return fused_causal_supported(d) ? fused_causal_workspace(d) : causal_layout(d).total;
}

// The fused kernels where they apply (responsibilities on chip); otherwise responsibilities
// to the workspace, segment totals, then the scan.
hipError_t causal_forward(const Args& a) {
    if (fused_causal_supported(a.d)) return fused_causal_forward(a);
    const gma_desc& d = a.d;
    const Geo g = geometry(d);
    const CausalLayout L = causal_layout(d);
    bf16_t* W = reinterpret_cast<bf16_t*>(a.ws + L.W);
    float* cvec = reinterpret_cast<float*>(a.ws + L.C);
    bf16_t* GQ = reinterpret_cast<bf16_t*>(a.ws + L.gq);
    bf16_t* GK = reinterpret_cast<bf16_t*>(a.ws + L.gk);
    float* tpart = reinterpret_cast<float*>(a.ws + L.tpart);
    const int BH = d.B * d.H;
    const int NTS = L.Dvs / 32;
    hipError_t e;

    const int nph = resp_phases(g);
    RespFn rf = nph ? select_resp(g, nph) : nullptr;
    TotFn tf;
    ScanFn sf;
    if (!rf || !select_scan(g, NTS, tf, sf)) return hipErrorNotSupported;

    if ((e = launch_prep(a, g, W, cvec)) != hipSuccess) return e;

    if ((e = launch_resp(a, g, rf, nph, L.Np, 2, W, cvec, GQ, GK)) != hipSuccess) return e;

    if (L.S > 1) {
        const size_t tl = totals_lds_bytes(g, L.Dvs);
        if ((e = set_lds(reinterpret_cast<const void*>(tf), tl)) != hipSuccess) return e;
        rec_begin(a, "gma_causal_totals");
        hipLaunchKernelGGL(tf, dim3(BH * L.nsub, L.NS), dim3(kThreads), tl, a.stream, GK,
                           static_cast<const bf16_t*>(a.v), tpart, BH, d.N, L.Np, d.d_v, L.NS, L.nsub, L.sub_len);
        rec_end(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    const size_t sl = scan_lds_bytes(g, L.Dvs);
    if ((e = set_lds(reinterpret_cast<const void*>(sf), sl)) != hipSuccess) return e;
    rec_begin(a, "gma_causal_scan");
    hipLaunchKernelGGL(sf, dim3(BH * L.S, L.NS), dim3(kThreads), sl, a.stream, GQ, GK, static_cast<const bf16_t*>(a.v),
                       tpart, static_cast<bf16_t*>(a.out), a.eps, BH, d.N, L.Np, d.d_v, L.S, L.NS, L.seg_len, L.TS);
    rec_end(a);
    return hipGetLastError();
}

// Causal memory (prefill) on the causal kernels: Gamma_K of every position (the
// responsibilities kernel on the key side only), Gamma_K^T [V | 1] of nsub sub-segments
// (the totals kernel over the whole sequence), then their ordered sum into the state.
// Used where the fused write kernel of the bidirectional path does not fit in LDS.
struct MemoryLayout {
    size_t W, C, gk, tpart, total;
    int Np, NS, Dvs, nsub, sub_len;
};

static MemoryLayout memory_layout(const gma_desc& d) {
    const Geo g = geometry(d);
    const int BH = d.B * d.H;
    MemoryLayout L;
    L.Dvs = g.Dvp < kSliceV ? g.Dvp : kSliceV;
    L.NS = g.Dvp / L.Dvs;
    const int groups = (d.N + kGroup - 1) / kGroup;
    L.Np = groups * kGroup;
    int s = (256 + BH * L.NS - 1) / (BH * L.NS);
    if (s > groups) s = groups;
    if (s < 1) s = 1;
    L.sub_len = ((d.N + s - 1) / s + kGroup - 1) / kGroup * kGroup;
    L.nsub = d.N > 0 ? (d.N + L.sub_len - 1) / L.sub_len : 0;
    size_t off = 0;
    L.W = off;
    off += align_up((size_t)d.H * g.Kp * 4 * g.Dp * sizeof(bf16_t));
    L.C = off;
    off += align_up((size_t)d.H * g.Kp * sizeof(float));
    L.gk = off;
    off += align_up((size_t)BH * L.Np * g.Kp * sizeof(bf16_t));
    L.tpart = off;
    off += align_up((size_t)BH * L.nsub * L.NS * g.Kp * (L.Dvs + 1) * sizeof(float));
    L.total = off;
    return L;
}

size_t causal_memory_workspace(const gma_desc& d) { return memory_layout(d).total; }

hipError_t causal_memory(const Args& a) {
    const gma_desc& d = a.d;
    const Geo g = geometry(d);
    const MemoryLayout L = memory_layout(d);
    bf16_t* W = reinterpret_cast<bf16_t*>(a.ws + L.W);
    float* cvec = reinterpret_cast<float*>(a.ws + L.C);
    bf16_t* GK = reinterpret_cast<bf16_t*>(a.ws + L.gk);
    float* tpart = reinterpret_cast<float*>(a.ws + L.tpart);
    const int BH = d.B * d.H;
    const int NTS = L.Dvs / 32;
    hipError_t e;
    const int nph = resp_phases(g);
    RespFn rf = nph ? select_resp(g, nph) : nullptr;
    TotFn tf;
    ScanFn sf;
    if (!rf || !select_scan(g, NTS, tf, sf)) return hipErrorNotSupported;
    if (L.nsub > 0) {
        if ((e = launch_prep(a, g, W, cvec)) != hipSuccess) return e;
        if ((e = launch_resp(a, g, rf, nph, L.Np, 1, W, cvec, nullptr, GK)) != hipSuccess) return e;
        const size_t tl = totals_lds_bytes(g, L.Dvs);
        if ((e = set_lds(reinterpret_cast<const void*>(tf), tl)) != hipSuccess) return e;
        rec_begin(a, "gma_causal_totals");
        hipLaunchKernelGGL(tf, dim3(BH * L.nsub, L.NS), dim3(kThreads), tl, a.stream, GK,
                           static_cast<const bf16_t*>(a.v), tpart, BH, d.N, L.Np, d.d_v, L.NS, L.nsub, L.sub_len);
        rec_end(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int per = d.K * (d.d_v + 1);
    rec_begin(a, "gma_causal_memory_reduce");
    gma_causal_memory_reduce<<<dim3((unsigned)((per + 255) / 256), (unsigned)(BH < 65535 ? BH : 65535)), dim3(256),
                               0, a.stream>>>(tpart, a.state, BH, L.nsub, L.NS, d.K, g.Kp, d.d_v, L.Dvs);
    rec_end(a);
    return hipGetLastError();
}

// Responsibility statistics on the matrix cores: the hard assignment of every row of a.kr
// into hard [B H][N] and the soft usage partials of every (b h, part) workgroup into
// upart [B H parts][Kp] (parts = resp_parts(B H, Np)); coefficients into W, cvec.  Np = N
// rounded up to 128.
bool stats_supported(const gma_desc& d) {
    if (d.dtype != GMA_BF16 || d.d_r % 8 != 0) return false;
    return resp_phases(geometry(d)) > 0;
}

int stats_np(const gma_desc& d) { return (d.N + kGroup - 1) / kGroup * kGroup; }

hipError_t stats_resp(const Args& a, bf16_t* W, float* cvec, float* upart, int* hard) {
    const gma_desc& d = a.d;
    const Geo g = geometry(d);
    const int nph = resp_phases(g);
    RespFn rf = nph ? select_resp(g, nph, kRespStats) : nullptr;
    if (!rf) return hipErrorNotSupported;
    hipError_t e;
    if ((e = launch_prep(a, g, W, cvec)) != hipSuccess) return e;
    return launch_resp(a, g, rf, nph, stats_np(d), 1, W, cvec, nullptr, reinterpret_cast<bf16_t*>(upart), hard);
}

// Responsibilities of both sides as float32 rows [2][B H][N][K] (queries, then keys) for
// the backward of bf16 inputs: logits on the matrix cores (coefficients into W, cvec).
hipError_t resp_rows(const Args& a, bf16_t* W, float* cvec, float* gamma) {
    const gma_desc& d = a.d;
    const Geo g = geometry(d);
    const int nph = resp_phases(g);
    RespFn rf = nph ? select_resp(g, nph, kRespRows) : nullptr;
    if (!rf) return hipErrorNotSupported;
    hipError_t e;
    if ((e = launch_prep(a, g, W, cvec)) != hipSuccess) return e;
    const int Np = (d.N + kGroup - 1) / kGroup * kGroup;
    bf16_t* gq = reinterpret_cast<bf16_t*>(gamma);
    bf16_t* gk = reinterpret_cast<bf16_t*>(gamma + (size_t)d.B * d.H * d.N * d.K);
    return launch_resp(a, g, rf, nph, Np, 2, W, cvec, gq, gk);
}

}  // namespace mf
}  // namespace gma
