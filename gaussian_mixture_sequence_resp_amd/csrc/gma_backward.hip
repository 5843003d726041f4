// Backward of the GMA forward mixer (bidirectional and causal): SIMT kernels, with
// matrix-core forms for bf16 inputs: the causal chunk walks on fp32 matrix cores; the
// bidirectional row passes, the segment partials and the parameter sums on bf16 matrix cores
// over exact three-piece bf16 splits of their fp32 operands; dqr, dkr on bf16 matrix cores
// over exact hi/lo pairs.
//
// Method: Gaussian Mixture Attention (arXiv 2606.18283).  The mixture parameters are trained
// end to end by backpropagation ("Core mechanism" item 3); the pages analyse the gradients'
// structure (responsibility-modulated).  Given dO = dL/dO this computes dL/d(qr, kr, v, mu,
// var_raw, prior_logits) by the chain rule of the forward:
//   num_i = gamma_Q,i S_i, den_i = gamma_Q,i . z_i + eps, O_i = num_i / den_i, with [S_i | z_i]
//   the memory totals (bidirectional) or the inclusive prefix up to i (causal);
//   g_num_i = dO_i / den_i, g_den_i = -(dO_i . O_i) / den_i;
//   dgamma_Q,i = S_i g_num_i + z_i g_den_i;
//   [R_j | r_j] = sum of gamma_Q,i (x) [g_num_i | g_den_i] over the rows i that read row j
//   (all rows, or i >= j when causal);  dv_j = gamma_K,j R_j,  dgamma_K,j = R_j v_j + r_j;
//   softmax: dl = gamma (dgamma - gamma . dgamma);
//   log joint: dx_d = -sum_k dl_k (x_d - mu_kd) / var_kd, dmu_kd = sum dl_k (x_d - mu_kd) / var_kd,
//   dvar_kd = sum dl_k (-1/2)(1/var_kd - (x_d - mu_kd)^2 / var_kd^2), dlog pi_k = sum dl_k;
//   dvar_raw = dvar sigmoid(var_raw), dprior = dlog pi - pi sum_k dlog pi_k.
//
// Kernels (caller's stream, in this order):
//   params_kernel, resp_kernel   (the SIMT forward's) 1/var and constants; gamma_Q, gamma_K
//                                (in double for float32 inputs); for bf16 inputs the
//                                matrix-core responsibilities kernel (gma_prep, then
//                                gma_causal_resp writing float rows) gives gamma instead
//   per pass (pass 1 gives g_num, g_den and dl_Q; pass 2 gives dv and dl_K), the rows of each
//   head cut into SEG contiguous segments:
//   bwd_seg_partial  the segment's weighted rows summed in order (K x (d_v + 1) per segment,
//                  LDS-tiled; bwd_seg_partial_bf16 for bf16 inputs: split-bf16 matrix-core
//                  products over 32-row blocks staged in LDS)
//   bwd_seg_start    each segment's starting state from those partials in segment order: the
//                  prefix before it (causal pass 1), the suffix after it (causal pass 2) or
//                  the head's total (bidirectional)
//   bwd_causal_mfma  causal, bf16 inputs (K <= 128, d_v = 32, 64 or 128): one wave per
//                  (b, h, segment) walks its rows in chunks of 32 (pass 2 in reverse), the
//                  chunk's products as fp32 matrix-core tiles against the state in LDS
//   bwd_causal_mfma2 the same for 128 < K <= 256 with two waves per (b, h, segment), each
//                  half the components (the contractions over the components added
//                  through LDS)
//   bwd_seg_chunks   causal otherwise, when the state and a chunk's rows fit LDS: the same
//                  chunk walk, 16 rows at a time, on the vector ALUs
//   bwd_seg_rows     causal otherwise: one workgroup per (b, h, segment) walks its rows (pass
//                  2 in reverse) with the state in LDS (in the workspace when it does not fit)
//   bwd_bidir_bf16 bidirectional, bf16 inputs: the per-row arithmetic against the head's
//                  total as split-bf16 matrix-core products over 32-row tiles
//   bwd_bidir_rows   bidirectional otherwise: the same per-row arithmetic, each wave of a
//                  workgroup walking its own rows
//   bwd_x_bf16     bf16 inputs, d_r <= 64: dqr, dkr = Q - x P with P = dl lam, Q = dl (mu lam)
//                  on bf16 matrix cores, every fp32 operand split exactly into a bf16 pair
//                  (hi.hi + lo.hi + hi.lo); the lam / mu lam pieces prepared by bwd_x_pieces
//   bwd_x_mfma     bf16 inputs otherwise: the same as fp32 matrix-core products over 32-row
//                  tiles
//   bwd_x          otherwise: the same with LDS-tiled contractions over the components (in A)
//   bwd_param_part per chunk of rows (both sides, all b), LDS-tiled sums S0 = sum dl,
//                  S1 = sum dl x, S2 = sum dl x^2 per (h, k, d) (in A), stored in double;
//                  bwd_param_bf16 the same for bf16 inputs as split-bf16 matrix-core products
//   bwd_param_final, bwd_prior_final the chunk sums added in chunk order; dmu, dvar_raw;
//                  dprior
// Every sum has a fixed order: results are deterministic.
#include <math.h>

#include "gma_internal.h"
#include "gma_mfma_geo.h"
#include "gma_numeric.h"

namespace gma {
namespace {

constexpr int kBwdThreads = 256;
constexpr size_t kScanLdsMax = 150 * 1024;  // dynamic LDS cap of the row, chunk and dx kernels
constexpr int kParamChunks = 64;  // most chunks of rows of the parameter sums

// Sums over rows are split into SEG contiguous segments of L rows per head.  The state of a
// pass is [K][W] (W = d_v + 1), kept in A: double for float32 inputs (gamma included: the
// chain rule cancels, e.g. R v_j + r against gamma . dgamma, and a sharp posterior's
// dl = gamma (dgamma - s) is far smaller than float's rounding of gamma times dgamma; the
// 1e-5 gate needs double); float for bf16.
//   pass 1: rows u_j = [v_j | 1] weighted by gamma_K,j  (the forward's memory / prefix);
//   pass 2: rows u_i = [g_num_i | g_den_i] weighted by gamma_Q,i  ([R | r]; suffix for causal).

// Row j of a pass's weighted rows: weight gamma_j[k], row entry c (c < d_v: v or g_num; c = d_v:
// 1 or g_den).
template <typename T, typename A, int PASS>
__device__ __forceinline__ A pass_row(const T* v_bh, const A* gnum_bh, const A* gden_bh, int dv, int j, int c) {
    if constexpr (PASS == 1)
        return c < dv ? (A)Elem<T>::load(v_bh, (size_t)j * dv + c) : (A)1;
    else
        return c < dv ? gnum_bh[(size_t)j * dv + c] : gden_bh[j];
}

// Partial state of every segment: part[bh][seg][k][c] = sum over the segment's rows j, in
// order, of gamma[side][bh][j][k] * u_j[c], for a tile of 32 components x 64 columns per
// workgroup (rows staged 64 at a time in LDS; each thread one component and 8 columns).
// Grid (ceil(K / 32) ceil(W / 64), BH * SEG).
constexpr int kSK = 32, kSC = 64, kSR = 64;
template <typename T, typename A, int PASS>
__global__ void __launch_bounds__(kBwdThreads)
    bwd_seg_partial(const A* __restrict__ gamma, const T* __restrict__ v, const A* __restrict__ gnum,
                    const A* __restrict__ gden, A* __restrict__ part, int BH, int N, int K, int dv, int SEG, int L) {
    __shared__ A sg[kSR][kSK + 1];
    __shared__ A su[kSR][kSC + 1];
    const int W = dv + 1;
    const int t = threadIdx.x;
    const int nkt = (K + kSK - 1) / kSK;
    const int k0 = (blockIdx.x % nkt) * kSK, c0 = (blockIdx.x / nkt) * kSC;
    const int bs = blockIdx.y, bh = bs / SEG, seg = bs % SEG;
    const int side = PASS == 1 ? 1 : 0;  // pass 1 weights by gamma_K, pass 2 by gamma_Q
    const A* g = gamma + ((size_t)side * BH + bh) * N * K;
    const T* v_bh = v + (size_t)bh * N * dv;
    const A* gnum_bh = gnum + (size_t)bh * N * dv;
    const A* gden_bh = gden + (size_t)bh * N;
    const int j0 = seg * L, j1 = min(N, j0 + L);
    const int kl = t >> 3, cg = t & 7;
    A acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0;
    for (int jb = j0; jb < j1; jb += kSR) {
        for (int idx = t; idx < kSR * kSK; idx += kBwdThreads) {
            const int rr = idx / kSK, kk = idx % kSK;
            const int j = jb + rr, k = k0 + kk;
            sg[rr][kk] = (j < j1 && k < K) ? g[(size_t)j * K + k] : (A)0;
        }
        for (int idx = t; idx < kSR * kSC; idx += kBwdThreads) {
            const int rr = idx / kSC, cc = idx % kSC;
            const int j = jb + rr, c = c0 + cc;
            su[rr][cc] = (j < j1 && c < W) ? pass_row<T, A, PASS>(v_bh, gnum_bh, gden_bh, dv, j, c) : (A)0;
        }
        __syncthreads();
#pragma unroll 4
        for (int rr = 0; rr < kSR; ++rr) {
            const A gv = sg[rr][kl];
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] += gv * su[rr][cg + 8 * q];
        }
        __syncthreads();
    }
    const int k = k0 + kl;
    if (k >= K) return;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int c = c0 + cg + 8 * q;
        if (c < W) part[(size_t)bs * K * W + (size_t)k * W + c] = acc[q];
    }
}

// Starting state of every segment from the partials, summed in segment order: causal pass 1
// the exclusive prefix (segments before), causal pass 2 the exclusive suffix (segments after);
// bidirectional the total of all segments (slot 0 only).  Grid (ceil(K W / 256), BH).
template <typename A, int PASS>
__global__ void __launch_bounds__(kBwdThreads)
    bwd_seg_start(const A* __restrict__ part, A* __restrict__ start, int K, int dv, int SEG, int causal) {
    const int W = dv + 1;
    const int e = blockIdx.x * kBwdThreads + threadIdx.x;
    const int bh = blockIdx.y;
    if (e >= K * W) return;
    const size_t base = (size_t)bh * SEG * K * W + e;
    A acc = 0;
    if (!causal) {
        for (int s = 0; s < SEG; ++s) acc += part[base + (size_t)s * K * W];
        start[base] = acc;
    } else if (PASS == 1) {
        for (int s = 0; s < SEG; ++s) {
            start[base + (size_t)s * K * W] = acc;
            acc += part[base + (size_t)s * K * W];
        }
    } else {
        for (int s = SEG - 1; s >= 0; --s) {
            start[base + (size_t)s * K * W] = acc;
            acc += part[base + (size_t)s * K * W];
        }
    }
}

// Wave-wide sum (64 lanes).
template <typename A>
__device__ __forceinline__ A wave_sum(A x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

constexpr int kRowThreads = 256;
constexpr int kRowWaves = kRowThreads / 64;

// sum_{k in [k0, k1)} g[k] st[k W + c], four independent partial sums (added in a fixed order).
template <typename A>
__device__ __forceinline__ A dot_k(const A* g, const A* st, int W, int c, int k0, int k1) {
    A p0 = 0, p1 = 0, p2 = 0, p3 = 0;
    int k = k0;
    for (; k + 4 <= k1; k += 4) {
        p0 += g[k] * st[(size_t)k * W + c];
        p1 += g[k + 1] * st[(size_t)(k + 1) * W + c];
        p2 += g[k + 2] * st[(size_t)(k + 2) * W + c];
        p3 += g[k + 3] * st[(size_t)(k + 3) * W + c];
    }
    for (; k < k1; ++k) p0 += g[k] * st[(size_t)k * W + c];
    return (p0 + p1) + (p2 + p3);
}

// sum_c st[k W + c] u[c] over all W columns, four independent partial sums.
template <typename A>
__device__ __forceinline__ A dot_c(const A* st, const A* u, int W, int k) {
    const A* r = st + (size_t)k * W;
    A p0 = 0, p1 = 0, p2 = 0, p3 = 0;
    int c = 0;
    for (; c + 4 <= W; c += 4) {
        p0 += r[c] * u[c];
        p1 += r[c + 1] * u[c + 1];
        p2 += r[c + 2] * u[c + 2];
        p3 += r[c + 3] * u[c + 3];
    }
    for (; c < W; ++c) p0 += r[c] * u[c];
    return (p0 + p1) + (p2 + p3);
}

// One workgroup (4 waves) per (bh, segment): the segment's rows in order (pass 1: ascending;
// pass 2: descending), the state st [K][W] in LDS (or in the workspace at st_global when it
// does not fit), starting from the segment's start state.  Causal: the row's own weighted row
// is added first (the sums are inclusive).  Pass 1 row i: num | den = gamma_Q,i . st, g_num,
// g_den, dgamma_Q = st g, dl_Q.  Pass 2 row j: dv_j = gamma_K,j . st (value part),
// dgamma_K = st [v_j | 1], dl_K.  Contractions over k are split into one contiguous range of
// components per wave, and the four wave partials are added in wave order.  LDS scratch after
// the state: sga [K] (the row's gamma), sgb [K] (the other side's, then dgamma), su [W],
// sw [W], spart [4][W], sred [4].
template <typename T, typename A, int PASS>
__global__ void __launch_bounds__(kRowThreads)
    bwd_seg_rows(const A* __restrict__ gamma, const T* __restrict__ v, const T* __restrict__ dout,
                 A* __restrict__ gnum, A* __restrict__ gden, A* __restrict__ dl, T* __restrict__ dv_out,
                 const A* __restrict__ start, A* st_global, int BH, int N, int K, int dv, float eps, int causal,
                 int SEG, int L) {
    extern __shared__ double smem_d[];
    A* smem = reinterpret_cast<A*>(smem_d);
    const int W = dv + 1;
    const int KW = K * W;
    const int bs = blockIdx.x, bh = bs / SEG, seg = bs % SEG;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    A* st = st_global ? st_global + (size_t)bs * KW : smem;
    A* sga = st_global ? smem : smem + (size_t)KW;
    A* sgb = sga + K;
    A* su = sgb + K;
    A* sw = su + W;
    A* spart = sw + W;
    A* sred = spart + kRowWaves * W;
    const A* gq = gamma + (size_t)bh * N * K;
    const A* gk = gamma + ((size_t)BH + bh) * N * K;
    const T* v_bh = v + (size_t)bh * N * dv;
    const T* do_bh = dout + (size_t)bh * N * dv;
    A* gnum_bh = gnum + (size_t)bh * N * dv;
    A* gden_bh = gden + (size_t)bh * N;
    const A* st0 = start + ((size_t)bh * SEG + (causal ? seg : 0)) * KW;
    for (int e = t; e < KW; e += kRowThreads) st[e] = st0[e];
    // this wave's component range of the k-contractions
    const int kq = (K + kRowWaves - 1) / kRowWaves;
    const int k0 = min(K, wv * kq), k1 = min(K, k0 + kq);
    const int i0 = seg * L, i1 = min(N, i0 + L);
    for (int step = 0; step < i1 - i0; ++step) {
        const int i = PASS == 1 ? i0 + step : i1 - 1 - step;
        __syncthreads();
        // sga: this row's gamma on the reading side; sgb, su: the weighted row added to the state
        const A* grow = (PASS == 1 ? gq : gk) + (size_t)i * K;
        for (int k = t; k < K; k += kRowThreads) sga[k] = grow[k];
        if (causal) {
            const A* wrow = (PASS == 1 ? gk : gq) + (size_t)i * K;
            for (int k = t; k < K; k += kRowThreads) sgb[k] = wrow[k];
            for (int c = t; c < W; c += kRowThreads) su[c] = pass_row<T, A, PASS>(v_bh, gnum_bh, gden_bh, dv, i, c);
            __syncthreads();
            for (int k = wv; k < K; k += kRowWaves) {
                const A gkk = sgb[k];
                for (int c = lane; c < W; c += 64) st[(size_t)k * W + c] += gkk * su[c];
            }
        }
        __syncthreads();
        // gamma . st over this wave's components, for the value columns (and den in pass 1)
        const int ncol = PASS == 1 ? W : dv;
        for (int c = lane; c < ncol; c += 64) spart[wv * W + c] = dot_k(sga, st, W, c, k0, k1);
        __syncthreads();
        if constexpr (PASS == 1) {
            for (int c = t; c < W; c += kRowThreads) sw[c] = ((spart[c] + spart[W + c]) + spart[2 * W + c]) + spart[3 * W + c];
            __syncthreads();
            const A den = sw[dv] + (A)eps;
            if (wv == 0) {
                A dot = 0;
                for (int c = lane; c < dv; c += 64) dot += (A)Elem<T>::load(do_bh, (size_t)i * dv + c) * (sw[c] / den);
                dot = wave_sum(dot);
                if (lane == 0) sred[0] = -dot / den;
            }
            __syncthreads();
            const A gd = sred[0];
            for (int c = t; c < W; c += kRowThreads) {
                const A g = c < dv ? (A)Elem<T>::load(do_bh, (size_t)i * dv + c) / den : gd;
                sw[c] = g;
                if (c < dv) gnum_bh[(size_t)i * dv + c] = g;
            }
            if (t == 0) gden_bh[i] = gd;
        } else {
            T* dv_bh = dv_out + (size_t)bh * N * dv;
            for (int c = t; c < dv; c += kRowThreads)
                Elem<T>::store(dv_bh, (size_t)i * dv + c,
                               (float)(((spart[c] + spart[W + c]) + spart[2 * W + c]) + spart[3 * W + c]));
            for (int c = t; c < W; c += kRowThreads) sw[c] = c < dv ? (A)Elem<T>::load(v_bh, (size_t)i * dv + c) : (A)1;
        }
        __syncthreads();
        // dgamma = st sw, then the softmax backward dl = gamma (dgamma - gamma . dgamma)
        A part = 0;
        for (int k = t; k < K; k += kRowThreads) {
            const A a = dot_c(st, sw, W, k);
            sgb[k] = a;  // sgb is free once the state update above is done
            part += sga[k] * a;
        }
        part = wave_sum(part);
        if (lane == 0) sred[1 + wv] = part;  // sred[1..4]
        __syncthreads();
        const A s = ((sred[1] + sred[2]) + sred[3]) + sred[4];
        A* dl_row = dl + ((size_t)(PASS == 1 ? 0 : BH) + bh) * N * K + (size_t)i * K;
        for (int k = t; k < K; k += kRowThreads) dl_row[k] = sga[k] * (sgb[k] - s);
    }
}

// Bidirectional rows: the state (the head's total) is the same for every row, so each wave
// walks its own rows of the segment (rows i0 + wave, i0 + wave + 4, ...) with wave-private
// LDS scratch and no workgroup barrier in the loop; the per-row arithmetic is that of
// bwd_seg_rows with every contraction over components taken by one wave.  LDS: the state
// [K][W], then per wave sga [K], sgb [K], sw [W].
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

template <typename T, typename A, int PASS>
__global__ void __launch_bounds__(kRowThreads)
    bwd_bidir_rows(const A* __restrict__ gamma, const T* __restrict__ v, const T* __restrict__ dout,
                   A* __restrict__ gnum, A* __restrict__ gden, A* __restrict__ dl, T* __restrict__ dv_out,
                   const A* __restrict__ start, const A* st_global, int BH, int N, int K, int dv, float eps, int SEG,
                   int L) {
    extern __shared__ double smem_d[];
    A* smem = reinterpret_cast<A*>(smem_d);
    const int W = dv + 1;
    const int KW = K * W;
    const int bs = blockIdx.x, bh = bs / SEG, seg = bs % SEG;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const A* st0 = start + (size_t)bh * SEG * KW;  // slot 0: the head's total
    A* st_lds = smem;
    const A* st = st_global ? st0 : st_lds;
    A* scratch = st_global ? smem : smem + (size_t)KW;
    A* sga = scratch + (size_t)wv * (2 * K + W);
    A* sgb = sga + K;
    A* sw = sgb + K;
    if (!st_global) {
        for (int e = t; e < KW; e += kRowThreads) st_lds[e] = st0[e];
        __syncthreads();
    }
    const A* gq = gamma + (size_t)bh * N * K;
    const A* gk = gamma + ((size_t)BH + bh) * N * K;
    const T* v_bh = v + (size_t)bh * N * dv;
    const T* do_bh = dout + (size_t)bh * N * dv;
    A* gnum_bh = gnum + (size_t)bh * N * dv;
    A* gden_bh = gden + (size_t)bh * N;
    const int i0 = seg * L, i1 = min(N, i0 + L);
    for (int i = i0 + wv; i < i1; i += kRowWaves) {
        const A* grow = (PASS == 1 ? gq : gk) + (size_t)i * K;
        for (int k = lane; k < K; k += 64) sga[k] = grow[k];
        wave_lds_sync();
        if constexpr (PASS == 1) {
            for (int c = lane; c < W; c += 64) sw[c] = dot_k(sga, st, W, c, 0, K);
            wave_lds_sync();
            const A den = sw[dv] + (A)eps;
            A dot = 0;
            for (int c = lane; c < dv; c += 64) dot += (A)Elem<T>::load(do_bh, (size_t)i * dv + c) * (sw[c] / den);
            const A gd = -wave_sum(dot) / den;
            wave_lds_sync();
            for (int c = lane; c < W; c += 64) {
                const A g = c < dv ? (A)Elem<T>::load(do_bh, (size_t)i * dv + c) / den : gd;
                sw[c] = g;
                if (c < dv) gnum_bh[(size_t)i * dv + c] = g;
            }
            if (lane == 0) gden_bh[i] = gd;
        } else {
            T* dv_bh = dv_out + (size_t)bh * N * dv;
            for (int c = lane; c < dv; c += 64) Elem<T>::store(dv_bh, (size_t)i * dv + c, (float)dot_k(sga, st, W, c, 0, K));
            for (int c = lane; c < W; c += 64) sw[c] = c < dv ? (A)Elem<T>::load(v_bh, (size_t)i * dv + c) : (A)1;
        }
        wave_lds_sync();
        A part = 0;
        for (int k = lane; k < K; k += 64) {
            const A a = dot_c(st, sw, W, k);
            sgb[k] = a;
            part += sga[k] * a;
        }
        const A s = wave_sum(part);
        A* dl_row = dl + ((size_t)(PASS == 1 ? 0 : BH) + bh) * N * K + (size_t)i * K;
        for (int k = lane; k < K; k += 64) dl_row[k] = sga[k] * (sgb[k] - s);
        wave_lds_sync();
    }
}

// Matrix-core forms for bf16 inputs (float state, gamma and row gradients).  The fp32 form
// (v_mfma_f32_32x32x2_f32, used by the causal chunk walks) pairs one contraction index of
// each lane half per step, chosen so that the B operand of the step is a register the lane
// already holds in the C layout (lane l, register i of tile m: index 32 m + 8 (i / 4) +
// 4 (l / 32) + i % 4 of row l % 32).  The split-bf16 forms (v_mfma_f32_32x32x16_bf16 on
// hi/lo pairs) stage or regroup their operands into 8 consecutive contraction indices per
// lane.  Row kernels take blocks of RB rows of one head, their waves 32-row tiles in turn.
constexpr int kMfRowThreads = 256;
constexpr int kMfRowBlock = 512;  // rows per workgroup of bwd_bidir_bf16: 4 tiles per wave
using mf::f32x16;
using mf::sum_halves;

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Two fp32 values as their bf16 hi and lo pairs (element 0 in the low half): hi = rne(v),
// lo = rne(v - hi), v to ~2^-17 relative.
__device__ __forceinline__ void split_pair(float v0, float v1, uint32_t& hi, uint32_t& lo) {
    hi = mf::pack_bf16(v0, v1);
    lo = mf::pack_bf16(v0 - mf::bf16lo_to_f32(hi), v1 - mf::bf16hi_to_f32(hi));
}

// Two fp32 values as three bf16 pieces each, v = p1 + p2 + p3 exactly (8 + 8 + 8 significant
// bits; every residual is exact in fp32): for sums whose terms cancel (the parameter
// gradients, the states the chunk walks start from), where two pieces (~2^-17) lost accuracy.
__device__ __forceinline__ void split3_pair(float v0, float v1, uint32_t& p1, uint32_t& p2, uint32_t& p3) {
    p1 = mf::pack_bf16(v0, v1);
    const float r0 = v0 - mf::bf16lo_to_f32(p1), r1 = v1 - mf::bf16hi_to_f32(p1);
    p2 = mf::pack_bf16(r0, r1);
    p3 = mf::pack_bf16(r0 - mf::bf16lo_to_f32(p2), r1 - mf::bf16hi_to_f32(p2));
}

// Causal rows in chunks of kCh positions (the chunked form of the walk, as the forward's
// scan): with St the state before the chunk (pass 1: the prefix before it; pass 2: the
// suffix after it), rows r of the chunk and the chunk's own rows j on the inclusive side
// (pass 1: j <= r; pass 2: j >= r),
//   read_r   = ga_r St + sum_j (ga_r . gb_j) w_j        (pass 1: num; pass 2: dv)
//   dgamma_r = St x_r + sum_j (w_j . x_r) gb_j          (x: g_r in pass 1, [v_r | 1] in pass 2)
// with ga the row's own gamma (pass 1 gamma_Q, pass 2 gamma_K), gb the weighted side's
// gamma and w its rows ([v | 1], or [g_num | g_den]); then St += sum_j gb_j (x) w_j.  The
// same sums as the row-at-a-time walk, regrouped, with one workgroup barrier per step of a
// chunk instead of per row.  LDS: St [K][W], sga, sgb [kCh][K + 1], sw, sx [kCh][W + 1],
// sP, sQ [kCh][kCh].
constexpr int kCh = 16;

template <typename A>
__device__ __forceinline__ A sum16(A x) {  // over the 16 lanes of a row group
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

template <typename T, typename A, int PASS>
__global__ void __launch_bounds__(kBwdThreads)
    bwd_seg_chunks(const A* __restrict__ gamma, const T* __restrict__ v, const T* __restrict__ dout,
                   A* __restrict__ gnum, A* __restrict__ gden, A* __restrict__ dl, T* __restrict__ dv_out,
                   const A* __restrict__ start, int BH, int N, int K, int dv, float eps, int SEG, int L) {
    extern __shared__ double smem_d[];
    A* st = reinterpret_cast<A*>(smem_d);
    const int W = dv + 1, KW = K * W, K1 = K + 1, W1 = W + 1;
    A* sga = st + KW;
    A* sgb = sga + kCh * K1;
    A* sw = sgb + kCh * K1;
    A* sx = sw + kCh * W1;
    A* sP = sx + kCh * W1;
    A* sQ = sP + kCh * kCh;
    const int bs = blockIdx.x, bh = bs / SEG, seg = bs % SEG;
    const int t = threadIdx.x;
    const A* st0 = start + ((size_t)bh * SEG + seg) * KW;
    for (int e = t; e < KW; e += kBwdThreads) st[e] = st0[e];
    const A* gq = gamma + (size_t)bh * N * K;
    const A* gk = gamma + ((size_t)BH + bh) * N * K;
    const A* ga_g = PASS == 1 ? gq : gk;  // the row's own side
    const A* gb_g = PASS == 1 ? gk : gq;  // the weighted side
    const T* v_bh = v + (size_t)bh * N * dv;
    const T* do_bh = dout + (size_t)bh * N * dv;
    A* gnum_bh = gnum + (size_t)bh * N * dv;
    A* gden_bh = gden + (size_t)bh * N;
    A* dl_bh = dl + ((size_t)(PASS == 1 ? 0 : BH) + bh) * N * K;
    const int i0 = seg * L, i1 = min(N, i0 + L);
    const int nch = (i1 - i0 + kCh - 1) / kCh;
    const int rg = t >> 4, l16 = t & 15;  // row group of 16 lanes
    for (int q = 0; q < nch; ++q) {
        const int c0 = PASS == 1 ? i0 + kCh * q : max(i0, i1 - kCh * (q + 1));
        const int c1 = PASS == 1 ? min(i1, c0 + kCh) : i1 - kCh * q;
        const int nr = c1 - c0;
        __syncthreads();
        for (int idx = t; idx < kCh * K; idx += kBwdThreads) {
            const int r = idx / K, k = idx % K;
            sga[r * K1 + k] = r < nr ? ga_g[(size_t)(c0 + r) * K + k] : (A)0;
            sgb[r * K1 + k] = r < nr ? gb_g[(size_t)(c0 + r) * K + k] : (A)0;
        }
        for (int idx = t; idx < kCh * W; idx += kBwdThreads) {
            const int r = idx / W, c = idx % W;
            A wv = 0, xv = 0;
            if (r < nr) {
                const A u = c < dv ? (A)Elem<T>::load(v_bh, (size_t)(c0 + r) * dv + c) : (A)1;
                if constexpr (PASS == 1) {
                    wv = u;
                } else {
                    wv = c < dv ? gnum_bh[(size_t)(c0 + r) * dv + c] : gden_bh[c0 + r];
                    xv = u;
                }
            }
            sw[r * W1 + c] = wv;
            sx[r * W1 + c] = xv;
        }
        __syncthreads();
        // P[r][j] = ga_r . gb_j on the inclusive side
        {
            const int r = t >> 4, j = t & 15;
            A a = 0;
            if (PASS == 1 ? j <= r : j >= r)
                for (int k = 0; k < K; ++k) a += sga[r * K1 + k] * sgb[j * K1 + k];
            sP[r * kCh + j] = a;
        }
        __syncthreads();
        // read_r[c] = ga_r St[:, c] + sum_j P[r][j] w_j[c]
        const int ncol = PASS == 1 ? W : dv;
        for (int idx = t; idx < kCh * ncol; idx += kBwdThreads) {
            const int r = idx / ncol, c = idx % ncol;
            A a0 = 0, a1 = 0;
            int k = 0;
            for (; k + 2 <= K; k += 2) {
                a0 += sga[r * K1 + k] * st[(size_t)k * W + c];
                a1 += sga[r * K1 + k + 1] * st[(size_t)(k + 1) * W + c];
            }
            for (; k < K; ++k) a0 += sga[r * K1 + k] * st[(size_t)k * W + c];
            A a = a0 + a1;
            for (int j = 0; j < kCh; ++j) a += sP[r * kCh + j] * sw[j * W1 + c];
            if constexpr (PASS == 1) {
                sx[r * W1 + c] = a;  // num, turned into g below
            } else if (r < nr) {
                Elem<T>::store(dv_out + (size_t)bh * N * dv, (size_t)(c0 + r) * dv + c, (float)a);
            }
        }
        __syncthreads();
        if constexpr (PASS == 1) {
            // g_r = [dout_r / den_r | -(dout_r . num_r / den_r) / den_r], 16 lanes per row
            const int r = rg;
            const bool ok = r < nr;
            const A den = sx[r * W1 + dv] + (A)eps;
            A dot = 0;
            for (int c = l16; c < dv; c += 16)
                if (ok) dot += (A)Elem<T>::load(do_bh, (size_t)(c0 + r) * dv + c) * (sx[r * W1 + c] / den);
            const A gd = -sum16(dot) / den;
            for (int c = l16; c < W; c += 16) {
                const A gv = c < dv ? (ok ? (A)Elem<T>::load(do_bh, (size_t)(c0 + r) * dv + c) / den : (A)0) : (ok ? gd : (A)0);
                sx[r * W1 + c] = gv;
                if (ok && c < dv) gnum_bh[(size_t)(c0 + r) * dv + c] = gv;
            }
            if (ok && l16 == 0) gden_bh[c0 + r] = gd;
            __syncthreads();
        }
        // Q[r][j] = w_j . x_r on the inclusive side
        {
            const int r = t >> 4, j = t & 15;
            A a = 0;
            if (PASS == 1 ? j <= r : j >= r)
                for (int c = 0; c < W; ++c) a += sw[j * W1 + c] * sx[r * W1 + c];
            sQ[r * kCh + j] = a;
        }
        __syncthreads();
        // dgamma_r[k] = St[k] . x_r + sum_j Q[r][j] gb_j[k]; s_r; dl_r = ga_r (dgamma_r - s_r)
        {
            const int r = rg;
            constexpr int kMaxPer = GMA_MAX_K / 16;
            A dg[kMaxPer];
            A part = 0;
#pragma unroll
            for (int m = 0; m < kMaxPer; ++m) {
                const int k = l16 + 16 * m;
                A a = 0;
                if (k < K) {
                    const A* srow = st + (size_t)k * W;
                    A b0 = 0, b1 = 0;
                    int c = 0;
                    for (; c + 2 <= W; c += 2) {
                        b0 += srow[c] * sx[r * W1 + c];
                        b1 += srow[c + 1] * sx[r * W1 + c + 1];
                    }
                    for (; c < W; ++c) b0 += srow[c] * sx[r * W1 + c];
                    a = b0 + b1;
                    for (int j = 0; j < kCh; ++j) a += sQ[r * kCh + j] * sgb[j * K1 + k];
                    part += sga[r * K1 + k] * a;
                }
                dg[m] = a;
            }
            const A sdot = sum16(part);
            if (r < nr) {
#pragma unroll
                for (int m = 0; m < kMaxPer; ++m) {
                    const int k = l16 + 16 * m;
                    if (k < K) dl_bh[(size_t)(c0 + r) * K + k] = sga[r * K1 + k] * (dg[m] - sdot);
                }
            }
        }
        __syncthreads();
        // St += sum_j gb_j (x) w_j over the chunk (rows past its end are zero)
        for (int e = t; e < KW; e += kBwdThreads) {
            const int k = e / W, c = e - k * W;
            A a = st[e];
            for (int j = 0; j < kCh; ++j) a += sgb[j * K1 + k] * sw[j * W1 + c];
            st[e] = a;
        }
    }
}

// Causal rows on the matrix cores (bf16 inputs: float gamma and state): one wave per
// (b, h, segment) walks the segment in chunks of 32 positions (pass 1 ascending, pass 2
// descending), the state St (value columns [Kp][32 NTW + 1] and the normaliser column z
// [Kp]) in LDS.  For chunk rows r and the chunk's rows j on the inclusive side (pass 1:
// j <= r, pass 2: j >= r), with ga the rows' own gamma, gb the weighted side's, W the
// weighted rows (pass 1 [v | 1], pass 2 [g_num | g_den]) and X the rows' multipliers
// (pass 1 [g_num | g_den], formed here; pass 2 [v | 1]):
//   P^T[j][r]   = gb_j . ga_r                   (masked to the inclusive side)
//   READ^T      = St^T ga^T + W^T P^T           (pass 1: [num | den - eps]; pass 2: dv)
//   Q^T[j][r]   = W_j . X_r                     (masked)
//   DG^T        = St X^T + gb^T Q^T             (dgamma of every row)
//   dl_r        = ga_r (dg_r - s_r),  s_r = ga_r . dg_r = X_r . READ0_r + Q_r . P_r
//   St         += gb^T W
// where READ0 = ga St is READ without the chunk's own rows: the regrouped row sum s_r
// lets each 32-component tile of DG be finished and stored as soon as it is formed.
// v_mfma_f32_32x32x2_f32 throughout (fp32 products and sums).  A step contracts one index
// per lane half, paired so that the register operands are read in the C layout (lane l,
// register i of a tile: row 8 (i / 4) + 4 (l / 32) + i % 4 of the tile, column l % 32):
// ga, gb, P^T, X^T and Q^T in that layout; St from LDS (odd row stride: the 32 rows of one
// column fall in distinct banks); gb^T (gb with rows and components swapped) and W rows
// loaded from global memory in the operand order each step needs.  The z column (value
// dv) is handled alongside on the vector ALUs.
template <int MT, int NTW>
struct CausalMf {
    static constexpr int Kp = 32 * MT, Wv = 32 * NTW, Ws = Wv + 1;
    static size_t lds_bytes() { return ((size_t)Kp * Ws + Kp) * sizeof(float); }
};

__device__ __forceinline__ int tile_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

template <typename T, int PASS, int MT, int NTW>
__global__ void __launch_bounds__(64)
    bwd_causal_mfma(const float* __restrict__ gamma, const T* __restrict__ v, const T* __restrict__ dout,
                    float* __restrict__ gnum, float* __restrict__ gden, float* __restrict__ dl,
                    T* __restrict__ dv_out, const float* __restrict__ start, int BH, int N, int K, int dv, float eps,
                    int SEG, int L) {
    extern __shared__ double smem_d[];
    using C = CausalMf<MT, NTW>;
    constexpr int Kp = C::Kp, Wv = C::Wv, Ws = C::Ws;
    float* sS = reinterpret_cast<float*>(smem_d);  // [Kp][Ws]: value columns
    float* sZ = sS + (size_t)Kp * Ws;               // [Kp]: the normaliser column
    const int W = dv + 1;                           // dv == Wv
    const int bs = blockIdx.x, bh = bs / SEG, seg = bs % SEG;
    const int l = threadIdx.x, col = l & 31, h = l >> 5;
    const float* st0 = start + ((size_t)bh * SEG + seg) * K * W;
    for (int e = l; e < Kp * Wv; e += 64) {
        const int k = e / Wv, c = e % Wv;
        sS[k * Ws + c] = k < K ? st0[(size_t)k * W + c] : 0.0f;
    }
    for (int k = l; k < Kp; k += 64) sZ[k] = k < K ? st0[(size_t)k * W + dv] : 0.0f;
    const float* ga_g = gamma + ((size_t)(PASS == 1 ? 0 : BH) + bh) * N * K;  // the rows' own side
    const float* gb_g = gamma + ((size_t)(PASS == 1 ? BH : 0) + bh) * N * K;  // the weighted side
    const T* v_bh = v + (size_t)bh * N * dv;
    const T* do_bh = dout + (size_t)bh * N * dv;
    float* gnum_bh = gnum + (size_t)bh * N * dv;
    float* gden_bh = gden + (size_t)bh * N;
    float* dl_bh = dl + ((size_t)(PASS == 1 ? 0 : BH) + bh) * N * K;
    T* dvo_bh = dv_out + (size_t)bh * N * dv;
    const bool vec_k = (K & 3) == 0;
    const int i0 = seg * L, i1 = min(N, i0 + L);
    const int nch = (i1 - i0 + 31) / 32;
    // W row j (value columns) and its last entry, in float
    auto wval = [&](int p, int c) -> float {
        if constexpr (PASS == 1) return Elem<T>::load(v_bh, (size_t)p * dv + c);
        else return gnum_bh[(size_t)p * dv + c];
    };
    auto wz = [&](int p) -> float {
        if constexpr (PASS == 1) return 1.0f;
        else return gden_bh[p];
    };
    // this lane's row p at its C-layout components 32 m + 8 q + 4 h + (0..3) of tile m (zeros
    // past K); rows outside the segment are loaded (clamped) and zeroed at the chunk's start,
    // so that no wait for these loads falls where they are issued
    auto gamma_tile = [&](const float* g, int p, int m, f32x16& out) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k0 = 32 * m + 8 * q + 4 * h;
            if (vec_k && k0 < K) {
                const float4 x = *reinterpret_cast<const float4*>(g + (size_t)p * K + k0);
                out[4 * q] = x.x;
                out[4 * q + 1] = x.y;
                out[4 * q + 2] = x.z;
                out[4 * q + 3] = x.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) out[4 * q + e] = k0 + e < K ? g[(size_t)p * K + k0 + e] : 0.0f;
            }
        }
    };
    auto gamma_c = [&](const float* g, int p, f32x16 (&out)[MT]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) gamma_tile(g, p, m, out[m]);
    };
    // chunk qc's rows r are positions base(qc) + r; rows outside [i0, i1) take no part
    auto base_of = [&](int qc) { return PASS == 1 ? i0 + 32 * qc : i1 - 32 * (qc + 1); };
    // gamma of a chunk's rows in the C layout; loaded for chunk 0 here and for chunk qc + 1
    // into each register array as soon as chunk qc is done with it (ga after the dl tiles,
    // gb one component tile at a time during the state update), so the loads overlap that
    // chunk's matrix work
    f32x16 ga[MT], gb[MT];
    {
        const int b0 = base_of(0), p0 = min(max(b0 + col, i0), i1 - 1);
        gamma_c(ga_g, p0, ga);
        gamma_c(gb_g, p0, gb);
    }
    for (int qc = 0; qc < nch; ++qc) {
        const int base = base_of(qc);
        auto in_seg = [&](int r) { return base + r >= i0 && base + r < i1; };
        auto clampp = [&](int r) { return min(max(base + r, i0), i1 - 1); };
        const bool okr = in_seg(col);
        const int pr = clampp(col);  // this lane's row (as r, and as j in the C layouts)
        // the next chunk's row of this lane (for the refills at the end)
        const int nbase = base_of(qc + 1);
        const int pn = min(max(nbase + col, i0), i1 - 1);
        if (!okr) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 16; ++i) ga[m][i] = gb[m][i] = 0.0f;
        }
        // ---- P^T = gb ga^T, masked to the inclusive side
        f32x16 pt;
#pragma unroll
        for (int i = 0; i < 16; ++i) pt[i] = 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) pt = mfma_f32(gb[m][i], ga[m][i], pt);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = tile_row(i, h);
            if (!(PASS == 1 ? j <= col : j >= col)) pt[i] = 0.0f;
        }
        // ---- W rows in the operand orders used below: wa[n][i] = W[j = tile_row(i, h)][32 n + col]
        float wa[NTW][16], wzj[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int pj = clampp(tile_row(i, h));
            wzj[i] = wz(pj);
#pragma unroll
            for (int n = 0; n < NTW; ++n) wa[n][i] = wval(pj, 32 * n + col);
        }
        // the epilogue's dO (pass 1) or v (pass 2) at this lane's columns and Q's W operand
        // (row col at columns 32 n + tile_row(i, h)): loaded now, used after READ0
        float xrow[NTW][16];
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int c = 32 * n + tile_row(i, h);
                xrow[n][i] = PASS == 1 ? (float)Elem<T>::load(do_bh, (size_t)pr * dv + c)
                                       : (float)Elem<T>::load(v_bh, (size_t)pr * dv + c);
            }
        // ---- READ0^T = St^T ga^T (value columns) and its z entry; PW^T = W^T P^T
        f32x16 rd0[NTW], pw[NTW];
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) rd0[n][i] = pw[n][i] = 0.0f;
        float r0z = 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int k = 32 * m + tile_row(i, h);
                const float* srow = sS + k * Ws + col;
#pragma unroll
                for (int n = 0; n < NTW; ++n) rd0[n] = mfma_f32(srow[32 * n], ga[m][i], rd0[n]);
                r0z = fmaf(ga[m][i], sZ[k], r0z);
            }
        r0z = sum_halves(r0z);
        float pwz = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
#pragma unroll
            for (int n = 0; n < NTW; ++n) pw[n] = mfma_f32(wa[n][i], pt[i], pw[n]);
            pwz = fmaf(pt[i], wzj[i], pwz);
        }
        pwz = sum_halves(pwz);
        // ---- the rows' multipliers X^T (C layout: register i of tile n is column 32 n + tile_row(i, h))
        f32x16 x[NTW];
        float xz;
        if constexpr (PASS == 1) {
            const float den = r0z + pwz + eps;
            float dot = 0.0f;
            const float(&dov)[NTW][16] = xrow;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) dot = fmaf(dov[n][i], (rd0[n][i] + pw[n][i]) / den, dot);
            const float gd = -sum_halves(dot) / den;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float g = okr ? dov[n][i] / den : 0.0f;
                    x[n][i] = g;
                    if (okr) gnum_bh[(size_t)pr * dv + 32 * n + tile_row(i, h)] = g;
                }
            xz = okr ? gd : 0.0f;
            if (okr && h == 0) gden_bh[pr] = gd;
        } else {
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int c = 32 * n + tile_row(i, h);
                    if (okr) Elem<T>::store(dvo_bh, (size_t)pr * dv + c, rd0[n][i] + pw[n][i]);
                    x[n][i] = okr ? xrow[n][i] : 0.0f;
                }
            xz = okr ? 1.0f : 0.0f;
        }
        // ---- Q^T = W X^T, masked (A: W row col at column 32 n + tile_row(i, h))
        f32x16 qt;
#pragma unroll
        for (int i = 0; i < 16; ++i) qt[i] = 0.0f;
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) qt = mfma_f32(wval(pr, 32 * n + tile_row(i, h)), x[n][i], qt);
        // z: Q^T[j][r] += W[j][dv] X[r][dv]; X[r][dv] of this register's column r = col is this lane's
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = tile_row(i, h);
            qt[i] = (PASS == 1 ? j <= col : j >= col) ? fmaf(wzj[i], xz, qt[i]) : 0.0f;
        }
        // ---- s_r = X_r . READ0_r + Q_r . P_r
        float sp = xz * r0z * 0.5f;  // both halves add it: half each
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) sp = fmaf(x[n][i], rd0[n][i], sp);
#pragma unroll
        for (int i = 0; i < 16; ++i) sp = fmaf(qt[i], pt[i], sp);
        const float s = sum_halves(sp);
        // ---- gb^T: gbt[m][i] = gb[j = tile_row(i, h)][32 m + col] (reusing gb's registers)
        f32x16 (&gbt)[MT] = gb;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int rj = tile_row(i, h);
            const bool okj = in_seg(rj);
            const int pj = clampp(rj);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int k = 32 * m + col;
                gbt[m][i] = (okj && k < K) ? gb_g[(size_t)pj * K + k] : 0.0f;
            }
        }
        // ---- DG^T tile m, then dl; register i of tile m is component 32 m + tile_row(i, h)
        float* dl_r = dl_bh + (size_t)pr * K;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            f32x16 dg;
#pragma unroll
            for (int i = 0; i < 16; ++i) dg[i] = 0.0f;
            const float* srow = sS + (32 * m + col) * Ws;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) dg = mfma_f32(srow[32 * n + tile_row(i, h)], x[n][i], dg);
#pragma unroll
            for (int i = 0; i < 16; ++i) dg = mfma_f32(gbt[m][i], qt[i], dg);
            if (okr) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k0 = 32 * m + 8 * q + 4 * h;
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float dgz = fmaf(sZ[k0 + e], xz, dg[4 * q + e]);
                        o[e] = ga[m][4 * q + e] * (dgz - s);
                    }
                    if (vec_k && k0 < K) {
                        *reinterpret_cast<float4*>(dl_r + k0) = make_float4(o[0], o[1], o[2], o[3]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (k0 + e < K) dl_r[k0 + e] = o[e];
                    }
                }
            }
        }
        // ga is done with: the next chunk's rows go in now
        if (qc + 1 < nch) gamma_c(ga_g, pn, ga);
        // ---- St += gb^T W (rows k of tile m, columns 32 n + col), z += gb^T W[:, dv]; then
        //      tile m of gb^T is done with and takes tile m of the next chunk's gb
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                f32x16 u;
#pragma unroll
                for (int i = 0; i < 16; ++i) u[i] = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) u = mfma_f32(gbt[m][i], wa[n][i], u);
                float old_s[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) old_s[i] = sS[(32 * m + tile_row(i, h)) * Ws + 32 * n + col];
#pragma unroll
                for (int i = 0; i < 16; ++i) sS[(32 * m + tile_row(i, h)) * Ws + 32 * n + col] = old_s[i] + u[i];
            }
            float zp = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) zp = fmaf(gbt[m][i], wzj[i], zp);
            zp = sum_halves(zp);
            if (h == 0) sZ[32 * m + col] += zp;
            if (qc + 1 < nch) gamma_tile(gb_g, pn, m, gb[m]);
        }
    }
}

// The same chunk walk with the components split over two waves (K up to 256: wave w takes
// component tiles 4 w .. 4 w + 3), so that a workgroup's state is worked on by two SIMDs and
// two workgroups fit in a CU's LDS: each wave forms its components' part of P^T and READ0^T
// (contractions over the components), wave 1 hands its parts to wave 0 through LDS, wave 0
// adds them (wave 0's part first) and hands the sums back, and both then form PW^T, X^T,
// Q^T and s from the same sums (bitwise the same on both waves); DG^T, dl and the state
// update are per component, each wave its own tiles.  Two barriers per chunk.
template <int NTW>
struct CausalMf2 {
    static constexpr int MT = 8, MTH = 4, Kp = 32 * MT, Wv = 32 * NTW, Ws = Wv + 1;
    // exchange block: P^T part (16 floats per lane), READ0^T part (NTW x 16), r0z part (1)
    static constexpr int XF = 16 + 16 * NTW + 1;
    static size_t lds_bytes() { return ((size_t)Kp * Ws + Kp + (size_t)64 * XF) * sizeof(float); }
};

template <typename T, int PASS, int NTW>
__global__ void __launch_bounds__(128)
    bwd_causal_mfma2(const float* __restrict__ gamma, const T* __restrict__ v, const T* __restrict__ dout,
                     float* __restrict__ gnum, float* __restrict__ gden, float* __restrict__ dl,
                     T* __restrict__ dv_out, const float* __restrict__ start, int BH, int N, int K, int dv, float eps,
                     int SEG, int L) {
    extern __shared__ double smem_d[];
    using C = CausalMf2<NTW>;
    constexpr int MTH = C::MTH, Kp = C::Kp, Wv = C::Wv, Ws = C::Ws, XF = C::XF;
    float* sS = reinterpret_cast<float*>(smem_d);  // [Kp][Ws]: value columns
    float* sZ = sS + (size_t)Kp * Ws;               // [Kp]: the normaliser column
    float* sX = sZ + Kp;                            // [XF][64]: the exchange block
    const int W = dv + 1;                           // dv == Wv
    const int bs = blockIdx.x, bh = bs / SEG, seg = bs % SEG;
    const int l = threadIdx.x & 63, col = l & 31, h = l >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kb = 32 * MTH * wv;  // this wave's first component
    const float* st0 = start + ((size_t)bh * SEG + seg) * K * W;
    // each wave loads (and later updates) only its own components' state rows
    for (int e = l; e < 32 * MTH * Wv; e += 64) {
        const int k = kb + e / Wv, c = e % Wv;
        sS[k * Ws + c] = k < K ? st0[(size_t)k * W + c] : 0.0f;
    }
    for (int k = kb + l; k < kb + 32 * MTH; k += 64) sZ[k] = k < K ? st0[(size_t)k * W + dv] : 0.0f;
    const float* ga_g = gamma + ((size_t)(PASS == 1 ? 0 : BH) + bh) * N * K;  // the rows' own side
    const float* gb_g = gamma + ((size_t)(PASS == 1 ? BH : 0) + bh) * N * K;  // the weighted side
    const T* v_bh = v + (size_t)bh * N * dv;
    const T* do_bh = dout + (size_t)bh * N * dv;
    float* gnum_bh = gnum + (size_t)bh * N * dv;
    float* gden_bh = gden + (size_t)bh * N;
    float* dl_bh = dl + ((size_t)(PASS == 1 ? 0 : BH) + bh) * N * K;
    T* dvo_bh = dv_out + (size_t)bh * N * dv;
    const bool vec_k = (K & 3) == 0;
    const int i0 = seg * L, i1 = min(N, i0 + L);
    const int nch = (i1 - i0 + 31) / 32;
    auto wval = [&](int p, int c) -> float {
        if constexpr (PASS == 1) return Elem<T>::load(v_bh, (size_t)p * dv + c);
        else return gnum_bh[(size_t)p * dv + c];
    };
    auto wz = [&](int p) -> float {
        if constexpr (PASS == 1) return 1.0f;
        else return gden_bh[p];
    };
    // this lane's row p at its C-layout components kb + 32 m + 8 q + 4 h + (0..3) (zeros past K)
    auto gamma_tile = [&](const float* g, int p, int m, f32x16& out) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k0 = kb + 32 * m + 8 * q + 4 * h;
            if (vec_k && k0 < K) {
                const float4 x = *reinterpret_cast<const float4*>(g + (size_t)p * K + k0);
                out[4 * q] = x.x;
                out[4 * q + 1] = x.y;
                out[4 * q + 2] = x.z;
                out[4 * q + 3] = x.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) out[4 * q + e] = k0 + e < K ? g[(size_t)p * K + k0 + e] : 0.0f;
            }
        }
    };
    auto gamma_c = [&](const float* g, int p, f32x16 (&out)[MTH]) {
#pragma unroll
        for (int m = 0; m < MTH; ++m) gamma_tile(g, p, m, out[m]);
    };
    auto base_of = [&](int qc) { return PASS == 1 ? i0 + 32 * qc : i1 - 32 * (qc + 1); };
    f32x16 ga[MTH], gb[MTH];
    {
        const int b0 = base_of(0), p0 = min(max(b0 + col, i0), i1 - 1);
        gamma_c(ga_g, p0, ga);
        gamma_c(gb_g, p0, gb);
    }
    for (int qc = 0; qc < nch; ++qc) {
        const int base = base_of(qc);
        auto in_seg = [&](int r) { return base + r >= i0 && base + r < i1; };
        auto clampp = [&](int r) { return min(max(base + r, i0), i1 - 1); };
        const bool okr = in_seg(col);
        const int pr = clampp(col);
        const int nbase = base_of(qc + 1);
        const int pn = min(max(nbase + col, i0), i1 - 1);
        if (!okr) {
#pragma unroll
            for (int m = 0; m < MTH; ++m)
#pragma unroll
                for (int i = 0; i < 16; ++i) ga[m][i] = gb[m][i] = 0.0f;
        }
        // ---- this wave's parts of P^T = gb ga^T and READ0^T = St^T ga^T (and its z entry)
        f32x16 pt, rd0[NTW];
#pragma unroll
        for (int i = 0; i < 16; ++i) pt[i] = 0.0f;
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) rd0[n][i] = 0.0f;
#pragma unroll
        for (int m = 0; m < MTH; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) pt = mfma_f32(gb[m][i], ga[m][i], pt);
        // ---- W rows in the operand orders used below (loads in flight during READ0)
        float wa[NTW][16], wzj[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int pj = clampp(tile_row(i, h));
            wzj[i] = wz(pj);
#pragma unroll
            for (int n = 0; n < NTW; ++n) wa[n][i] = wval(pj, 32 * n + col);
        }
        float xrow[NTW][16];
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int c = 32 * n + tile_row(i, h);
                xrow[n][i] = PASS == 1 ? (float)Elem<T>::load(do_bh, (size_t)pr * dv + c)
                                       : (float)Elem<T>::load(v_bh, (size_t)pr * dv + c);
            }
        float r0z = 0.0f;
#pragma unroll
        for (int m = 0; m < MTH; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int k = kb + 32 * m + tile_row(i, h);
                const float* srow = sS + k * Ws + col;
#pragma unroll
                for (int n = 0; n < NTW; ++n) rd0[n] = mfma_f32(srow[32 * n], ga[m][i], rd0[n]);
                r0z = fmaf(ga[m][i], sZ[k], r0z);
            }
        // ---- exchange: wave 1's parts to wave 0, the sums (wave 0's part first) back
        if (wv == 1) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sX[i * 64 + l] = pt[i];
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) sX[(16 + 16 * n + i) * 64 + l] = rd0[n][i];
            sX[(XF - 1) * 64 + l] = r0z;
        }
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                pt[i] = pt[i] + sX[i * 64 + l];
                sX[i * 64 + l] = pt[i];
            }
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    rd0[n][i] = rd0[n][i] + sX[(16 + 16 * n + i) * 64 + l];
                    sX[(16 + 16 * n + i) * 64 + l] = rd0[n][i];
                }
            r0z = r0z + sX[(XF - 1) * 64 + l];
            sX[(XF - 1) * 64 + l] = r0z;
        }
        __syncthreads();
        if (wv == 1) {
#pragma unroll
            for (int i = 0; i < 16; ++i) pt[i] = sX[i * 64 + l];
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) rd0[n][i] = sX[(16 + 16 * n + i) * 64 + l];
            r0z = sX[(XF - 1) * 64 + l];
        }
        r0z = sum_halves(r0z);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = tile_row(i, h);
            if (!(PASS == 1 ? j <= col : j >= col)) pt[i] = 0.0f;
        }
        // ---- PW^T = W^T P^T (both waves, from the same sums)
        f32x16 pw[NTW];
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) pw[n][i] = 0.0f;
        float pwz = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
#pragma unroll
            for (int n = 0; n < NTW; ++n) pw[n] = mfma_f32(wa[n][i], pt[i], pw[n]);
            pwz = fmaf(pt[i], wzj[i], pwz);
        }
        pwz = sum_halves(pwz);
        // ---- X^T (the rows' outputs are stored by wave 0)
        f32x16 x[NTW];
        float xz;
        if constexpr (PASS == 1) {
            const float den = r0z + pwz + eps;
            float dot = 0.0f;
            const float(&dov)[NTW][16] = xrow;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) dot = fmaf(dov[n][i], (rd0[n][i] + pw[n][i]) / den, dot);
            const float gd = -sum_halves(dot) / den;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float g = okr ? dov[n][i] / den : 0.0f;
                    x[n][i] = g;
                    if (okr && wv == 0) gnum_bh[(size_t)pr * dv + 32 * n + tile_row(i, h)] = g;
                }
            xz = okr ? gd : 0.0f;
            if (okr && h == 0 && wv == 0) gden_bh[pr] = gd;
        } else {
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int c = 32 * n + tile_row(i, h);
                    if (okr && wv == 0) Elem<T>::store(dvo_bh, (size_t)pr * dv + c, rd0[n][i] + pw[n][i]);
                    x[n][i] = okr ? xrow[n][i] : 0.0f;
                }
            xz = okr ? 1.0f : 0.0f;
        }
        // ---- Q^T = W X^T, masked (both waves)
        f32x16 qt;
#pragma unroll
        for (int i = 0; i < 16; ++i) qt[i] = 0.0f;
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) qt = mfma_f32(wval(pr, 32 * n + tile_row(i, h)), x[n][i], qt);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = tile_row(i, h);
            qt[i] = (PASS == 1 ? j <= col : j >= col) ? fmaf(wzj[i], xz, qt[i]) : 0.0f;
        }
        // ---- s_r = X_r . READ0_r + Q_r . P_r (both waves, the same order)
        float sp = xz * r0z * 0.5f;
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) sp = fmaf(x[n][i], rd0[n][i], sp);
#pragma unroll
        for (int i = 0; i < 16; ++i) sp = fmaf(qt[i], pt[i], sp);
        const float s = sum_halves(sp);
        // ---- gb^T of this wave's tiles (reusing gb's registers)
        f32x16 (&gbt)[MTH] = gb;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int rj = tile_row(i, h);
            const bool okj = in_seg(rj);
            const int pj = clampp(rj);
#pragma unroll
            for (int m = 0; m < MTH; ++m) {
                const int k = kb + 32 * m + col;
                gbt[m][i] = (okj && k < K) ? gb_g[(size_t)pj * K + k] : 0.0f;
            }
        }
        // ---- DG^T of this wave's tiles, then dl
        float* dl_r = dl_bh + (size_t)pr * K;
#pragma unroll
        for (int m = 0; m < MTH; ++m) {
            f32x16 dg;
#pragma unroll
            for (int i = 0; i < 16; ++i) dg[i] = 0.0f;
            const float* srow = sS + (kb + 32 * m + col) * Ws;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) dg = mfma_f32(srow[32 * n + tile_row(i, h)], x[n][i], dg);
#pragma unroll
            for (int i = 0; i < 16; ++i) dg = mfma_f32(gbt[m][i], qt[i], dg);
            if (okr) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k0 = kb + 32 * m + 8 * q + 4 * h;
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float dgz = fmaf(sZ[k0 + e], xz, dg[4 * q + e]);
                        o[e] = ga[m][4 * q + e] * (dgz - s);
                    }
                    if (vec_k && k0 < K) {
                        *reinterpret_cast<float4*>(dl_r + k0) = make_float4(o[0], o[1], o[2], o[3]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (k0 + e < K) dl_r[k0 + e] = o[e];
                    }
                }
            }
        }
        if (qc + 1 < nch) gamma_c(ga_g, pn, ga);
        // ---- St += gb^T W, z += gb^T W[:, dv] over this wave's tiles
#pragma unroll
        for (int m = 0; m < MTH; ++m) {
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                f32x16 u;
#pragma unroll
                for (int i = 0; i < 16; ++i) u[i] = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) u = mfma_f32(gbt[m][i], wa[n][i], u);
                float old_s[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) old_s[i] = sS[(kb + 32 * m + tile_row(i, h)) * Ws + 32 * n + col];
#pragma unroll
                for (int i = 0; i < 16; ++i) sS[(kb + 32 * m + tile_row(i, h)) * Ws + 32 * n + col] = old_s[i] + u[i];
            }
            float zp = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) zp = fmaf(gbt[m][i], wzj[i], zp);
            zp = sum_halves(zp);
            if (h == 0) sZ[kb + 32 * m + col] += zp;
            if (qc + 1 < nch) gamma_tile(gb_g, pn, m, gb[m]);
        }
    }
}

// dx of both sides: dx[side][bh][i][d] = -sum_k dl_k (x_d - mu_kd) lam_kd = Q_d - x_d P_d with
// P_d = sum_k dl_k lam_kd and Q_d = sum_k dl_k mu_kd lam_kd: a tile of 64 rows of one (side, bh)
// and 64 dims per workgroup, the components in blocks of 32 staged in LDS (in A), each
// thread 16 dims of one row; the sums over k in component order.
// Grid (ceil(N / 64), 2 BH, ceil(d_r / 64)).
constexpr int kXR = 64, kXD = 64, kXK = 32;
template <typename T, typename A>
__global__ void __launch_bounds__(kBwdThreads)
    bwd_x(const T* __restrict__ qr, const T* __restrict__ kr, const float* __restrict__ mu,
          const double* __restrict__ lam, const A* __restrict__ dl, T* __restrict__ dqr, T* __restrict__ dkr,
          int BH, int H, int N, int K, int dr) {
    __shared__ A sdl[kXR][kXK + 1];
    __shared__ A sl[kXK][kXD + 1], sml[kXK][kXD + 1];
    const int t = threadIdx.x;
    const int i0 = blockIdx.x * kXR, sb = blockIdx.y, d0 = blockIdx.z * kXD;
    const int side = sb / BH, bh = sb % BH, h = bh % H;
    const A* dl_r = dl + ((size_t)side * BH + bh) * N * K;
    const float* mu_h = mu + (size_t)h * K * dr;
    const double* lam_h = lam + (size_t)h * K * dr;
    const int rl = t >> 2, dg = t & 3;
    A P[16], Q[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) P[j] = Q[j] = 0;
    for (int kb = 0; kb < K; kb += kXK) {
        for (int idx = t; idx < kXR * kXK; idx += kBwdThreads) {
            const int rr = idx / kXK, kk = idx % kXK;
            const int i = i0 + rr, k = kb + kk;
            sdl[rr][kk] = (i < N && k < K) ? dl_r[(size_t)i * K + k] : (A)0;
        }
        for (int idx = t; idx < kXK * kXD; idx += kBwdThreads) {
            const int kk = idx / kXD, dd = idx % kXD;
            const int k = kb + kk, d = d0 + dd;
            A lv = 0, mv = 0;
            if (k < K && d < dr) {
                const double l = lam_h[(size_t)k * dr + d];
                lv = (A)l;
                mv = (A)((double)mu_h[(size_t)k * dr + d] * l);
            }
            sl[kk][dd] = lv;
            sml[kk][dd] = mv;
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < kXK; ++kk) {
            const A g = sdl[rl][kk];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                P[j] += g * sl[kk][dg + 4 * j];
                Q[j] += g * sml[kk][dg + 4 * j];
            }
        }
        __syncthreads();
    }
    const int i = i0 + rl;
    if (i >= N) return;
    const T* x = (side == 0 ? qr : kr) + ((size_t)bh * N + i) * dr;
    T* dx = (side == 0 ? dqr : dkr) + ((size_t)bh * N + i) * dr;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int d = d0 + dg + 4 * j;
        if (d < dr) Elem<T>::store(dx, d, (float)(Q[j] - (A)Elem<T>::load(x, d) * P[j]));
    }
}

// dx of both sides on the matrix cores (bf16 inputs, float dl): per 32-row tile of one
// (side, bh), P^T = lam^T dl^T and Q^T = (mu lam)^T dl^T (d_r x 32 each) with
// v_mfma_f32_32x32x2_f32 over the components in blocks of 32; step i of a block contracts
// component kb + 8 (i / 4) + 4 h + i % 4 of lane half h, so the B operand is the lane's own
// dl register.  lam and mu lam of the head (float) sit in LDS as [32 ceil(K / 32)][32 NTD + 1].
// Grid (ceil(N / (128 kXTiles)), 2 BH); each wave takes kXTiles tiles of 32 rows, one after
// the other, against the one staged copy of lam and mu lam.
constexpr int kXTiles = 4;
template <typename T, int NTD>
__global__ void __launch_bounds__(kMfRowThreads)
    bwd_x_mfma(const T* __restrict__ qr, const T* __restrict__ kr, const float* __restrict__ mu,
               const double* __restrict__ lam, const float* __restrict__ dl, T* __restrict__ dqr, T* __restrict__ dkr,
               int BH, int H, int N, int K, int dr) {
    extern __shared__ double smem_d[];
    constexpr int Ds = 32 * NTD + 1;
    const int Kp = (K + 31) & ~31;
    float* sL = reinterpret_cast<float*>(smem_d);
    float* sM = sL + (size_t)Kp * Ds;
    const int t = threadIdx.x, l = t & 63, wv = t >> 6, col = l & 31, half = l >> 5;
    const int sb = blockIdx.y, side = sb / BH, bh = sb % BH, h = bh % H;
    const float* mu_h = mu + (size_t)h * K * dr;
    const double* lam_h = lam + (size_t)h * K * dr;
    for (int e = t; e < Kp * 32 * NTD; e += kMfRowThreads) {
        const int k = e / (32 * NTD), d = e % (32 * NTD);
        float lv = 0.0f, mv = 0.0f;
        if (k < K && d < dr) {
            const double lm = lam_h[(size_t)k * dr + d];
            lv = (float)lm;
            mv = (float)((double)mu_h[(size_t)k * dr + d] * lm);
        }
        sL[k * Ds + d] = lv;
        sM[k * Ds + d] = mv;
    }
    __syncthreads();
    for (int rt = 0; rt < kXTiles; ++rt) {
        const int row = blockIdx.x * (128 * kXTiles) + 128 * rt + 32 * wv + col;
        const bool ok = row < N;
        const size_t rr = (size_t)(ok ? row : N - 1);
        const float* dl_r = dl + (((size_t)side * BH + bh) * N + rr) * K;
        const bool vec_k = (K & 3) == 0;
        f32x16 P[NTD], Q[NTD];
#pragma unroll
        for (int n = 0; n < NTD; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) P[n][i] = Q[n][i] = 0.0f;
        for (int kb = 0; kb < Kp; kb += 32) {
            float g[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k0 = kb + 8 * q + 4 * half;
                if (vec_k && k0 < K) {
                    const float4 x = *reinterpret_cast<const float4*>(dl_r + k0);
                    g[4 * q] = x.x;
                    g[4 * q + 1] = x.y;
                    g[4 * q + 2] = x.z;
                    g[4 * q + 3] = x.w;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) g[4 * q + j] = k0 + j < K ? dl_r[k0 + j] : 0.0f;
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int k = kb + 8 * (i >> 2) + 4 * half + (i & 3);
#pragma unroll
                for (int n = 0; n < NTD; ++n) {
                    P[n] = mfma_f32(sL[k * Ds + 32 * n + col], g[i], P[n]);
                    Q[n] = mfma_f32(sM[k * Ds + 32 * n + col], g[i], Q[n]);
                }
            }
        }
        if (!ok) continue;
        const T* x = (side == 0 ? qr : kr) + ((size_t)bh * N + rr) * dr;
        T* dx = (side == 0 ? dqr : dkr) + ((size_t)bh * N + rr) * dr;
#pragma unroll
        for (int n = 0; n < NTD; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int d = 32 * n + 8 * (i >> 2) + 4 * half + (i & 3);
                if (d < dr) Elem<T>::store(dx, d, Q[n][i] - Elem<T>::load(x, d) * P[n][i]);
            }
    }
}

template <typename T, int NTD>
hipError_t launch_x_mfma_t(const Args& a, const BwdArgs& g, const double* lam, const float* dl) {
    const gma_desc& d = a.d;
    const int BH = d.B * d.H;
    const size_t lds = 2 * (size_t)((d.K + 31) & ~31) * (32 * NTD + 1) * sizeof(float);
    hipError_t e;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_x_mfma<T, NTD>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
        return e;
    const unsigned gx = (unsigned)((d.N + 128 * kXTiles - 1) / (128 * kXTiles));
    bwd_x_mfma<T, NTD><<<dim3(gx, (unsigned)(2 * BH)), dim3(kMfRowThreads), lds, a.stream>>>(
        static_cast<const T*>(a.qr), static_cast<const T*>(a.kr), a.mu, lam, dl, static_cast<T*>(g.dqr),
        static_cast<T*>(g.dkr), BH, d.H, d.N, d.K, d.d_r);
    return hipGetLastError();
}

// dx on the bf16 matrix cores (bf16 inputs, d_r <= 64): the same P^T = lam^T dl^T and
// Q^T = (mu lam)^T dl^T per 32-row tile, with every fp32 operand split exactly into a bf16
// pair (hi = bf16(v), lo = bf16(v - hi)) and each product formed as hi.hi + lo.hi + hi.lo on
// v_mfma_f32_32x32x16_bf16 (the dropped lo.lo is below 2^-16 of the product).  The A operand
// (lam and mu lam, as four bf16 pieces [lam hi, lam lo, (mu lam) hi, (mu lam) lo], each
// [32 NTD dims][KS components] per head) is prepared once per call by bwd_x_pieces and copied
// to LDS by each workgroup; the B operand is the lane's own dl row: 8 consecutive components
// per lane half and contraction step, split in registers.
__host__ __device__ constexpr int x_pieces_stride(int K) { return ((K + 15) & ~15) + 8; }
constexpr int kXSC = 4;  // contraction steps of 16 components per dl chunk

template <int NTD>
__global__ void __launch_bounds__(256)
    bwd_x_pieces(const float* __restrict__ mu, const double* __restrict__ lam, bf16_t* __restrict__ xp, int K, int dr) {
    const int h = blockIdx.y, KS = x_pieces_stride(K);
    const int e = blockIdx.x * 256 + threadIdx.x;  // (dim, component) of the head's pieces
    if (e >= 32 * NTD * KS) return;
    const int d = e / KS, k = e % KS;
    float lv = 0.0f, mv = 0.0f;
    if (k < K && d < dr) {
        const double lm = lam[((size_t)h * K + k) * dr + d];
        lv = (float)lm;
        mv = (float)((double)mu[((size_t)h * K + k) * dr + d] * lm);
    }
    const bf16_t lh = f32_to_bf16(lv), mh = f32_to_bf16(mv);
    const size_t piece = (size_t)32 * NTD * KS;
    bf16_t* dst = xp + (size_t)h * 4 * piece + e;
    dst[0] = lh;
    dst[piece] = f32_to_bf16(lv - bf16_to_f32(lh));
    dst[2 * piece] = mh;
    dst[3 * piece] = f32_to_bf16(mv - bf16_to_f32(mh));
}

template <typename T, int NTD, bool FAST>
__global__ void __launch_bounds__(kMfRowThreads)
    bwd_x_bf16(const T* __restrict__ qr, const T* __restrict__ kr, const bf16_t* __restrict__ xp,
               const float* __restrict__ dl, T* __restrict__ dqr, T* __restrict__ dkr, int BH, int H, int N, int K,
               int dr) {
    extern __shared__ double smem_d[];
    bf16_t* sP = reinterpret_cast<bf16_t*>(smem_d);  // [4][32 NTD][KS]
    const int KS = x_pieces_stride(K), K16 = (K + 15) & ~15;
    const size_t piece = (size_t)32 * NTD * KS;
    const int t = threadIdx.x, l = t & 63, wv = t >> 6, col = l & 31, half = l >> 5;
    const int sb = blockIdx.y, side = sb / BH, bh = sb % BH, h = bh % H;
    {
        const uint4* src = reinterpret_cast<const uint4*>(xp + (size_t)h * 4 * piece);
        uint4* dst = reinterpret_cast<uint4*>(sP);
        const int nvec = (int)(4 * piece / 8);
        for (int i = t; i < nvec; i += kMfRowThreads) dst[i] = src[i];
    }
    __syncthreads();
    const bool vec_k = (K & 3) == 0;
    for (int rt = 0; rt < kXTiles; ++rt) {
        const int row = blockIdx.x * (128 * kXTiles) + 128 * rt + 32 * wv + col;
        const bool ok = row < N;
        const size_t rr = (size_t)(ok ? row : N - 1);
        const float* dl_r = dl + (((size_t)side * BH + bh) * N + rr) * K;
        f32x16 P[NTD], Q[NTD];
#pragma unroll
        for (int n = 0; n < NTD; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) P[n][i] = Q[n][i] = 0.0f;
        // the row's dl in chunks of kXSC contraction steps, the next chunk's loads in flight
        // during this chunk's MFMAs (two register buffers, chunks taken in pairs)
        auto load_chunk = [&](int kb0, float (&gb)[kXSC][8]) {
#pragma unroll
            for (int sc = 0; sc < kXSC; ++sc)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int kq = kb0 + 16 * sc + 8 * half + 4 * q;
                    if (FAST || (vec_k && kq < K)) {
                        const float4 x = *reinterpret_cast<const float4*>(dl_r + kq);
                        gb[sc][4 * q] = x.x;
                        gb[sc][4 * q + 1] = x.y;
                        gb[sc][4 * q + 2] = x.z;
                        gb[sc][4 * q + 3] = x.w;
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) gb[sc][4 * q + j] = kq + j < K ? dl_r[kq + j] : 0.0f;
                    }
                }
        };
        auto run_chunk = [&](int kb0, const float (&gb)[kXSC][8]) {
#pragma unroll
            for (int sc = 0; sc < kXSC; ++sc) {
                const int kb = kb0 + 16 * sc;
                if (kb >= K16) break;
                const int k0 = kb + 8 * half;
                mf::u32x4 gh, gl;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    gh[j] = mf::pack_bf16(gb[sc][2 * j], gb[sc][2 * j + 1]);
                    gl[j] = mf::pack_bf16(gb[sc][2 * j] - mf::bf16lo_to_f32(gh[j]),
                                          gb[sc][2 * j + 1] - mf::bf16hi_to_f32(gh[j]));
                }
                const mf::bf16x8 bh8 = __builtin_bit_cast(mf::bf16x8, gh), bl8 = __builtin_bit_cast(mf::bf16x8, gl);
#pragma unroll
                for (int n = 0; n < NTD; ++n) {
                    const bf16_t* arow = sP + (size_t)(32 * n + col) * KS + k0;
                    const mf::bf16x8 lh = *reinterpret_cast<const mf::bf16x8*>(arow);
                    const mf::bf16x8 ll = *reinterpret_cast<const mf::bf16x8*>(arow + piece);
                    const mf::bf16x8 mh = *reinterpret_cast<const mf::bf16x8*>(arow + 2 * piece);
                    const mf::bf16x8 ml = *reinterpret_cast<const mf::bf16x8*>(arow + 3 * piece);
                    P[n] = mf::mfma(lh, bh8, P[n]);
                    Q[n] = mf::mfma(mh, bh8, Q[n]);
                    P[n] = mf::mfma(ll, bh8, P[n]);
                    Q[n] = mf::mfma(ml, bh8, Q[n]);
                    P[n] = mf::mfma(lh, bl8, P[n]);
                    Q[n] = mf::mfma(mh, bl8, Q[n]);
                }
            }
        };
        float ga[kXSC][8], gb[kXSC][8];
        load_chunk(0, ga);
        for (int kb0 = 0; kb0 < K16; kb0 += 32 * kXSC) {
            if (kb0 + 16 * kXSC < K16) load_chunk(kb0 + 16 * kXSC, gb);
            run_chunk(kb0, ga);
            if (kb0 + 16 * kXSC >= K16) break;
            if (kb0 + 32 * kXSC < K16) load_chunk(kb0 + 32 * kXSC, ga);
            run_chunk(kb0 + 16 * kXSC, gb);
        }
        if (!ok) continue;
        const T* x = (side == 0 ? qr : kr) + ((size_t)bh * N + rr) * dr;
        T* dx = (side == 0 ? dqr : dkr) + ((size_t)bh * N + rr) * dr;
        if constexpr (FAST) {
            // d_r = 32 NTD: every group of 4 dims is whole, 8-byte loads and stores
            uint2 xv[NTD][4];
#pragma unroll
            for (int n = 0; n < NTD; ++n)
#pragma unroll
                for (int q = 0; q < 4; ++q) xv[n][q] = *reinterpret_cast<const uint2*>(x + 32 * n + 8 * q + 4 * half);
#pragma unroll
            for (int n = 0; n < NTD; ++n)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint2 u = xv[n][q];
                    const float x0 = mf::bf16lo_to_f32(u.x), x1 = mf::bf16hi_to_f32(u.x);
                    const float x2 = mf::bf16lo_to_f32(u.y), x3 = mf::bf16hi_to_f32(u.y);
                    uint2 o;
                    o.x = mf::pack_bf16(Q[n][4 * q] - x0 * P[n][4 * q], Q[n][4 * q + 1] - x1 * P[n][4 * q + 1]);
                    o.y = mf::pack_bf16(Q[n][4 * q + 2] - x2 * P[n][4 * q + 2], Q[n][4 * q + 3] - x3 * P[n][4 * q + 3]);
                    *reinterpret_cast<uint2*>(dx + 32 * n + 8 * q + 4 * half) = o;
                }
        } else {
#pragma unroll
            for (int n = 0; n < NTD; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int d = 32 * n + 8 * (i >> 2) + 4 * half + (i & 3);
                    if (d < dr) Elem<T>::store(dx, d, Q[n][i] - Elem<T>::load(x, d) * P[n][i]);
                }
        }
    }
}

// LDS bytes of bwd_x_bf16 (0: the shape is not taken: d_r > 64).
size_t x_bf16_lds(const gma_desc& d) {
    const int ntd = (d.d_r + 31) / 32;
    if (ntd > 2) return 0;
    const size_t lds = 4 * (size_t)(32 * ntd) * x_pieces_stride(d.K) * sizeof(bf16_t);
    return lds <= kScanLdsMax ? lds : 0;
}
size_t x_bf16_pieces_bytes(const gma_desc& d) {
    const int ntd = (d.d_r + 31) / 32;
    return (size_t)d.H * 4 * (32 * ntd) * x_pieces_stride(d.K) * sizeof(bf16_t);
}

template <typename T, int NTD>
hipError_t launch_x_bf16_t(const Args& a, const BwdArgs& g, const double* lam, const float* dl, bf16_t* xp) {
    const gma_desc& d = a.d;
    const int BH = d.B * d.H;
    const int KS = x_pieces_stride(d.K);
    bwd_x_pieces<NTD><<<dim3((unsigned)((32 * NTD * KS + 255) / 256), (unsigned)d.H), dim3(256), 0, a.stream>>>(
        a.mu, lam, xp, d.K, d.d_r);
    hipError_t e;
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t lds = 4 * (size_t)(32 * NTD) * KS * sizeof(bf16_t);
    // whole 16-component steps and whole 4-dim groups: unconditional loads and stores
    const bool fast = d.K % 16 == 0 && d.d_r == 32 * NTD;
    auto kern = fast ? &bwd_x_bf16<T, NTD, true> : &bwd_x_bf16<T, NTD, false>;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds)) != hipSuccess)
        return e;
    const unsigned gx = (unsigned)((d.N + 128 * kXTiles - 1) / (128 * kXTiles));
    kern<<<dim3(gx, (unsigned)(2 * BH)), dim3(kMfRowThreads), lds, a.stream>>>(
        static_cast<const T*>(a.qr), static_cast<const T*>(a.kr), xp, dl, static_cast<T*>(g.dqr),
        static_cast<T*>(g.dkr), BH, d.H, d.N, d.K, d.d_r);
    return hipGetLastError();
}

// LDS bytes of bwd_x_mfma (0: the shape is not taken).
size_t x_mfma_lds(const gma_desc& d) {
    const int ntd = (d.d_r + 31) / 32;
    if (ntd > 4) return 0;
    const size_t lds = 2 * (size_t)((d.K + 31) & ~31) * (32 * ntd + 1) * sizeof(float);
    return lds <= kScanLdsMax ? lds : 0;
}

// Parameter-gradient sums of chunk c of head h's 2 B N rows (side, b, i in that order), for a
// tile of 32 components x 64 dims: S0_k = sum dl_k, S1_kd = sum dl_k x_d, S2_kd = sum dl_k x_d^2
// (in A, over the chunk's rows in order; rows staged 64 at a time in LDS).  Each thread owns one
// component and 8 dims.  Grid (ceil(K / 32) ceil(d_r / 64), H, chunks).
constexpr int kPK = 32, kPD = 64, kPR = 64;
template <typename T, typename A>
__global__ void __launch_bounds__(kBwdThreads)
    bwd_param_part(const T* __restrict__ qr, const T* __restrict__ kr, const A* __restrict__ dl,
                   double* __restrict__ p1, double* __restrict__ p2, double* __restrict__ p0, int B, int H, int N,
                   int K, int dr, int per_chunk) {
    __shared__ A sdl[kPR][kPK + 1];
    __shared__ A sx[kPR][kPD + 1];
    const int t = threadIdx.x;
    const int nkt = (K + kPK - 1) / kPK;
    const int k0 = (blockIdx.x % nkt) * kPK, d0 = (blockIdx.x / nkt) * kPD;
    const int h = blockIdx.y, c = blockIdx.z;
    const int BH = B * H, BN = B * N;
    const int total = 2 * BN;
    const int u0 = c * per_chunk, u1 = min(total, u0 + per_chunk);
    const int kl = t >> 3, dg = t & 7;
    A s0 = 0, s1[8], s2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s1[j] = s2[j] = 0;
    // row u of the head -> (side, flat row of dl [side][BH][N], row of x [BH][N])
    auto rows_of = [&](int u, size_t& dl_row, size_t& x_row, int& side) {
        side = u / BN;
        const int rem = u - side * BN;
        const int b = rem / N, i = rem - b * N;
        x_row = (size_t)(b * H + h) * N + i;
        dl_row = (size_t)side * BH * N + x_row;
    };
    for (int ub = u0; ub < u1; ub += kPR) {
        for (int idx = t; idx < kPR * kPK; idx += kBwdThreads) {
            const int rr = idx / kPK, kk = idx % kPK;
            const int u = ub + rr, k = k0 + kk;
            A g = 0;
            if (u < u1 && k < K) {
                size_t dr_, xr_;
                int sd;
                rows_of(u, dr_, xr_, sd);
                g = dl[dr_ * K + k];
            }
            sdl[rr][kk] = g;
        }
        for (int idx = t; idx < kPR * kPD; idx += kBwdThreads) {
            const int rr = idx / kPD, dd = idx % kPD;
            const int u = ub + rr, d = d0 + dd;
            A xv = 0;
            if (u < u1 && d < dr) {
                size_t dr_, xr_;
                int sd;
                rows_of(u, dr_, xr_, sd);
                xv = (A)Elem<T>::load(sd == 0 ? qr : kr, xr_ * dr + d);
            }
            sx[rr][dd] = xv;
        }
        __syncthreads();
#pragma unroll 4
        for (int rr = 0; rr < kPR; ++rr) {
            const A g = sdl[rr][kl];
            s0 += g;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const A xv = sx[rr][dg + 8 * j];
                const A gx = g * xv;
                s1[j] += gx;
                s2[j] += gx * xv;
            }
        }
        __syncthreads();
    }
    const int k = k0 + kl;
    if (k >= K) return;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int d = d0 + dg + 8 * j;
        if (d < dr) {
            const size_t o = ((size_t)c * H + h) * K * dr + (size_t)k * dr + d;
            p1[o] = (double)s1[j];
            p2[o] = (double)s2[j];
        }
    }
    if (d0 == 0 && dg == 0) p0[((size_t)c * H + h) * K + k] = (double)s0;
}

// The C chunk sums added in chunk order (double), one thread per (h, k, d):
// dmu = lam (S1 - mu S0), dvar = -lam S0 / 2 + lam^2 (S2 - 2 mu S1 + mu^2 S0) / 2,
// dvar_raw = dvar sigmoid(var_raw).  Grid (ceil(K d_r / 256), H).
__global__ void __launch_bounds__(kBwdThreads)
    bwd_param_final(const double* __restrict__ p1, const double* __restrict__ p2, const double* __restrict__ p0,
                    const float* __restrict__ mu, const double* __restrict__ lam, const float* __restrict__ var_raw,
                    float* __restrict__ dmu, float* __restrict__ dvar_raw, int H, int K, int dr, int C) {
    const int e = blockIdx.x * kBwdThreads + threadIdx.x, h = blockIdx.y;
    if (e >= K * dr) return;
    const int k = e / dr;
    double S0 = 0.0, S1 = 0.0, S2 = 0.0;
    for (int c = 0; c < C; ++c) {
        S0 += p0[((size_t)c * H + h) * K + k];
        S1 += p1[((size_t)c * H + h) * K * dr + e];
        S2 += p2[((size_t)c * H + h) * K * dr + e];
    }
    const size_t o = (size_t)h * K * dr + e;
    const double m = mu[o], l = lam[o], r = var_raw[o];
    dmu[o] = (float)(l * (S1 - m * S0));
    const double dvar = -0.5 * l * S0 + 0.5 * l * l * (S2 - 2.0 * m * S1 + m * m * S0);
    dvar_raw[o] = (float)(dvar / (1.0 + exp(-r)));
}

// One workgroup per head: dlog pi_k = S0_k (chunk sums in chunk order);
// dprior = dlog pi - pi sum dlog pi.
__global__ void __launch_bounds__(kBwdThreads)
    bwd_prior_final(const double* __restrict__ p0, const float* __restrict__ prior, float* __restrict__ dprior, int H,
                    int K, int C) {
    __shared__ double sdp[GMA_MAX_K];
    __shared__ double sred[3];
    const int h = blockIdx.x, t = threadIdx.x;
    for (int k = t; k < K; k += kBwdThreads) {
        double a = 0.0;
        for (int c = 0; c < C; ++c) a += p0[((size_t)c * H + h) * K + k];
        sdp[k] = a;
    }
    __syncthreads();
    if (t < 64) {
        // prior softmax: max, sum of exponentials, and the total of dlog pi, by the first wave
        // (lanes strided over k, then a fixed butterfly order: deterministic)
        double m = -INFINITY;
        for (int k = t; k < K; k += 64) m = fmax(m, (double)prior[(size_t)h * K + k]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
        double se = 0.0, tot = 0.0;
        for (int k = t; k < K; k += 64) {
            se += exp((double)prior[(size_t)h * K + k] - m);
            tot += sdp[k];
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            se += __shfl_xor(se, o, 64);
            tot += __shfl_xor(tot, o, 64);
        }
        if (t == 0) {
            sred[0] = m;
            sred[1] = se;
            sred[2] = tot;
        }
    }
    __syncthreads();
    for (int k = t; k < K; k += kBwdThreads) {
        const double pi = exp((double)prior[(size_t)h * K + k] - sred[0]) / sred[1];
        dprior[(size_t)h * K + k] = (float)(sdp[k] - pi * sred[2]);
    }
}

// Scratch of the rows kernel besides its state, and whether the state fits in LDS with it.
size_t acc_size(const gma_desc& d) { return d.dtype == GMA_F32 ? sizeof(double) : sizeof(float); }
size_t scan_scratch(const gma_desc& d) { return (2 * (size_t)d.K + 6 * ((size_t)d.d_v + 1) + 5) * acc_size(d); }
size_t scan_state(const gma_desc& d) { return (size_t)d.K * (d.d_v + 1) * acc_size(d); }
bool state_in_lds(const gma_desc& d) { return scan_state(d) + scan_scratch(d) <= kScanLdsMax; }

// Segments per head: about 2048 (head, segment) waves in all, at least 16 rows per segment,
// and the two per-segment state arrays bounded to ~256 MB.
void segments(const gma_desc& d, int& SEG, int& L) {
    const long BH = (long)d.B * d.H;
    long seg = BH > 0 ? (2048 + BH - 1) / BH : 1;
    const long by_rows = (d.N + 15) / 16;
    if (seg > by_rows) seg = by_rows;
    const long per = BH * (long)scan_state(d) * 2;
    while (seg > 1 && per * seg > (256l << 20)) seg >>= 1;
    if (seg < 1) seg = 1;
    L = d.N > 0 ? (int)((d.N + seg - 1) / seg) : 1;
    SEG = d.N > 0 ? (d.N + L - 1) / L : 1;
}

// bf16 inputs whose routing rows the matrix-core responsibilities kernel covers take gamma
// from it (fp32 logits, float rows); float32 inputs and other shapes from the SIMT kernel.
bool resp_on_mfma(const gma_desc& d) {
    return d.dtype == GMA_BF16 && d.algo != GMA_ALGO_SIMT && mf::stats_supported(d);
}

struct BwdLayout {
    size_t lam, W, C, gamma, dl, gnum, gden, part, start, state, pmu, pvar, ppi, xp, total;
    int chunks, per_chunk, seg, seg_len;
};

BwdLayout bwd_layout(const gma_desc& d) {
    BwdLayout L{};
    const size_t BH = (size_t)d.B * d.H;
    const size_t as = acc_size(d);
    segments(d, L.seg, L.seg_len);
    size_t off = 0;
    L.lam = off;
    off += simt_param_bytes(d);
    if (resp_on_mfma(d)) {
        const mf::Geo g = mf::geometry(d);
        L.W = off;
        off += align_up((size_t)d.H * g.Kp * 4 * g.Dp * sizeof(bf16_t));
        L.C = off;
        off += align_up((size_t)d.H * g.Kp * sizeof(float));
    }
    L.gamma = off;
    off += align_up(2 * BH * d.N * d.K * as);
    L.dl = off;
    off += align_up(2 * BH * d.N * d.K * as);
    L.gnum = off;
    off += align_up(BH * d.N * d.d_v * as);
    L.gden = off;
    off += align_up(BH * d.N * as);
    const size_t segs = BH * L.seg * scan_state(d);
    L.part = off;
    off += align_up(segs);
    L.start = off;
    off += align_up(segs);
    L.state = off;
    if (!state_in_lds(d)) off += align_up(segs);
    const int rows = 2 * d.B * d.N;
    // chunks of rows for the parameter sums: about 512 workgroups of the matrix-core sums
    // (H chunks ceil(K / 128) of them), 16 to 64 chunks (each chunk's sums are read once more
    // by bwd_param_final: fewer chunks, less traffic there)
    const int kzs = (d.K + 127) / 128;
    int nch = 512 / (d.H * kzs > 0 ? d.H * kzs : 1);
    nch = nch < 16 ? 16 : (nch > kParamChunks ? kParamChunks : nch);
    L.chunks = rows > 0 ? (rows < nch ? rows : nch) : 0;
    L.per_chunk = L.chunks ? (rows + L.chunks - 1) / L.chunks : 0;
    const size_t nc = L.chunks ? L.chunks : 1;
    L.pmu = off;
    off += align_up(nc * d.H * d.K * d.d_r * sizeof(double));
    L.pvar = off;
    off += align_up(nc * d.H * d.K * d.d_r * sizeof(double));
    L.ppi = off;
    off += align_up(nc * d.H * d.K * sizeof(double));
    L.xp = off;
    if (d.dtype == GMA_BF16 && x_bf16_lds(d) > 0) off += align_up(x_bf16_pieces_bytes(d));
    L.total = off;
    return L;
}

// One pass over the rows: segment partials, their ordered starts, then the segment walks.
template <typename T, int PASS, int MT, int NTW>
hipError_t launch_causal_mfma_t(const Args& a, const BwdArgs& g, const float* gamma, float* gnum, float* gden,
                                float* dl, const float* start, const BwdLayout& L) {
    const gma_desc& d = a.d;
    const int BH = d.B * d.H;
    const size_t lds = CausalMf<MT, NTW>::lds_bytes();
    hipError_t e;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_causal_mfma<T, PASS, MT, NTW>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
        return e;
    bwd_causal_mfma<T, PASS, MT, NTW><<<dim3((unsigned)(BH * L.seg)), dim3(64), lds, a.stream>>>(
        gamma, static_cast<const T*>(a.v), static_cast<const T*>(g.dout), gnum, gden, dl, static_cast<T*>(g.dv),
        start, BH, d.N, d.K, d.d_v, a.eps, L.seg, L.seg_len);
    return hipGetLastError();
}

template <typename T, int PASS, int NTW>
hipError_t launch_causal_mfma2_t(const Args& a, const BwdArgs& g, const float* gamma, float* gnum, float* gden,
                                 float* dl, const float* start, const BwdLayout& L) {
    const gma_desc& d = a.d;
    const int BH = d.B * d.H;
    const size_t lds = CausalMf2<NTW>::lds_bytes();
    hipError_t e;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_causal_mfma2<T, PASS, NTW>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
        return e;
    bwd_causal_mfma2<T, PASS, NTW><<<dim3((unsigned)(BH * L.seg)), dim3(128), lds, a.stream>>>(
        gamma, static_cast<const T*>(a.v), static_cast<const T*>(g.dout), gnum, gden, dl, static_cast<T*>(g.dv),
        start, BH, d.N, d.K, d.d_v, a.eps, L.seg, L.seg_len);
    return hipGetLastError();
}

// MT = 32-component tiles (1, 2, 4 or 8), NTW = 32-column value tiles (1, 2 or 4: d_v = 32 NTW).
// Eight component tiles (128 < K <= 256) take the two-wave form.
template <typename T, int PASS>
hipError_t launch_causal_mfma(const Args& a, const BwdArgs& g, int MT, int NTW, const float* gamma, float* gnum,
                              float* gden, float* dl, const float* start, const BwdLayout& L) {
    if (MT == 8) {
        if (NTW == 1) return launch_causal_mfma2_t<T, PASS, 1>(a, g, gamma, gnum, gden, dl, start, L);
        if (NTW == 2) return launch_causal_mfma2_t<T, PASS, 2>(a, g, gamma, gnum, gden, dl, start, L);
        if (NTW == 4) return launch_causal_mfma2_t<T, PASS, 4>(a, g, gamma, gnum, gden, dl, start, L);
    }
#define GMA_BWD_CMF(mt, ntw) \
    if (MT == mt && NTW == ntw) return launch_causal_mfma_t<T, PASS, mt, ntw>(a, g, gamma, gnum, gden, dl, start, L);
    GMA_BWD_CMF(1, 1) GMA_BWD_CMF(1, 2) GMA_BWD_CMF(1, 4)
    GMA_BWD_CMF(2, 1) GMA_BWD_CMF(2, 2) GMA_BWD_CMF(2, 4)
    GMA_BWD_CMF(4, 1) GMA_BWD_CMF(4, 2) GMA_BWD_CMF(4, 4)
#undef GMA_BWD_CMF
    return hipErrorInvalidValue;
}

// Bidirectional rows on bf16 matrix cores (v_mfma_f32_32x32x16_bf16) with the fp32 operands
// in three exact bf16 pieces (split3_pair; the six products of order <= 2, or three against
// an operand exact in bf16: the dl epilogue differences dgamma and its row sum, so the
// products are kept to fp32 accuracy).  Each wave takes 32 rows at
// a time.  With G the rows' own gamma (32 x K) and St the head's total (K x W, W = d_v + 1):
// C1 = St^T G^T (W x 32) is pass 1's [num | den - eps] of every row, pass 2's [dv | .]; the
// per-row epilogue turns C1 into w (pass 1 [g_num | g_den], pass 2 [v | 1]); C2 = St w^T
// (K x 32) is dgamma of every row; then dl = gamma (dgamma - gamma . dgamma).  St is staged
// once per workgroup as three bf16 piece rows [Kp][Wp] (row stride 2 Wp + 16 bytes);
//   C1 = St^T G^T: A = St^T (lane: column c, 8 consecutive k: transposed LDS reads of St),
//                  B = G^T (lane: its row's gamma at 8 consecutive k, loaded from the row and
//                  split in registers);
//   C2 = St w^T:   A = St (lane: row k, 8 consecutive c: 16-byte LDS reads), B = w^T (the
//                  epilogue's w, C layout, regrouped to 8 consecutive columns per lane by one
//                  lane-half swap per register pair, then split).
// Gamma in the C layout for dl is loaded after C2.  Grid (BH ceil(N / RB)).
template <typename T, int PASS, int MT, int NTW>
__global__ void __launch_bounds__(kMfRowThreads, 2)
    bwd_bidir_bf16(const float* __restrict__ gamma, const T* __restrict__ v, const T* __restrict__ dout,
                   float* __restrict__ gnum, float* __restrict__ gden, float* __restrict__ dl, T* __restrict__ dv_out,
                   const float* __restrict__ start, int BH, int N, int K, int dv, float eps, int SEG, int RB) {
    extern __shared__ double smem_d[];
    constexpr int Kp = 32 * MT, Wp = 32 * NTW, SB = 2 * Wp + 16, KS = Kp / 16, CS = Wp / 16;
    unsigned char* sS1 = reinterpret_cast<unsigned char*>(smem_d);
    unsigned char* sS2 = sS1 + (size_t)Kp * SB;
    unsigned char* sS3 = sS2 + (size_t)Kp * SB;
    const int W = dv + 1;
    const int NB = (N + RB - 1) / RB;
    const int bs = blockIdx.x, bh = bs / NB, blk = bs % NB;
    const int t = threadIdx.x, l = t & 63, wv = t >> 6, col = l & 31, half = l >> 5;
    const float* st0 = start + (size_t)bh * SEG * K * W;  // slot 0: the head's total
    for (int e = t; e < Kp * Wp / 2; e += kMfRowThreads) {
        const int k = e / (Wp / 2), c = 2 * (e % (Wp / 2));
        const float v0 = (k < K && c < W) ? st0[(size_t)k * W + c] : 0.0f;
        const float v1 = (k < K && c + 1 < W) ? st0[(size_t)k * W + c + 1] : 0.0f;
        uint32_t a, b, d;
        split3_pair(v0, v1, a, b, d);
        *reinterpret_cast<uint32_t*>(sS1 + (size_t)k * SB + 2 * c) = a;
        *reinterpret_cast<uint32_t*>(sS2 + (size_t)k * SB + 2 * c) = b;
        *reinterpret_cast<uint32_t*>(sS3 + (size_t)k * SB + 2 * c) = d;
    }
    __syncthreads();
    const size_t side = PASS == 1 ? 0 : (size_t)BH;
    const float* g_bh = gamma + (side + bh) * N * K;
    float* dl_bh = dl + (side + bh) * N * K;
    const int i0 = blk * RB, i1 = min(N, i0 + RB);
    const bool vec_k = (K & 3) == 0;
    for (int tb = i0 + 32 * wv; tb < i1; tb += 32 * (kMfRowThreads / 64)) {
        const int row = tb + col;
        const bool ok = row < i1;
        const size_t rr = (size_t)(ok ? row : i0);  // rows past the segment read a valid row
        const float* grow = g_bh + rr * K;
        // ---- C1 = St^T G^T, G^T from this lane's row: k = 16 ks + 8 half + 0..7
        f32x16 c1[NTW];
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) c1[n][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k0 = 16 * ks + 8 * half;
            float x[8];
            if (vec_k) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float4 f = k0 + 4 * q < K ? *reinterpret_cast<const float4*>(grow + k0 + 4 * q)
                                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                    x[4 * q] = f.x;
                    x[4 * q + 1] = f.y;
                    x[4 * q + 2] = f.z;
                    x[4 * q + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = k0 + j < K ? grow[k0 + j] : 0.0f;
            }
            mf::u32x4 q1, q2, q3;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t a, b, d;
                split3_pair(x[2 * j], x[2 * j + 1], a, b, d);
                q1[j] = a;
                q2[j] = b;
                q3[j] = d;
            }
            const mf::bf16x8 g1 = __builtin_bit_cast(mf::bf16x8, q1), g2 = __builtin_bit_cast(mf::bf16x8, q2),
                             g3 = __builtin_bit_cast(mf::bf16x8, q3);
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                const mf::bf16x8 a1 = mf::lds_frag_tr(sS1, SB, 16 * ks, 32 * n);
                const mf::bf16x8 a2 = mf::lds_frag_tr(sS2, SB, 16 * ks, 32 * n);
                const mf::bf16x8 a3 = mf::lds_frag_tr(sS3, SB, 16 * ks, 32 * n);
                c1[n] = mf::mfma(a3, g1, c1[n]);
                c1[n] = mf::mfma(a2, g2, c1[n]);
                c1[n] = mf::mfma(a1, g3, c1[n]);
                c1[n] = mf::mfma(a2, g1, c1[n]);
                c1[n] = mf::mfma(a1, g2, c1[n]);
                c1[n] = mf::mfma(a1, g1, c1[n]);
            }
        }
        // epilogue: C1 register group q of tile n holds columns c0 = 32 n + 8 q + 4 h .. c0 + 3;
        // with d_v a multiple of 4 (VEC) a group is all value columns or none, and its row
        // values move as one 8-byte (bf16) or 16-byte (float) access
        const bool vec_v = (dv & 3) == 0;
        if constexpr (PASS == 1) {
            const T* do_r = dout + ((size_t)bh * N + rr) * dv;
            float dp = 0.0f;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * n + 8 * (i >> 2) + 4 * half + (i & 3) == dv) dp = c1[n][i];
            const float den = sum_halves(dp) + eps;
            const float rden = 1.0f / den;
            // dO of this lane's row at its C-layout columns (0 past d_v)
            float dov[NTW][16];
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c0 = 32 * n + 8 * q + 4 * half;
                    if (vec_v) {
                        const uint2 u = c0 < dv ? *reinterpret_cast<const uint2*>(do_r + c0) : make_uint2(0u, 0u);
                        dov[n][4 * q] = mf::bf16lo_to_f32(u.x);
                        dov[n][4 * q + 1] = mf::bf16hi_to_f32(u.x);
                        dov[n][4 * q + 2] = mf::bf16lo_to_f32(u.y);
                        dov[n][4 * q + 3] = mf::bf16hi_to_f32(u.y);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) dov[n][4 * q + j] = c0 + j < dv ? Elem<T>::load(do_r, c0 + j) : 0.0f;
                    }
                }
            float dot = 0.0f;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) dot += dov[n][i] * (c1[n][i] * rden);
            const float gd = -sum_halves(dot) * rden;
            float* gn = gnum + ((size_t)bh * N + rr) * dv;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c0 = 32 * n + 8 * q + 4 * half;
                    float wq[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c = c0 + j;
                        wq[j] = c < dv ? dov[n][4 * q + j] * rden : (c == dv ? gd : 0.0f);
                        c1[n][4 * q + j] = wq[j];
                    }
                    if (vec_v) {
                        if (ok && c0 < dv) *reinterpret_cast<float4*>(gn + c0) = make_float4(wq[0], wq[1], wq[2], wq[3]);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (ok && c0 + j < dv) gn[c0 + j] = wq[j];
                    }
                }
            if (ok && half == 0) gden[(size_t)bh * N + rr] = gd;
        } else {
            const T* v_r = v + ((size_t)bh * N + rr) * dv;
            T* dvo = dv_out + ((size_t)bh * N + rr) * dv;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c0 = 32 * n + 8 * q + 4 * half;
                    float cq[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) cq[j] = c1[n][4 * q + j];
                    if (vec_v) {
                        if (c0 < dv) {
                            if (ok)
                                *reinterpret_cast<uint2*>(dvo + c0) =
                                    make_uint2(mf::pack_bf16(cq[0], cq[1]), mf::pack_bf16(cq[2], cq[3]));
                            const uint2 u = *reinterpret_cast<const uint2*>(v_r + c0);
                            cq[0] = mf::bf16lo_to_f32(u.x);
                            cq[1] = mf::bf16hi_to_f32(u.x);
                            cq[2] = mf::bf16lo_to_f32(u.y);
                            cq[3] = mf::bf16hi_to_f32(u.y);
                        } else {
#pragma unroll
                            for (int j = 0; j < 4; ++j) cq[j] = c0 + j == dv ? 1.0f : 0.0f;
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int c = c0 + j;
                            if (ok && c < dv) Elem<T>::store(dvo, c, cq[j]);
                            cq[j] = c < dv ? Elem<T>::load(v_r, c) : (c == dv ? 1.0f : 0.0f);
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) c1[n][4 * q + j] = cq[j];
                }
        }
        // ---- C2 = St w^T: per 16-column block cs = 2 n + b, w regrouped so that each lane holds
        // columns 16 cs + 8 half + 0..7 of its row (registers 8 b .. 8 b + 7 of tile n hold
        // columns 16 b + 4 half + 0..3 and 16 b + 8 + 4 half + 0..3), then split
        f32x16 c2[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) c2[m][i] = 0.0f;
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) {
            const int n = cs >> 1, i0 = 8 * (cs & 1);
            // pass 1: w = [g_num | g_den] in three pieces; pass 2: w = [v | 1], exact in bf16
            uint32_t p1[4], p2[4], p3[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split3_pair(c1[n][i0 + 2 * j], c1[n][i0 + 2 * j + 1], p1[j], p2[j], p3[j]);
            // p[0], p[1]: columns +0..3 of this half's first group; p[2], p[3]: of its second
            auto regroup = [](const uint32_t (&p)[4]) {
                auto x = __builtin_amdgcn_permlane32_swap(p[0], p[2], false, false);
                auto y = __builtin_amdgcn_permlane32_swap(p[1], p[3], false, false);
                mf::u32x4 r;
                r[0] = x[0]; r[1] = y[0]; r[2] = x[1]; r[3] = y[1];
                return __builtin_bit_cast(mf::bf16x8, r);
            };
            const mf::bf16x8 w1 = regroup(p1);
            const mf::bf16x8 w2 = PASS == 1 ? regroup(p2) : w1;
            const mf::bf16x8 w3 = PASS == 1 ? regroup(p3) : w1;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const size_t off = (size_t)(32 * m + col) * SB + 2 * (16 * cs + 8 * half);
                const mf::bf16x8 a1 = *reinterpret_cast<const mf::bf16x8*>(sS1 + off);
                const mf::bf16x8 a2 = *reinterpret_cast<const mf::bf16x8*>(sS2 + off);
                const mf::bf16x8 a3 = *reinterpret_cast<const mf::bf16x8*>(sS3 + off);
                if (PASS == 1) {
                    c2[m] = mf::mfma(a3, w1, c2[m]);
                    c2[m] = mf::mfma(a2, w2, c2[m]);
                    c2[m] = mf::mfma(a1, w3, c2[m]);
                    c2[m] = mf::mfma(a2, w1, c2[m]);
                    c2[m] = mf::mfma(a1, w2, c2[m]);
                    c2[m] = mf::mfma(a1, w1, c2[m]);
                } else {
                    c2[m] = mf::mfma(a3, w1, c2[m]);
                    c2[m] = mf::mfma(a2, w1, c2[m]);
                    c2[m] = mf::mfma(a1, w1, c2[m]);
                }
            }
        }
        // gamma of this lane's row at its C-layout indices (zero past K), for dl
        f32x16 g[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k0 = 32 * m + 8 * q + 4 * half;
                if (vec_k && k0 < K) {
                    const float4 x = *reinterpret_cast<const float4*>(grow + k0);
                    g[m][4 * q] = x.x;
                    g[m][4 * q + 1] = x.y;
                    g[m][4 * q + 2] = x.z;
                    g[m][4 * q + 3] = x.w;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) g[m][4 * q + j] = k0 + j < K ? grow[k0 + j] : 0.0f;
                }
            }
        // dl = gamma (dgamma - gamma . dgamma)
        float sp = 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) sp += g[m][i] * c2[m][i];
        const float s = sum_halves(sp);
        if (ok) {
            float* dl_r = dl_bh + rr * K;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k0 = 32 * m + 8 * q + 4 * half;
                    float4 x;
                    x.x = g[m][4 * q] * (c2[m][4 * q] - s);
                    x.y = g[m][4 * q + 1] * (c2[m][4 * q + 1] - s);
                    x.z = g[m][4 * q + 2] * (c2[m][4 * q + 2] - s);
                    x.w = g[m][4 * q + 3] * (c2[m][4 * q + 3] - s);
                    if (vec_k && k0 < K) {
                        *reinterpret_cast<float4*>(dl_r + k0) = x;
                    } else {
                        if (k0 < K) dl_r[k0] = x.x;
                        if (k0 + 1 < K) dl_r[k0 + 1] = x.y;
                        if (k0 + 2 < K) dl_r[k0 + 2] = x.z;
                        if (k0 + 3 < K) dl_r[k0 + 3] = x.w;
                    }
                }
        }
    }
}

template <typename T, int PASS, int MT, int NTW>
hipError_t launch_bidir_bf16_t(const Args& a, const BwdArgs& g, const float* gamma, float* gnum, float* gden,
                               float* dl, const float* start, const BwdLayout& L) {
    const gma_desc& d = a.d;
    const int BH = d.B * d.H;
    const size_t lds = (size_t)3 * (32 * MT) * (2 * 32 * NTW + 16);
    hipError_t e;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_bidir_bf16<T, PASS, MT, NTW>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
        return e;
    const int nb = (d.N + kMfRowBlock - 1) / kMfRowBlock;
    bwd_bidir_bf16<T, PASS, MT, NTW><<<dim3((unsigned)(BH * nb)), dim3(kMfRowThreads), lds, a.stream>>>(
        gamma, static_cast<const T*>(a.v), static_cast<const T*>(g.dout), gnum, gden, dl, static_cast<T*>(g.dv),
        start, BH, d.N, d.K, d.d_v, a.eps, L.seg, kMfRowBlock);
    return hipGetLastError();
}

// MT = 32-component tiles (1, 2 or 4), NTW = 32-column tiles of the state (1, 2 or 3).
template <typename T, int PASS>
hipError_t launch_bidir_mfma(const Args& a, const BwdArgs& g, int MT, int NTW, const float* gamma, float* gnum,
                             float* gden, float* dl, const float* start, const BwdLayout& L) {
#define GMA_BWD_MF(mt, ntw) \
    if (MT == mt && NTW == ntw) return launch_bidir_bf16_t<T, PASS, mt, ntw>(a, g, gamma, gnum, gden, dl, start, L);
    GMA_BWD_MF(1, 1) GMA_BWD_MF(1, 2) GMA_BWD_MF(1, 3)
    GMA_BWD_MF(2, 1) GMA_BWD_MF(2, 2) GMA_BWD_MF(2, 3)
    GMA_BWD_MF(4, 1) GMA_BWD_MF(4, 2) GMA_BWD_MF(4, 3)
#undef GMA_BWD_MF
    return hipErrorInvalidValue;
}

// ---- split-bf16 row contractions (bf16 inputs).  A sum over rows of G[r][k] U[r][c] with
// fp32 G and U runs on v_mfma_f32_32x32x16_bf16: every fp32 value is staged as three bf16
// pieces p1 + p2 + p3 that add up to it exactly (split3_pair), and a product as the six
// piece products of order <= 2 (p1q1, p2q1, p1q2, p3q1, p2q2, p1q3: the dropped ones are
// below 2^-24 of it); an operand that is bf16 already (the value rows, the routing rows) is
// one piece, and its products with the three pieces of the other are exact.  Blocks of 32 rows are staged in LDS
// row-major as bf16 (row strides padded by 32 bytes) and read as MFMA fragments with the
// transposed LDS reads; the next block's values are loaded into registers while the current
// block's products run.

// Segment partials: part[bs] = G^T U over the segment's rows (K x W),
// G the weighting side's gamma rows (K columns, three pieces), U = [v | 1] (pass 1: bf16
// values, exact: three products) or [g_num | g_den] (pass 2: fp32, three pieces: six
// products).  The MT x NTW output tiles are dealt over the 4 waves.
// Staging in groups of 4 columns per thread; VEC (K and d_v multiples of 4): one 16-byte load
// of gamma / g_num or one 8-byte load of v per group.  Grid (BH * SEG).
template <typename T, int PASS, int MT, int NTW, bool VEC>
__global__ void __launch_bounds__(kMfRowThreads)
    bwd_seg_partial_bf16(const float* __restrict__ gamma, const T* __restrict__ v, const float* __restrict__ gnum,
                         const float* __restrict__ gden, float* __restrict__ part, int BH, int N, int K, int dv,
                         int SEG, int L) {
    static_assert(sizeof(T) == 2, "bf16 values");
    extern __shared__ double smem_d[];
    constexpr int GC = 32 * MT, UC = 32 * NTW;       // staged columns
    constexpr int GB = 2 * GC + 32, UB = 2 * UC + 32;  // row strides, bytes
    constexpr bool USPLIT = PASS == 2;                 // U in three pieces
    constexpr int NG = 32 * (GC / 4) / kMfRowThreads;  // column groups per thread and block
    constexpr int NU = 32 * (UC / 4) / kMfRowThreads;
    constexpr int kTiles = MT * NTW, kWaves = kMfRowThreads / 64, TPW = (kTiles + kWaves - 1) / kWaves;
    unsigned char* sG1 = reinterpret_cast<unsigned char*>(smem_d);
    unsigned char* sG2 = sG1 + 32 * GB;
    unsigned char* sG3 = sG2 + 32 * GB;
    unsigned char* sU1 = sG3 + 32 * GB;
    unsigned char* sU2 = sU1 + 32 * UB;
    unsigned char* sU3 = sU2 + 32 * UB;
    const int W = dv + 1;
    const int bs = blockIdx.x, bh = bs / SEG, seg = bs % SEG;
    const int t = threadIdx.x, l = t & 63, wv = t >> 6, col = l & 31, half = l >> 5;
    const int side = PASS == 1 ? 1 : 0;  // pass 1 weights by gamma_K, pass 2 by gamma_Q
    const float* g = gamma + ((size_t)side * BH + bh) * N * K;
    const T* v_bh = v + (size_t)bh * N * dv;
    const float* gnum_bh = gnum + (size_t)bh * N * dv;
    const float* gden_bh = gden + (size_t)bh * N;
    const int j0 = seg * L, j1 = min(N, j0 + L);
    float4 gv[NG];
    float4 uf[PASS == 2 ? NU : 1];  // pass 2: fp32 values
    uint2 ub[PASS == 1 ? NU : 1];   // pass 1: bf16 values (bits)
    auto load_blk = [&](int jb) {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int e = t + kMfRowThreads * i, r = e / (GC / 4), c = 4 * (e % (GC / 4)), j = jb + r;
            const float* gr = g + (size_t)min(j, N - 1) * K + c;
            const bool in = j < j1;
            if (VEC) {
                gv[i] = (in && c < K) ? *reinterpret_cast<const float4*>(gr) : make_float4(0.f, 0.f, 0.f, 0.f);
            } else {
                gv[i].x = (in && c < K) ? gr[0] : 0.0f;
                gv[i].y = (in && c + 1 < K) ? gr[1] : 0.0f;
                gv[i].z = (in && c + 2 < K) ? gr[2] : 0.0f;
                gv[i].w = (in && c + 3 < K) ? gr[3] : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int e = t + kMfRowThreads * i, r = e / (UC / 4), c = 4 * (e % (UC / 4)), j = jb + r;
            const size_t jj = (size_t)min(j, N - 1);
            const bool in = j < j1;
            if constexpr (PASS == 1) {
                // [v | 1]: value columns c < dv, the ones column at dv
                const T* vr = v_bh + jj * dv + c;
                uint32_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[q] = !in ? 0u : (c + q < dv ? (VEC ? 0u : (uint32_t)vr[q]) : (c + q == dv ? 0x3f80u : 0u));
                if (VEC && in && c < dv) {
                    const uint2 x = *reinterpret_cast<const uint2*>(vr);
                    ub[i] = x;
                } else {
                    ub[i] = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
                }
            } else {
                // [g_num | g_den]
                const float* gr = gnum_bh + jj * dv + c;
                float x[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    x[q] = !in ? 0.0f : (c + q < dv ? (VEC ? 0.0f : gr[q]) : (c + q == dv ? gden_bh[jj] : 0.0f));
                if (VEC && in && c < dv)
                    uf[i] = *reinterpret_cast<const float4*>(gr);
                else
                    uf[i] = make_float4(x[0], x[1], x[2], x[3]);
            }
        }
    };
    auto store_blk = [&]() {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int e = t + kMfRowThreads * i, r = e / (GC / 4), c = 4 * (e % (GC / 4));
            uint2 a, b, d;
            split3_pair(gv[i].x, gv[i].y, a.x, b.x, d.x);
            split3_pair(gv[i].z, gv[i].w, a.y, b.y, d.y);
            *reinterpret_cast<uint2*>(sG1 + r * GB + 2 * c) = a;
            *reinterpret_cast<uint2*>(sG2 + r * GB + 2 * c) = b;
            *reinterpret_cast<uint2*>(sG3 + r * GB + 2 * c) = d;
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int e = t + kMfRowThreads * i, r = e / (UC / 4), c = 4 * (e % (UC / 4));
            if constexpr (PASS == 1) {
                *reinterpret_cast<uint2*>(sU1 + r * UB + 2 * c) = ub[i];
            } else {
                uint2 a, b, d;
                split3_pair(uf[i].x, uf[i].y, a.x, b.x, d.x);
                split3_pair(uf[i].z, uf[i].w, a.y, b.y, d.y);
                *reinterpret_cast<uint2*>(sU1 + r * UB + 2 * c) = a;
                *reinterpret_cast<uint2*>(sU2 + r * UB + 2 * c) = b;
                *reinterpret_cast<uint2*>(sU3 + r * UB + 2 * c) = d;
            }
        }
    };
    f32x16 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[u][e] = 0.0f;
    if (j0 < j1) load_blk(j0);
    for (int jb = j0; jb < j1; jb += 32) {
        store_blk();
        __syncthreads();
        if (jb + 32 < j1) load_blk(jb + 32);  // in flight during the products
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int tau = wv + kWaves * u;
            if (tau < kTiles) {
                const int m = tau / NTW, n = tau % NTW;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const mf::bf16x8 a1 = mf::lds_frag_tr(sG1, GB, 16 * ks, 32 * m);
                    const mf::bf16x8 a2 = mf::lds_frag_tr(sG2, GB, 16 * ks, 32 * m);
                    const mf::bf16x8 a3 = mf::lds_frag_tr(sG3, GB, 16 * ks, 32 * m);
                    const mf::bf16x8 b1 = mf::lds_frag_tr(sU1, UB, 16 * ks, 32 * n);
                    if (USPLIT) {
                        const mf::bf16x8 b2 = mf::lds_frag_tr(sU2, UB, 16 * ks, 32 * n);
                        const mf::bf16x8 b3 = mf::lds_frag_tr(sU3, UB, 16 * ks, 32 * n);
                        acc[u] = mf::mfma(a3, b1, acc[u]);
                        acc[u] = mf::mfma(a2, b2, acc[u]);
                        acc[u] = mf::mfma(a1, b3, acc[u]);
                        acc[u] = mf::mfma(a2, b1, acc[u]);
                        acc[u] = mf::mfma(a1, b2, acc[u]);
                        acc[u] = mf::mfma(a1, b1, acc[u]);
                    } else {
                        acc[u] = mf::mfma(a3, b1, acc[u]);
                        acc[u] = mf::mfma(a2, b1, acc[u]);
                        acc[u] = mf::mfma(a1, b1, acc[u]);
                    }
                }
            }
        }
        __syncthreads();
    }
    float* out = part + (size_t)bs * K * W;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tau = wv + kWaves * u;
        if (tau < kTiles) {
            const int m = tau / NTW, n = tau % NTW, c = 32 * n + col;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int k = 32 * m + 8 * (e >> 2) + 4 * half + (e & 3);
                if (k < K && c < W) out[(size_t)k * W + c] = acc[u][e];
            }
        }
    }
}

template <int MT, int NTW>
constexpr size_t partial_bf16_lds() {
    return (size_t)32 * (3 * (64 * MT + 32) + 3 * (64 * NTW + 32));
}

template <typename T, int PASS, int MT, int NTW>
hipError_t launch_partial_bf16_t(const Args& a, const float* gamma, const float* gnum, const float* gden, float* part,
                                 const BwdLayout& L) {
    const gma_desc& d = a.d;
    constexpr size_t lds = partial_bf16_lds<MT, NTW>();
    const bool vec = d.K % 4 == 0 && d.d_v % 4 == 0;
    auto fn = vec ? &bwd_seg_partial_bf16<T, PASS, MT, NTW, true> : &bwd_seg_partial_bf16<T, PASS, MT, NTW, false>;
    hipError_t e;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds)) != hipSuccess)
        return e;
    fn<<<dim3((unsigned)(d.B * d.H * L.seg)), dim3(kMfRowThreads), lds, a.stream>>>(
        gamma, static_cast<const T*>(a.v), gnum, gden, part, d.B * d.H, d.N, d.K, d.d_v, L.seg, L.seg_len);
    return hipGetLastError();
}

template <typename T, int PASS>
hipError_t launch_partial_bf16(const Args& a, int MT, int NTW, const float* gamma, const float* gnum,
                               const float* gden, float* part, const BwdLayout& L) {
#define GMA_BWD_PB(mt, ntw) \
    if (MT == mt && NTW == ntw) return launch_partial_bf16_t<T, PASS, mt, ntw>(a, gamma, gnum, gden, part, L);
    GMA_BWD_PB(1, 1) GMA_BWD_PB(1, 2) GMA_BWD_PB(1, 3)
    GMA_BWD_PB(2, 1) GMA_BWD_PB(2, 2) GMA_BWD_PB(2, 3)
    GMA_BWD_PB(4, 1) GMA_BWD_PB(4, 2) GMA_BWD_PB(4, 3)
    GMA_BWD_PB(8, 1) GMA_BWD_PB(8, 2) GMA_BWD_PB(8, 3)
#undef GMA_BWD_PB
    return hipErrorInvalidValue;
}

template <typename T, typename A, int PASS>
hipError_t bwd_pass(const Args& a, const BwdArgs& g, const BwdLayout& L, A* gamma, A* dl, A* gnum, A* gden) {
    const gma_desc& d = a.d;
    const int BH = d.B * d.H;
    const int KW = d.K * (d.d_v + 1);
    A* part = reinterpret_cast<A*>(a.ws + L.part);
    A* start = reinterpret_cast<A*>(a.ws + L.start);
    A* st_global = state_in_lds(d) ? nullptr : reinterpret_cast<A*>(a.ws + L.state);
    const unsigned gx = (unsigned)((KW + kBwdThreads - 1) / kBwdThreads);
    const unsigned ptiles = (unsigned)(((d.K + kSK - 1) / kSK) * ((d.d_v + 1 + kSC - 1) / kSC));
    rec_begin(a, PASS == 1 ? "bwd_partial_1" : "bwd_partial_2");
    hipError_t e = hipSuccess;
    bool p_done = false;
    if constexpr (sizeof(A) == sizeof(float)) {
        // bf16 inputs: matrix-core partials when the tile shapes cover K and d_v + 1
        const int MT = d.K <= 32 ? 1 : (d.K <= 64 ? 2 : (d.K <= 128 ? 4 : (d.K <= 256 ? 8 : 0)));
        const int NTW = (d.d_v + 1 + 31) / 32;
        if (MT > 0 && NTW <= 3) {
            e = launch_partial_bf16<T, PASS>(a, MT, NTW, gamma, gnum, gden, part, L);
            p_done = true;
        }
    }
    if (!p_done) {
        bwd_seg_partial<T, A, PASS><<<dim3(ptiles, (unsigned)(BH * L.seg)), dim3(kBwdThreads), 0, a.stream>>>(
            gamma, static_cast<const T*>(a.v), gnum, gden, part, BH, d.N, d.K, d.d_v, L.seg, L.seg_len);
        e = hipGetLastError();
    }
    rec_end(a);
    if (e != hipSuccess) return e;
    rec_begin(a, PASS == 1 ? "bwd_start_1" : "bwd_start_2");
    bwd_seg_start<A, PASS><<<dim3(gx, (unsigned)BH), dim3(kBwdThreads), 0, a.stream>>>(part, start, d.K, d.d_v,
                                                                                       L.seg, a.causal);
    rec_end(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!a.causal) {
        if constexpr (sizeof(A) == sizeof(float)) {
            // bf16 inputs: 32-row tiles on the matrix cores when the state fits the tile shapes
            const int MT = d.K <= 32 ? 1 : (d.K <= 64 ? 2 : (d.K <= 128 ? 4 : 0));
            const int NTW = (d.d_v + 1 + 31) / 32;
            if (MT > 0 && NTW <= 3) {
                rec_begin(a, PASS == 1 ? "bwd_rows_1" : "bwd_rows_2");
                e = launch_bidir_mfma<T, PASS>(a, g, MT, NTW, gamma, gnum, gden, dl, start, L);
                rec_end(a);
                return e;
            }
        }
        // rows independent given the head's total: each wave walks its own rows
        const size_t lds = (size_t)kRowWaves * (2 * d.K + d.d_v + 1) * acc_size(d) + (st_global ? 0 : scan_state(d));
        if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_bidir_rows<T, A, PASS>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
            return e;
        rec_begin(a, PASS == 1 ? "bwd_rows_1" : "bwd_rows_2");
        bwd_bidir_rows<T, A, PASS><<<dim3((unsigned)(BH * L.seg)), dim3(kRowThreads), lds, a.stream>>>(
            gamma, static_cast<const T*>(a.v), static_cast<const T*>(g.dout), gnum, gden, dl, static_cast<T*>(g.dv),
            start, st_global ? start : nullptr, BH, d.N, d.K, d.d_v, a.eps, L.seg, L.seg_len);
        rec_end(a);
        return hipGetLastError();
    }
    if constexpr (sizeof(A) == sizeof(float)) {
        // bf16 inputs: the chunk walk on the matrix cores, one wave per segment
        const int MT = d.K <= 32 ? 1 : (d.K <= 64 ? 2 : (d.K <= 128 ? 4 : (d.K <= 256 ? 8 : 0)));
        const int NTW = d.d_v == 32 ? 1 : (d.d_v == 64 ? 2 : (d.d_v == 128 ? 4 : 0));
        if (MT > 0 && NTW > 0) {
            rec_begin(a, PASS == 1 ? "bwd_rows_1" : "bwd_rows_2");
            e = launch_causal_mfma<T, PASS>(a, g, MT, NTW, gamma, gnum, gden, dl, start, L);
            rec_end(a);
            return e;
        }
    }
    const size_t chunk_lds = scan_state(d) + (size_t)(2 * kCh * (d.K + 1) + 2 * kCh * (d.d_v + 2) + 2 * kCh * kCh) *
                                                 acc_size(d);
    if (chunk_lds <= kScanLdsMax) {
        // causal: the segment walked in chunks of kCh positions
        if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_seg_chunks<T, A, PASS>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)chunk_lds)) != hipSuccess)
            return e;
        rec_begin(a, PASS == 1 ? "bwd_rows_1" : "bwd_rows_2");
        bwd_seg_chunks<T, A, PASS><<<dim3((unsigned)(BH * L.seg)), dim3(kBwdThreads), chunk_lds, a.stream>>>(
            gamma, static_cast<const T*>(a.v), static_cast<const T*>(g.dout), gnum, gden, dl, static_cast<T*>(g.dv),
            start, BH, d.N, d.K, d.d_v, a.eps, L.seg, L.seg_len);
        rec_end(a);
        return hipGetLastError();
    }
    const size_t lds = scan_scratch(d) + (st_global ? 0 : scan_state(d));
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_seg_rows<T, A, PASS>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
        return e;
    rec_begin(a, PASS == 1 ? "bwd_rows_1" : "bwd_rows_2");
    bwd_seg_rows<T, A, PASS><<<dim3((unsigned)(BH * L.seg)), dim3(kRowThreads), lds, a.stream>>>(
        gamma, static_cast<const T*>(a.v), static_cast<const T*>(g.dout), gnum, gden, dl, static_cast<T*>(g.dv),
        start, st_global, BH, d.N, d.K, d.d_v, a.eps, a.causal, L.seg, L.seg_len);
    rec_end(a);
    return hipGetLastError();
}

// Parameter-gradient sums on bf16 matrix cores (bf16 inputs, float dl; the split-bf16 form
// of the row contractions above): for chunk c of head h, S1 = dl^T x, S2 = dl^T x^2 and
// S0 = dl^T 1 over the chunk's rows (both sides, all b), dl in three exact pieces, x exact
// in bf16 (S1, S0: exact products), x^2 split exactly into hi/lo (x^2 of a bf16 value has at
// most 16 significant bits; S2: the five products of order <= 2).  The final gradients
// difference these sums (dmu = lam (S1 - mu S0), ...), so they are kept to fp32 accuracy.
// The MT x NTD tiles of S1 and S2 are dealt over the 4 waves; the wave of tile (m, 0) also
// forms S0 of component tile m against a ones operand.  Staging in groups of 4 columns; VEC
// (K and d_r multiples of 4): one 16-byte load of dl and one 8-byte load of x per group.
// Workgroup z takes components [32 MT z, 32 MT (z + 1)).  Grid (H, chunks, ceil(K / (32 MT))).
template <typename T, int MT, int NTD, bool VEC>
__global__ void __launch_bounds__(kMfRowThreads, 2)
    bwd_param_bf16(const T* __restrict__ qr, const T* __restrict__ kr, const float* __restrict__ dl,
                   double* __restrict__ p1, double* __restrict__ p2, double* __restrict__ p0, int B, int H, int N,
                   int K, int dr, int per_chunk) {
    static_assert(sizeof(T) == 2, "bf16 routing rows");
    extern __shared__ double smem_d[];
    constexpr int GC = 32 * MT, XC = 32 * NTD;
    constexpr int GB = 2 * GC + 32, XB = 2 * XC + 32;
    constexpr int NG = 32 * (GC / 4) / kMfRowThreads, NX = (32 * (XC / 4) + kMfRowThreads - 1) / kMfRowThreads;
    constexpr int kTiles = MT * NTD, kWaves = kMfRowThreads / 64, TPW = (kTiles + kWaves - 1) / kWaves;
    unsigned char* sG1 = reinterpret_cast<unsigned char*>(smem_d);
    unsigned char* sG2 = sG1 + 32 * GB;
    unsigned char* sG3 = sG2 + 32 * GB;
    unsigned char* sX = sG3 + 32 * GB;
    unsigned char* sX2h = sX + 32 * XB;
    unsigned char* sX2l = sX2h + 32 * XB;
    const int t = threadIdx.x, l = t & 63, wv = t >> 6, col = l & 31, half = l >> 5;
    const int h = blockIdx.x, c = blockIdx.y, kz = 32 * MT * blockIdx.z;
    const int BH = B * H, BN = B * N;
    const int u0 = c * per_chunk, u1 = min(2 * BN, u0 + per_chunk);
    // row u of the chunk: side u / BN (queries, keys), batch and position; the row of dl is
    // side * BH * N + (b H + h) N + i, the routing row (b H + h) N + i of qr or kr
    auto rows = [&](int u, size_t& drow, const T*& xrow) {
        const int uu = min(u, u1 - 1);
        const int side = uu / BN, rem = uu - side * BN, b = rem / N, i = rem - b * N;
        const size_t r = ((size_t)b * H + h) * N + i;
        drow = (size_t)side * BH * N + r;
        xrow = (side == 0 ? qr : kr) + r * dr;
    };
    float4 gv[NG];
    uint2 xv[NX];
    auto load_blk = [&](int ub) {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int e = t + kMfRowThreads * i, r = e / (GC / 4), k = 4 * (e % (GC / 4)), u = ub + r;
            size_t drow;
            const T* xrow;
            rows(u, drow, xrow);
            const float* g = dl + drow * K + kz + k;
            const bool in = u < u1;
            if (VEC) {
                gv[i] = (in && kz + k < K) ? *reinterpret_cast<const float4*>(g) : make_float4(0.f, 0.f, 0.f, 0.f);
            } else {
                gv[i].x = (in && kz + k < K) ? g[0] : 0.0f;
                gv[i].y = (in && kz + k + 1 < K) ? g[1] : 0.0f;
                gv[i].z = (in && kz + k + 2 < K) ? g[2] : 0.0f;
                gv[i].w = (in && kz + k + 3 < K) ? g[3] : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int e = t + kMfRowThreads * i, r = e / (XC / 4), d = 4 * (e % (XC / 4)), u = ub + r;
            size_t drow;
            const T* xrow;
            rows(u, drow, xrow);
            const bool in = u < u1 && r < 32;
            if (VEC) {
                xv[i] = (in && d < dr) ? *reinterpret_cast<const uint2*>(xrow + d) : make_uint2(0u, 0u);
            } else {
                uint32_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = (in && d + q < dr) ? (uint32_t)xrow[d + q] : 0u;
                xv[i] = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
            }
        }
    };
    auto store_blk = [&]() {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int e = t + kMfRowThreads * i, r = e / (GC / 4), k = 4 * (e % (GC / 4));
            uint2 a, b, d;
            split3_pair(gv[i].x, gv[i].y, a.x, b.x, d.x);
            split3_pair(gv[i].z, gv[i].w, a.y, b.y, d.y);
            *reinterpret_cast<uint2*>(sG1 + r * GB + 2 * k) = a;
            *reinterpret_cast<uint2*>(sG2 + r * GB + 2 * k) = b;
            *reinterpret_cast<uint2*>(sG3 + r * GB + 2 * k) = d;
        }
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int e = t + kMfRowThreads * i, r = e / (XC / 4), d = 4 * (e % (XC / 4));
            if (r < 32) {
                const float x0 = mf::bf16lo_to_f32(xv[i].x), x1 = mf::bf16hi_to_f32(xv[i].x);
                const float x2 = mf::bf16lo_to_f32(xv[i].y), x3 = mf::bf16hi_to_f32(xv[i].y);
                uint2 hi, lo;
                split_pair(x0 * x0, x1 * x1, hi.x, lo.x);  // exact: x^2 has <= 16 significant bits
                split_pair(x2 * x2, x3 * x3, hi.y, lo.y);
                *reinterpret_cast<uint2*>(sX + r * XB + 2 * d) = xv[i];
                *reinterpret_cast<uint2*>(sX2h + r * XB + 2 * d) = hi;
                *reinterpret_cast<uint2*>(sX2l + r * XB + 2 * d) = lo;
            }
        }
    };
    f32x16 a1[TPW], a2[TPW], a0[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) a1[u][e] = a2[u][e] = a0[u][e] = 0.0f;
    mf::bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (short)0x3f80;
    if (u0 < u1) load_blk(u0);
    for (int ub = u0; ub < u1; ub += 32) {
        store_blk();
        __syncthreads();
        if (ub + 32 < u1) load_blk(ub + 32);  // in flight during the products
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int tau = wv + kWaves * u;
            if (tau < kTiles) {
                const int m = tau / NTD, n = tau % NTD;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const mf::bf16x8 g1 = mf::lds_frag_tr(sG1, GB, 16 * ks, 32 * m);
                    const mf::bf16x8 g2 = mf::lds_frag_tr(sG2, GB, 16 * ks, 32 * m);
                    const mf::bf16x8 g3 = mf::lds_frag_tr(sG3, GB, 16 * ks, 32 * m);
                    const mf::bf16x8 bx = mf::lds_frag_tr(sX, XB, 16 * ks, 32 * n);
                    const mf::bf16x8 b2h = mf::lds_frag_tr(sX2h, XB, 16 * ks, 32 * n);
                    const mf::bf16x8 b2l = mf::lds_frag_tr(sX2l, XB, 16 * ks, 32 * n);
                    a1[u] = mf::mfma(g3, bx, a1[u]);
                    a1[u] = mf::mfma(g2, bx, a1[u]);
                    a1[u] = mf::mfma(g1, bx, a1[u]);
                    a2[u] = mf::mfma(g3, b2h, a2[u]);
                    a2[u] = mf::mfma(g2, b2l, a2[u]);
                    a2[u] = mf::mfma(g2, b2h, a2[u]);
                    a2[u] = mf::mfma(g1, b2l, a2[u]);
                    a2[u] = mf::mfma(g1, b2h, a2[u]);
                    if (n == 0) {
                        a0[u] = mf::mfma(g3, ones, a0[u]);
                        a0[u] = mf::mfma(g2, ones, a0[u]);
                        a0[u] = mf::mfma(g1, ones, a0[u]);
                    }
                }
            }
        }
        __syncthreads();
    }
    const size_t base = ((size_t)c * H + h) * K;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tau = wv + kWaves * u;
        if (tau < kTiles) {
            const int m = tau / NTD, n = tau % NTD, d = 32 * n + col;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int k = kz + 32 * m + 8 * (e >> 2) + 4 * half + (e & 3);
                if (k < K && d < dr) {
                    p1[(base + k) * dr + d] = (double)a1[u][e];
                    p2[(base + k) * dr + d] = (double)a2[u][e];
                }
                if (n == 0 && col == 0 && k < K) p0[base + k] = (double)a0[u][e];
            }
        }
    }
}

template <typename T, int MT, int NTD>
hipError_t launch_param_bf16_t(const Args& a, const BwdLayout& L, const float* dl, double* pmu, double* pvar,
                               double* ppi) {
    const gma_desc& d = a.d;
    const size_t lds = (size_t)32 * (3 * (64 * MT + 32) + 3 * (64 * NTD + 32));
    const bool vec = d.K % 4 == 0 && d.d_r % 4 == 0;
    auto fn = vec ? &bwd_param_bf16<T, MT, NTD, true> : &bwd_param_bf16<T, MT, NTD, false>;
    hipError_t e;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds)) != hipSuccess)
        return e;
    const unsigned kzs = (unsigned)((d.K + 32 * MT - 1) / (32 * MT));
    fn<<<dim3((unsigned)d.H, (unsigned)L.chunks, kzs), dim3(kMfRowThreads), lds, a.stream>>>(
        static_cast<const T*>(a.qr), static_cast<const T*>(a.kr), dl, pmu, pvar, ppi, d.B, d.H, d.N, d.K, d.d_r,
        L.per_chunk);
    return hipGetLastError();
}

// MT = 32-component tiles per workgroup (1, 2, 4), NTD = 32-dim tiles (1, 2).
template <typename T>
hipError_t launch_param_bf16(const Args& a, int MT, int NTD, const BwdLayout& L, const float* dl, double* pmu,
                             double* pvar, double* ppi) {
#define GMA_BWD_PPB(mt, ntd) \
    if (MT == mt && NTD == ntd) return launch_param_bf16_t<T, mt, ntd>(a, L, dl, pmu, pvar, ppi);
    GMA_BWD_PPB(1, 1) GMA_BWD_PPB(1, 2) GMA_BWD_PPB(2, 1) GMA_BWD_PPB(2, 2)
    GMA_BWD_PPB(4, 1) GMA_BWD_PPB(4, 2)
#undef GMA_BWD_PPB
    return hipErrorInvalidValue;
}


template <typename T, typename A>
hipError_t backward_t(const Args& a, const BwdArgs& g) {
    const gma_desc& d = a.d;
    const BwdLayout L = bwd_layout(d);
    const int BH = d.B * d.H;
    double* lam = reinterpret_cast<double*>(a.ws + L.lam);
    double* cst = reinterpret_cast<double*>(a.ws + L.lam + align_up((size_t)d.H * d.K * d.d_r * sizeof(double)));
    A* gamma = reinterpret_cast<A*>(a.ws + L.gamma);
    A* dl = reinterpret_cast<A*>(a.ws + L.dl);
    A* gnum = reinterpret_cast<A*>(a.ws + L.gnum);
    A* gden = reinterpret_cast<A*>(a.ws + L.gden);
    double* pmu = reinterpret_cast<double*>(a.ws + L.pmu);
    double* pvar = reinterpret_cast<double*>(a.ws + L.pvar);
    double* ppi = reinterpret_cast<double*>(a.ws + L.ppi);
    hipError_t e;
    if ((e = simt_params(a, lam, cst)) != hipSuccess) return e;
    if (d.N > 0) {
        if constexpr (sizeof(A) == sizeof(float)) {
            if (resp_on_mfma(d)) {
                if ((e = mf::resp_rows(a, reinterpret_cast<bf16_t*>(a.ws + L.W), reinterpret_cast<float*>(a.ws + L.C),
                                       gamma)) != hipSuccess)
                    return e;
            } else if ((e = simt_gamma(a, gamma, lam, cst)) != hipSuccess) {
                return e;
            }
        } else if ((e = simt_gamma(a, gamma, lam, cst)) != hipSuccess) {
            return e;
        }
        if ((e = bwd_pass<T, A, 1>(a, g, L, gamma, dl, gnum, gden)) != hipSuccess) return e;
        if ((e = bwd_pass<T, A, 2>(a, g, L, gamma, dl, gnum, gden)) != hipSuccess) return e;
        rec_begin(a, "bwd_x");
        bool x_done = false;
        if constexpr (sizeof(A) == sizeof(float)) {
            if (x_bf16_lds(d) > 0) {
                bf16_t* xp = reinterpret_cast<bf16_t*>(a.ws + L.xp);
                e = (d.d_r + 31) / 32 == 1 ? launch_x_bf16_t<T, 1>(a, g, lam, dl, xp)
                                           : launch_x_bf16_t<T, 2>(a, g, lam, dl, xp);
                x_done = true;
            } else if (x_mfma_lds(d) > 0) {
                const int ntd = (d.d_r + 31) / 32;
                e = ntd == 1   ? launch_x_mfma_t<T, 1>(a, g, lam, dl)
                    : ntd == 2 ? launch_x_mfma_t<T, 2>(a, g, lam, dl)
                    : ntd == 3 ? launch_x_mfma_t<T, 3>(a, g, lam, dl)
                               : launch_x_mfma_t<T, 4>(a, g, lam, dl);
                x_done = true;
            }
        }
        if (!x_done) {
            bwd_x<T, A><<<dim3((unsigned)((d.N + kXR - 1) / kXR), (unsigned)(2 * BH), (unsigned)((d.d_r + kXD - 1) / kXD)),
                          dim3(kBwdThreads), 0, a.stream>>>(static_cast<const T*>(a.qr), static_cast<const T*>(a.kr),
                                                            a.mu, lam, dl, static_cast<T*>(g.dqr),
                                                            static_cast<T*>(g.dkr), BH, d.H, d.N, d.K, d.d_r);
            e = hipGetLastError();
        }
        rec_end(a);
        if (e != hipSuccess) return e;
        rec_begin(a, "bwd_param_part");
        bool p_done = false;
        if constexpr (sizeof(A) == sizeof(float)) {
            // bf16 inputs: matrix-core sums, at most 4 component tiles per workgroup (more
            // components are split over grid z: 16 tiles in one workgroup leave one wave per
            // SIMD and measured slower than the LDS-tiled kernel), d_r <= 64
            const int MT = d.K <= 32 ? 1 : (d.K <= 64 ? 2 : 4);
            const int NTD = (d.d_r + 31) / 32;
            if (NTD <= 2) {
                e = launch_param_bf16<T>(a, MT, NTD, L, dl, pmu, pvar, ppi);
                p_done = true;
            }
        }
        if (!p_done) {
            const int ptiles = ((d.K + kPK - 1) / kPK) * ((d.d_r + kPD - 1) / kPD);
            bwd_param_part<T, A><<<dim3((unsigned)ptiles, d.H, L.chunks), dim3(kBwdThreads), 0, a.stream>>>(
                static_cast<const T*>(a.qr), static_cast<const T*>(a.kr), dl, pmu, pvar, ppi, d.B, d.H, d.N, d.K,
                d.d_r, L.per_chunk);
            e = hipGetLastError();
        }
        rec_end(a);
        if (e != hipSuccess) return e;
    }
    rec_begin(a, "bwd_param_final");
    bwd_param_final<<<dim3((unsigned)((d.K * d.d_r + kBwdThreads - 1) / kBwdThreads), d.H), dim3(kBwdThreads), 0,
                      a.stream>>>(pmu, pvar, ppi, a.mu, lam, a.var_raw, g.dmu, g.dvar_raw, d.H, d.K, d.d_r, L.chunks);
    rec_end(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    rec_begin(a, "bwd_prior_final");
    bwd_prior_final<<<dim3(d.H), dim3(kBwdThreads), 0, a.stream>>>(ppi, a.prior, g.dprior, d.H, d.K, L.chunks);
    rec_end(a);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace(const gma_desc& d) { return bwd_layout(d).total; }

// The row passes index both sides of the batch's rows of a head, 2 B N, in int.
bool backward_supported(const gma_desc& d) {
    if (2 * (int64_t)d.B * d.N > INT32_MAX) return false;
    return scan_scratch(d) <= kScanLdsMax;
}

hipError_t backward_run(const Args& a, const BwdArgs& g) {
    return a.d.dtype == GMA_F32 ? backward_t<float, double>(a, g) : backward_t<bf16_t, float>(a, g);
}

}  // namespace gma
