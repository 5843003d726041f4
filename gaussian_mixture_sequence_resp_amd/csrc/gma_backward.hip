// Backward of the GMA forward mixer (bidirectional and causal), SIMT kernels.
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
//   bwd_scan       one workgroup per (b, h), the state K x (d_v + 1) in LDS (in the workspace
//                  when it does not fit; double for float32 inputs): pass 1 over the
//                  rows in order (forming the prefix, or the totals first) gives g_num, g_den
//                  and dl_Q; pass 2 over the rows in reverse (the suffix, or the totals) gives
//                  dv and dl_K
//   bwd_x          dqr, dkr: one thread per (side, row, dim), double accumulation over k
//   bwd_param_part per chunk of rows (both sides, all b), one thread per (h, k, d): partial
//                  dmu, dvar and dlog pi in double
//   bwd_param_final the partials summed in chunk order; dvar_raw, dprior
// Every sum has a fixed order: results are deterministic.
#include <math.h>

#include "gma_internal.h"
#include "gma_mfma_geo.h"
#include "gma_numeric.h"

namespace gma {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kParamChunks = 64;

// Per-head scan, in A: double for float32 inputs (gamma included: the chain rule cancels,
// e.g. R v_j + r against gamma . dgamma, and a sharp posterior's dl = gamma (dgamma - s) is
// far smaller than float's rounding of gamma times dgamma; the 1e-5 gate needs double);
// float for bf16.  st [K][W] (W = d_v + 1: the state, then reused for [R | r]) lives in LDS when it
// fits (st_global == null) and otherwise in the workspace at st_global + bh K W; row scratch
// in LDS: sgq [K], sgk [K], sdg [K], srow [W] (v_j or [g_num | g_den]), sred [2].
template <typename T, typename A>
__global__ void __launch_bounds__(kBwdThreads)
    bwd_scan(const A* __restrict__ gamma, const T* __restrict__ v, const T* __restrict__ dout,
             A* __restrict__ gnum, A* __restrict__ gden, A* __restrict__ dl, T* __restrict__ dv_out,
             A* st_global, int BH, int N, int K, int dv, float eps, int causal) {
    extern __shared__ double smem_d[];
    A* smem = reinterpret_cast<A*>(smem_d);
    const int W = dv + 1;
    const int bh = blockIdx.x, t = threadIdx.x;
    A* st = st_global ? st_global + (size_t)bh * K * W : smem;
    A* sgq = st_global ? smem : smem + (size_t)K * W;
    A* sgk = sgq + K;
    A* sdg = sgk + K;
    A* srow = sdg + K;
    A* sred = srow + W;
    const A* gq = gamma + (size_t)bh * N * K;
    const A* gk = gamma + ((size_t)BH + bh) * N * K;
    const T* v_bh = v + (size_t)bh * N * dv;
    const T* do_bh = dout + (size_t)bh * N * dv;
    A* gnum_bh = gnum + (size_t)bh * N * dv;
    A* gden_bh = gden + (size_t)bh * N;
    A* dlq = dl + (size_t)bh * N * K;
    A* dlk = dl + ((size_t)BH + bh) * N * K;
    T* dv_bh = dv_out + (size_t)bh * N * dv;

    for (int e = t; e < K * W; e += kBwdThreads) st[e] = 0.0f;
    __syncthreads();
    // st += g (x) [u | w] for row j (u = v_j or g_num_j; w = 1 or g_den_j), staged in srow
    auto add_row = [&](const A* g) {
        for (int e = t; e < K * W; e += kBwdThreads) st[e] += g[e / W] * srow[e % W];
    };
    auto stage_v = [&](int j) {
        for (int c = t; c < W; c += kBwdThreads) srow[c] = c < dv ? (A)Elem<T>::load(v_bh, (size_t)j * dv + c) : (A)1;
    };
    auto stage_g = [&](int j) {
        for (int c = t; c < W; c += kBwdThreads) srow[c] = c < dv ? gnum_bh[(size_t)j * dv + c] : gden_bh[j];
    };

    // ---- pass 1: rows in order
    if (!causal)
        for (int j = 0; j < N; ++j) {
            __syncthreads();
            stage_v(j);
            __syncthreads();
            add_row(gk + (size_t)j * K);
        }
    for (int i = 0; i < N; ++i) {
        __syncthreads();
        if (causal) stage_v(i);
        for (int k = t; k < K; k += kBwdThreads) sgq[k] = gq[(size_t)i * K + k];
        __syncthreads();
        if (causal) {
            add_row(gk + (size_t)i * K);
            __syncthreads();
        }
        // num (c < d_v) and den (c = d_v) of row i
        for (int c = t; c < W; c += kBwdThreads) {
            A a = 0;
            for (int k = 0; k < K; ++k) a += sgq[k] * st[(size_t)k * W + c];
            srow[c] = a;
        }
        __syncthreads();
        if (t == 0) {
            const A den = srow[dv] + (A)eps;
            A dot = 0;
            for (int c = 0; c < dv; ++c) dot += (A)Elem<T>::load(do_bh, (size_t)i * dv + c) * (srow[c] / den);
            sred[0] = den;
            sred[1] = -dot / den;
            gden_bh[i] = sred[1];
        }
        __syncthreads();
        const A den = sred[0], gd = sred[1];
        __syncthreads();
        for (int c = t; c < W; c += kBwdThreads) {
            const A g = c < dv ? (A)Elem<T>::load(do_bh, (size_t)i * dv + c) / den : gd;
            srow[c] = g;
            if (c < dv) gnum_bh[(size_t)i * dv + c] = g;
        }
        __syncthreads();
        // dgamma_Q = S g_num + z g_den, then the softmax backward
        for (int k = t; k < K; k += kBwdThreads) {
            A a = 0;
            for (int c = 0; c < W; ++c) a += st[(size_t)k * W + c] * srow[c];
            sdg[k] = a;
        }
        __syncthreads();
        if (t == 0) {
            A s = 0;
            for (int k = 0; k < K; ++k) s += sgq[k] * sdg[k];
            sred[0] = s;
        }
        __syncthreads();
        for (int k = t; k < K; k += kBwdThreads) dlq[(size_t)i * K + k] = sgq[k] * (sdg[k] - sred[0]);
    }

    // ---- pass 2: rows in reverse, st now [R | r]
    __syncthreads();
    for (int e = t; e < K * W; e += kBwdThreads) st[e] = 0.0f;
    if (!causal)
        for (int j = 0; j < N; ++j) {
            __syncthreads();
            stage_g(j);
            __syncthreads();
            add_row(gq + (size_t)j * K);
        }
    for (int j = N - 1; j >= 0; --j) {
        __syncthreads();
        if (causal) stage_g(j);
        for (int k = t; k < K; k += kBwdThreads) sgk[k] = gk[(size_t)j * K + k];
        __syncthreads();
        if (causal) {
            add_row(gq + (size_t)j * K);
            __syncthreads();
        }
        // dv_j = gamma_K,j R ; stage v_j for dgamma_K
        for (int c = t; c < dv; c += kBwdThreads) {
            A a = 0;
            for (int k = 0; k < K; ++k) a += sgk[k] * st[(size_t)k * W + c];
            Elem<T>::store(dv_bh, (size_t)j * dv + c, (float)a);
        }
        __syncthreads();
        stage_v(j);
        __syncthreads();
        // dgamma_K = R v_j + r  (srow[d_v] = 1 multiplies r)
        for (int k = t; k < K; k += kBwdThreads) {
            A a = 0;
            for (int c = 0; c < W; ++c) a += st[(size_t)k * W + c] * srow[c];
            sdg[k] = a;
        }
        __syncthreads();
        if (t == 0) {
            A s = 0;
            for (int k = 0; k < K; ++k) s += sgk[k] * sdg[k];
            sred[0] = s;
        }
        __syncthreads();
        for (int k = t; k < K; k += kBwdThreads) dlk[(size_t)j * K + k] = sgk[k] * (sdg[k] - sred[0]);
    }
}

// dx of both sides: dx[side][bh][i][d] = -sum_k dl (x_d - mu_kd) lam_kd.
template <typename T, typename A>
__global__ void __launch_bounds__(kBwdThreads)
    bwd_x(const T* __restrict__ qr, const T* __restrict__ kr, const float* __restrict__ mu,
          const double* __restrict__ lam, const A* __restrict__ dl, T* __restrict__ dqr, T* __restrict__ dkr,
          int BH, int H, int N, int K, int dr) {
    const size_t per_side = (size_t)BH * N * dr;
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= 2 * per_side) return;
    const int side = (int)(e / per_side);
    const size_t r = e % per_side;
    const size_t row = r / dr;  // bh * N + i
    const int d = (int)(r % dr);
    const int h = (int)((row / N) % H);
    const T* x = side == 0 ? qr : kr;
    const double xd = (double)Elem<T>::load(x, r);
    const A* dlr = dl + ((size_t)side * BH * N + row) * K;
    const float* mu_h = mu + (size_t)h * K * dr;
    const double* lam_h = lam + (size_t)h * K * dr;
    double a = 0.0;
    for (int k = 0; k < K; ++k) a -= (double)dlr[k] * (xd - (double)mu_h[(size_t)k * dr + d]) * lam_h[(size_t)k * dr + d];
    Elem<T>::store(side == 0 ? dqr : dkr, r, (float)a);
}

// Partial parameter gradients of chunk c of head h's 2 B N rows (side, b, i in that order):
// thread (k, d); the d = 0 thread of each k also sums dlog pi_k.
template <typename T, typename A>
__global__ void __launch_bounds__(kBwdThreads)
    bwd_param_part(const T* __restrict__ qr, const T* __restrict__ kr, const float* __restrict__ mu,
                   const double* __restrict__ lam, const A* __restrict__ dl, double* __restrict__ pmu,
                   double* __restrict__ pvar, double* __restrict__ ppi, int B, int H, int N, int K, int dr,
                   int per_chunk) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    const int h = blockIdx.y, c = blockIdx.z;
    if (e >= K * dr) return;
    const int k = e / dr, d = e % dr;
    const int BH = B * H;
    const int total = 2 * B * N;
    const int u0 = c * per_chunk, u1 = min(total, u0 + per_chunk);
    const double m = mu[(size_t)h * K * dr + e], l = lam[(size_t)h * K * dr + e];
    double am = 0.0, av = 0.0, ap = 0.0;
    for (int u = u0; u < u1; ++u) {
        const int side = u / (B * N), rem = u % (B * N);
        const int b = rem / N, i = rem % N;
        const size_t row = (size_t)(b * H + h) * N + i;
        const double g = dl[((size_t)side * BH * N + row) * K + k];
        const double diff = (double)Elem<T>::load(side == 0 ? qr : kr, row * dr + d) - m;
        am += g * diff * l;
        av += g * -0.5 * (l - diff * diff * l * l);
        ap += g;
    }
    const size_t o = ((size_t)c * H + h) * K * dr + e;
    pmu[o] = am;
    pvar[o] = av;
    if (d == 0) ppi[((size_t)c * H + h) * K + k] = ap;
}

// One workgroup per head: the C partials in chunk order; dvar_raw = dvar sigmoid(var_raw);
// dprior = dlog pi - pi sum dlog pi.
__global__ void __launch_bounds__(kBwdThreads)
    bwd_param_final(const double* __restrict__ pmu, const double* __restrict__ pvar, const double* __restrict__ ppi,
                    const float* __restrict__ var_raw, const float* __restrict__ prior, float* __restrict__ dmu,
                    float* __restrict__ dvar_raw, float* __restrict__ dprior, int H, int K, int dr, int C) {
    __shared__ double sdp[GMA_MAX_K];
    __shared__ double sred[3];
    const int h = blockIdx.x, t = threadIdx.x;
    for (int e = t; e < K * dr; e += kBwdThreads) {
        double am = 0.0, av = 0.0;
        for (int c = 0; c < C; ++c) {
            am += pmu[((size_t)c * H + h) * K * dr + e];
            av += pvar[((size_t)c * H + h) * K * dr + e];
        }
        const double r = var_raw[(size_t)h * K * dr + e];
        dmu[(size_t)h * K * dr + e] = (float)am;
        dvar_raw[(size_t)h * K * dr + e] = (float)(av / (1.0 + exp(-r)));
    }
    for (int k = t; k < K; k += kBwdThreads) {
        double a = 0.0;
        for (int c = 0; c < C; ++c) a += ppi[((size_t)c * H + h) * K + k];
        sdp[k] = a;
    }
    __syncthreads();
    if (t == 0) {
        // prior softmax: max, sum of exponentials, and the total of dlog pi, in order
        double m = prior[(size_t)h * K];
        for (int k = 1; k < K; ++k) m = fmax(m, (double)prior[(size_t)h * K + k]);
        double se = 0.0, tot = 0.0;
        for (int k = 0; k < K; ++k) {
            se += exp((double)prior[(size_t)h * K + k] - m);
            tot += sdp[k];
        }
        sred[0] = m;
        sred[1] = se;
        sred[2] = tot;
    }
    __syncthreads();
    for (int k = t; k < K; k += kBwdThreads) {
        const double pi = exp((double)prior[(size_t)h * K + k] - sred[0]) / sred[1];
        dprior[(size_t)h * K + k] = (float)(sdp[k] - pi * sred[2]);
    }
}

constexpr size_t kScanLdsMax = 150 * 1024;

// Scratch of the scan besides its state, and whether the state fits in LDS with it.
size_t acc_size(const gma_desc& d) { return d.dtype == GMA_F32 ? sizeof(double) : sizeof(float); }
size_t scan_scratch(const gma_desc& d) { return (3 * (size_t)d.K + (d.d_v + 1) + 2) * acc_size(d); }
size_t scan_state(const gma_desc& d) { return (size_t)d.K * (d.d_v + 1) * acc_size(d); }
bool state_in_lds(const gma_desc& d) { return scan_state(d) + scan_scratch(d) <= kScanLdsMax; }

// bf16 inputs whose routing rows the matrix-core responsibilities kernel covers take gamma
// from it (fp32 logits, float rows); float32 inputs and other shapes from the SIMT kernel.
bool resp_on_mfma(const gma_desc& d) {
    return d.dtype == GMA_BF16 && d.algo != GMA_ALGO_SIMT && mf::stats_supported(d);
}

struct BwdLayout {
    size_t lam, W, C, gamma, dl, gnum, gden, state, pmu, pvar, ppi, total;
    int chunks, per_chunk;
};

BwdLayout bwd_layout(const gma_desc& d) {
    BwdLayout L{};
    const size_t BH = (size_t)d.B * d.H;
    const size_t as = acc_size(d);
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
    L.state = off;
    if (!state_in_lds(d)) off += align_up(BH * scan_state(d));
    const int rows = 2 * d.B * d.N;
    L.chunks = rows > 0 ? (rows < kParamChunks ? rows : kParamChunks) : 0;
    L.per_chunk = L.chunks ? (rows + L.chunks - 1) / L.chunks : 0;
    const size_t nc = L.chunks ? L.chunks : 1;
    L.pmu = off;
    off += align_up(nc * d.H * d.K * d.d_r * sizeof(double));
    L.pvar = off;
    off += align_up(nc * d.H * d.K * d.d_r * sizeof(double));
    L.ppi = off;
    off += align_up(nc * d.H * d.K * sizeof(double));
    L.total = off;
    return L;
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
    A* st_global = state_in_lds(d) ? nullptr : reinterpret_cast<A*>(a.ws + L.state);
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
        const size_t lds = scan_scratch(d) + (st_global ? 0 : scan_state(d));
        if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_scan<T, A>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
            return e;
        rec_begin(a, "bwd_scan");
        bwd_scan<T, A><<<dim3(BH), dim3(kBwdThreads), lds, a.stream>>>(
            gamma, static_cast<const T*>(a.v), static_cast<const T*>(g.dout), gnum, gden, dl, static_cast<T*>(g.dv),
            st_global, BH, d.N, d.K, d.d_v, a.eps, a.causal);
        rec_end(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const size_t nx = 2 * (size_t)BH * d.N * d.d_r;
        rec_begin(a, "bwd_x");
        bwd_x<T, A><<<dim3((unsigned)((nx + kBwdThreads - 1) / kBwdThreads)), dim3(kBwdThreads), 0, a.stream>>>(
            static_cast<const T*>(a.qr), static_cast<const T*>(a.kr), a.mu, lam, dl, static_cast<T*>(g.dqr),
            static_cast<T*>(g.dkr), BH, d.H, d.N, d.K, d.d_r);
        rec_end(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        rec_begin(a, "bwd_param_part");
        bwd_param_part<T, A><<<dim3((d.K * d.d_r + kBwdThreads - 1) / kBwdThreads, d.H, L.chunks),
                               dim3(kBwdThreads), 0, a.stream>>>(static_cast<const T*>(a.qr),
                                                                  static_cast<const T*>(a.kr), a.mu, lam, dl, pmu,
                                                                  pvar, ppi, d.B, d.H, d.N, d.K, d.d_r, L.per_chunk);
        rec_end(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    rec_begin(a, "bwd_param_final");
    bwd_param_final<<<dim3(d.H), dim3(kBwdThreads), 0, a.stream>>>(pmu, pvar, ppi, a.var_raw, a.prior, g.dmu,
                                                                   g.dvar_raw, g.dprior, d.H, d.K, d.d_r, L.chunks);
    rec_end(a);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace(const gma_desc& d) { return bwd_layout(d).total; }

bool backward_supported(const gma_desc& d) { return scan_scratch(d) <= kScanLdsMax; }

hipError_t backward_run(const Args& a, const BwdArgs& g) {
    return a.d.dtype == GMA_F32 ? backward_t<float, double>(a, g) : backward_t<bf16_t, float>(a, g);
}

}  // namespace gma
