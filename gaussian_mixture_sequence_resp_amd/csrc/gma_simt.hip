// SIMT family of the GMA forward: plain fp32 arithmetic, one thread per output element.
//
// Method: Gaussian Mixture Attention (arXiv 2606.18283), "Core mechanism" items 1-3:
// GMM posterior responsibilities with softplus variances and softmax priors, the write
// phase Vt = Gamma_K^T V, Z = Gamma_K^T 1, the read phase O = Gamma_Q Vt / (Gamma_Q Z + eps)
// and the causal variant built on inclusive prefix sums.
//
// This family serves float32 inputs and any supported shape.  The log-density is taken in
// its direct form, l_k(x) = c_k - 1/2 sum_d (x_d - mu_kd)^2 / var_kd with
// c_k = log pi_k - 1/2 sum_d log var_kd; the constant (d/2) log 2 pi is the same for every
// component of a row and cancels in the softmax, so it is not computed.  Logits reach
// magnitudes of hundreds while the softmax needs them to ~1e-6 absolute for fp32 parity, so
// they are accumulated in double (parameters lam, c also kept in double); everything after
// the max-shift (exp, sums, write, read, scan) is float32.  Responsibilities
// are materialised in the workspace (float32 Gamma_Q [B,H,N,K] then Gamma_K [B,H,Nk,K]; Nk = N
// except in the cross variant), then the write and read phases
// (or the causal scan) consume them.  Every sum runs in ascending index order, so results
// are deterministic.
#include <math.h>

#include "gma_internal.h"
#include "gma_numeric.h"

namespace gma {
namespace {

constexpr int kBlock = 256;

// One wave per (h, k): lam[h,k,d] = 1/var, cst[h,k] = log pi_k - 1/2 sum_d log var_kd, in
// double; lanes over the routing dims (and over the head's K prior logits for its log-sum-
// exp), the sums over the wave in a fixed butterfly order (deterministic).  Blocks stride
// over the H K pairs (grid min(H K, 2^20)).
__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
__global__ void __launch_bounds__(64) params_kernel(const float* __restrict__ var_raw,
                                                    const float* __restrict__ prior, int H, int K, int dr,
                                                    float var_floor, double* __restrict__ lam,
                                                    double* __restrict__ cst) {
    const int lane = threadIdx.x;
    for (int64_t p = blockIdx.x; p < (int64_t)H * K; p += gridDim.x) {
        const int64_t h = p / K;
        const int k = (int)(p % K);
        const float* ph = prior + h * K;
        // log-sum-exp of the prior logits of this head (softmax priors)
        double pmax = -INFINITY;
        for (int j = lane; j < K; j += 64) pmax = fmax(pmax, (double)ph[j]);
        pmax = wave_max_d(pmax);
        double psum = 0.0;
        for (int j = lane; j < K; j += 64) psum += exp((double)ph[j] - pmax);
        const double lse = pmax + log(wave_sum_d(psum));
        double half_logdet = 0.0;
        for (int d = lane; d < dr; d += 64) {
            const size_t i = (size_t)p * dr + d;
            const double r = var_raw[i];
            const double var = fmax(r, 0.0) + log1p(exp(-fabs(r))) + (double)var_floor;
            lam[i] = 1.0 / var;
            half_logdet += 0.5 * log(var);
        }
        half_logdet = wave_sum_d(half_logdet);
        if (lane == 0) cst[p] = (double)ph[k] - lse - half_logdet;
    }
}

// One thread per routing row (side, b, h, n) of either side: Gamma_Q rows [b,h,n] (Nq per head)
// then Gamma_K rows (Nk per head), each = softmax_k l_k(x).
template <typename T, typename G>
__global__ void __launch_bounds__(kBlock) resp_kernel(const T* __restrict__ qr,
                                                      const T* __restrict__ kr,
                                                      const float* __restrict__ mu,
                                                      const double* __restrict__ lam,
                                                      const double* __restrict__ cst,
                                                      G* __restrict__ gamma, int* __restrict__ hard,
                                                      int BH, int H, int Nq, int Nk, int dr, int K, int nblk) {
    const int side = blockIdx.y;
    const int N = side == 0 ? Nq : Nk;
    const int bh = blockIdx.x / nblk;
    const int n = (blockIdx.x % nblk) * kBlock + threadIdx.x;
    if (n >= N) return;
    const int h = bh % H;
    const T* x = (side == 0 ? qr : kr) + ((size_t)bh * N + n) * dr;
    G* g = gamma + ((size_t)side * BH * Nq + (size_t)bh * N + n) * K;
    const float* mu_h = mu + (size_t)h * K * dr;
    const double* lam_h = lam + (size_t)h * K * dr;
    // pass 1: row max of the logits (double) and its component (the first one reaching it:
    // the hard assignment, written for the key side when `hard` is given), pass 2: shifted
    // logits -> exp (float)
    double m = -INFINITY;
    int best = 0;
    for (int k = 0; k < K; ++k) {
        double q = 0.0;
        for (int d = 0; d < dr; ++d) {
            const double diff = (double)Elem<T>::load(x, d) - (double)mu_h[(size_t)k * dr + d];
            q = fma(lam_h[(size_t)k * dr + d] * diff, diff, q);
        }
        const double l = cst[(size_t)h * K + k] - 0.5 * q;
        if (l > m) {
            m = l;
            best = k;
        }
    }
    if (hard && side == 1) hard[(size_t)bh * N + n] = best;
    for (int k = 0; k < K; ++k) {
        double q = 0.0;
        for (int d = 0; d < dr; ++d) {
            const double diff = (double)Elem<T>::load(x, d) - (double)mu_h[(size_t)k * dr + d];
            q = fma(lam_h[(size_t)k * dr + d] * diff, diff, q);
        }
        g[k] = (G)(cst[(size_t)h * K + k] - 0.5 * q - m);
    }
    G s = 0;
    for (int k = 0; k < K; ++k) {
        G e;
        if constexpr (sizeof(G) == 4)
            e = expf(g[k]);
        else
            e = exp(g[k]);
        g[k] = e;
        s += e;
    }
    const G inv = (G)1 / s;
    for (int k = 0; k < K; ++k) g[k] *= inv;
}

// Bidirectional write: mem[b,h,k,c] = sum_n gamma_K[n,k] * [v[n,c] | 1], c in [0, d_v].
template <typename T>
__global__ void __launch_bounds__(kBlock) write_kernel(const float* __restrict__ gk,
                                                       const T* __restrict__ v,
                                                       float* __restrict__ mem, int N, int K,
                                                       int dv, int nblk) {
    const int bh = blockIdx.x / nblk;
    const int idx = (blockIdx.x % nblk) * kBlock + threadIdx.x;
    const int W = dv + 1;
    if (idx >= K * W) return;
    const int k = idx / W, c = idx % W;
    const float* g = gk + (size_t)bh * N * K;
    const T* vv = v + (size_t)bh * N * dv;
    float acc = 0.0f;
    if (c < dv) {
        for (int n = 0; n < N; ++n) acc = fmaf(g[(size_t)n * K + k], Elem<T>::load(vv, (size_t)n * dv + c), acc);
    } else {
        for (int n = 0; n < N; ++n) acc += g[(size_t)n * K + k];
    }
    mem[((size_t)bh * K + k) * W + c] = acc;
}

// Bidirectional read: out[b,h,n,c] = sum_k gq[n,k] mem[k,c] / (sum_k gq[n,k] mem[k,dv] + eps).
template <typename T>
__global__ void __launch_bounds__(kBlock) read_kernel(const float* __restrict__ gq,
                                                      const float* __restrict__ mem,
                                                      T* __restrict__ out, int N, int K, int dv,
                                                      float eps, int nblk) {
    const int bh = blockIdx.x / nblk;
    const size_t idx = (size_t)(blockIdx.x % nblk) * kBlock + threadIdx.x;
    if (idx >= (size_t)N * dv) return;
    const int n = (int)(idx / dv), c = (int)(idx % dv);
    const int W = dv + 1;
    const float* g = gq + ((size_t)bh * N + n) * K;
    const float* m = mem + (size_t)bh * K * W;
    float num = 0.0f, den = 0.0f;
    for (int k = 0; k < K; ++k) {
        num = fmaf(g[k], m[(size_t)k * W + c], num);
        den = fmaf(g[k], m[(size_t)k * W + dv], den);
    }
    Elem<T>::store(out, ((size_t)bh * N + n) * dv + c, num / (den + eps));
}

// Causal scan, one block per (b, h).  The state [S | z] (K x (d_v+1), float32) lives in LDS;
// for each position i: state += gamma_K[i] (x) [v_i | 1] (inclusive), then
// out_i = gamma_Q[i] . S / (gamma_Q[i] . z + eps).
template <typename T>
__global__ void __launch_bounds__(kBlock) causal_kernel(const float* __restrict__ gq,
                                                        const float* __restrict__ gk,
                                                        const T* __restrict__ v,
                                                        T* __restrict__ out, int N, int K,
                                                        int dv, float eps) {
    extern __shared__ float smem[];
    const int W = dv + 1;
    float* state = smem;             // [K][W]
    float* res = smem + (size_t)K * W;  // [W]
    const int bh = blockIdx.x;
    const float* gqh = gq + (size_t)bh * N * K;
    const float* gkh = gk + (size_t)bh * N * K;
    const T* vh = v + (size_t)bh * N * dv;
    T* oh = out + (size_t)bh * N * dv;
    for (int i = threadIdx.x; i < K * W; i += kBlock) state[i] = 0.0f;
    __syncthreads();
    for (int n = 0; n < N; ++n) {
        for (int i = threadIdx.x; i < K * W; i += kBlock) {
            const int k = i / W, c = i % W;
            const float g = gkh[(size_t)n * K + k];
            state[i] = (c < dv) ? fmaf(g, Elem<T>::load(vh, (size_t)n * dv + c), state[i]) : state[i] + g;
        }
        __syncthreads();
        for (int c = threadIdx.x; c < W; c += kBlock) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) acc = fmaf(gqh[(size_t)n * K + k], state[(size_t)k * W + c], acc);
            res[c] = acc;
        }
        __syncthreads();
        for (int c = threadIdx.x; c < dv; c += kBlock)
            Elem<T>::store(oh, (size_t)n * dv + c, res[c] / (res[dv] + eps));
        __syncthreads();
    }
}

struct SimtLayout {
    size_t lam, cst, gamma, mem, total;
};

SimtLayout simt_layout(const gma_desc& d, int Nk) {
    SimtLayout L;
    const size_t BH = (size_t)d.B * d.H;
    size_t off = 0;
    L.lam = off;
    off += align_up((size_t)d.H * d.K * d.d_r * sizeof(double));
    L.cst = off;
    off += align_up((size_t)d.H * d.K * sizeof(double));
    L.gamma = off;
    off += align_up(BH * ((size_t)d.N + Nk) * d.K * sizeof(float));
    L.mem = off;
    off += align_up(BH * d.K * (d.d_v + 1) * sizeof(float));
    L.total = off;
    return L;
}

template <typename T>
hipError_t simt_forward_t(const Args& a) {
    const gma_desc& d = a.d;
    const SimtLayout L = simt_layout(d, a.Nk);
    double* lam = reinterpret_cast<double*>(a.ws + L.lam);
    double* cst = reinterpret_cast<double*>(a.ws + L.cst);
    float* gamma = a.gamma_out ? a.gamma_out : reinterpret_cast<float*>(a.ws + L.gamma);
    float* mem = reinterpret_cast<float*>(a.ws + L.mem);
    const int BH = d.B * d.H;
    hipError_t e = simt_params(a, lam, cst);
    if (e != hipSuccess) return e;
    e = simt_gamma(a, gamma, lam, cst);
    if (e != hipSuccess) return e;
    const float* gq = gamma;
    const float* gk = gamma + (size_t)BH * d.N * d.K;
    const T* v = static_cast<const T*>(a.v);
    T* out = static_cast<T*>(a.out);
    if (!a.causal) {
        const int wblk = (d.K * (d.d_v + 1) + kBlock - 1) / kBlock;
        rec_begin(a, "simt_write");
        write_kernel<T><<<dim3(BH * wblk), dim3(kBlock), 0, a.stream>>>(gk, v, mem, a.Nk, d.K, d.d_v, wblk);
        rec_end(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int rblk = (int)(((size_t)d.N * d.d_v + kBlock - 1) / kBlock);
        rec_begin(a, "simt_read");
        read_kernel<T><<<dim3(BH * rblk), dim3(kBlock), 0, a.stream>>>(gq, mem, out, d.N, d.K, d.d_v, a.eps, rblk);
        rec_end(a);
        return hipGetLastError();
    }
    const size_t lds = ((size_t)d.K * (d.d_v + 1) + (d.d_v + 1)) * sizeof(float);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&causal_kernel<T>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    rec_begin(a, "simt_causal_scan");
    causal_kernel<T><<<dim3(BH), dim3(kBlock), lds, a.stream>>>(gq, gk, v, out, d.N, d.K, d.d_v, a.eps);
    rec_end(a);
    return hipGetLastError();
}

}  // namespace

size_t simt_param_bytes(const gma_desc& d) {
    return align_up((size_t)d.H * d.K * d.d_r * sizeof(double)) + align_up((size_t)d.H * d.K * sizeof(double));
}

size_t simt_workspace(const gma_desc& d, int /*causal*/, int Nk) { return simt_layout(d, Nk).total; }

hipError_t simt_params(const Args& a, double* lam, double* cst) {
    rec_begin(a, "simt_params");
    const int64_t pairs = (int64_t)a.d.H * a.d.K;
    if (pairs == 0) {
        rec_end(a);
        return hipSuccess;
    }
    const unsigned grid = (unsigned)(pairs < (1 << 20) ? pairs : (1 << 20));
    params_kernel<<<dim3(grid), dim3(64), 0, a.stream>>>(a.var_raw, a.prior, a.d.H, a.d.K, a.d.d_r, a.d.var_floor,
                                                          lam, cst);
    rec_end(a);
    return hipGetLastError();
}

template <typename G>
static hipError_t simt_gamma_t(const Args& a, G* gamma, const double* lam, const double* cst, int* hard) {
    const gma_desc& d = a.d;
    const int BH = d.B * d.H;
    const int nmax = d.N > a.Nk ? d.N : a.Nk;
    const int nblk = (nmax + kBlock - 1) / kBlock;
    dim3 grid(BH * nblk, 2);
    rec_begin(a, "simt_responsibilities");
    if (d.dtype == GMA_F32)
        resp_kernel<float, G><<<grid, dim3(kBlock), 0, a.stream>>>(
            static_cast<const float*>(a.qr), static_cast<const float*>(a.kr), a.mu, lam, cst, gamma, hard, BH,
            d.H, d.N, a.Nk, d.d_r, d.K, nblk);
    else
        resp_kernel<bf16_t, G><<<grid, dim3(kBlock), 0, a.stream>>>(
            static_cast<const bf16_t*>(a.qr), static_cast<const bf16_t*>(a.kr), a.mu, lam, cst, gamma, hard, BH,
            d.H, d.N, a.Nk, d.d_r, d.K, nblk);
    rec_end(a);
    return hipGetLastError();
}

hipError_t simt_gamma(const Args& a, float* gamma, const double* lam, const double* cst, int* hard) {
    return simt_gamma_t<float>(a, gamma, lam, cst, hard);
}

hipError_t simt_gamma(const Args& a, double* gamma, const double* lam, const double* cst) {
    return simt_gamma_t<double>(a, gamma, lam, cst, nullptr);
}

hipError_t simt_forward(const Args& a) {
    return a.d.dtype == GMA_F32 ? simt_forward_t<float>(a) : simt_forward_t<bf16_t>(a);
}

// Causal memory of the a.d.N positions of a.kr, a.v: Gamma_K (float32, workspace) and the
// write kernel straight into a.state ([B,H,K,d_v+1] is the write kernel's own layout).
size_t simt_memory_workspace(const gma_desc& d) {
    return simt_param_bytes(d) + align_up((size_t)d.B * d.H * d.N * d.K * sizeof(float));
}

template <typename T>
hipError_t simt_memory_t(const Args& a) {
    const gma_desc& d = a.d;
    double* lam = reinterpret_cast<double*>(a.ws);
    double* cst = reinterpret_cast<double*>(a.ws + align_up((size_t)d.H * d.K * d.d_r * sizeof(double)));
    float* gk = reinterpret_cast<float*>(a.ws + simt_param_bytes(d));
    hipError_t e = simt_params(a, lam, cst);
    if (e != hipSuccess) return e;
    // key side only: no query rows (Nq = 0), the N positions as keys
    Args ka = a;
    ka.d.N = 0;
    ka.Nk = d.N;
    ka.qr = a.kr;
    if (d.N > 0 && (e = simt_gamma(ka, gk, lam, cst)) != hipSuccess) return e;
    const int BH = d.B * d.H;
    const int wblk = (d.K * (d.d_v + 1) + kBlock - 1) / kBlock;
    rec_begin(a, "simt_write");
    write_kernel<T><<<dim3(BH * wblk), dim3(kBlock), 0, a.stream>>>(gk, static_cast<const T*>(a.v), a.state, d.N,
                                                                      d.K, d.d_v, wblk);
    rec_end(a);
    return hipGetLastError();
}

hipError_t simt_memory(const Args& a) {
    return a.d.dtype == GMA_F32 ? simt_memory_t<float>(a) : simt_memory_t<bf16_t>(a);
}

}  // namespace gma
