// Causal memory (prefill) and the single-token decode step of the GMA forward.
//
// Method: Gaussian Mixture Attention (arXiv 2606.18283), "Core mechanism" item 3: the
// causal variant keeps prefix sums of the memory Gamma_K^T V and of the normaliser
// Gamma_K^T 1.  Taken one position at a time this is a recurrence on the state
// [S | z] (K x (d_v + 1) per head): position t adds gamma_K,t (x) [v_t | 1] (the sum is
// inclusive of t) and reads O_t = gamma_Q,t S / (gamma_Q,t . z + eps).
//
//   memory_forward   state after the N positions of a prefix: the write phase over them
//                    (matrix-core write kernel and a split reduction for bf16 shapes it
//                    covers, the SIMT write otherwise).
//   decode_forward   one position per (b, h): gma_decode (below), after the SIMT parameter
//                    kernel (1/var and the log-prior constants in double).
#include <math.h>

#include "gma_internal.h"
#include "gma_numeric.h"

namespace gma {
namespace {

constexpr int kDecodeThreads = 256;  // >= GMA_MAX_K: one thread per component

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// One workgroup per (b, h).  1: the log joint of this position's query and key rows for
// every component (thread k; double, as the SIMT responsibilities); 2: softmax over the
// components (workgroup max and sum); 3: state update fused with the read: the columns
// c of [S | z] (the last one is z, with v_c = 1) are dealt to groups of threads, each group
// taking a contiguous range of components; the per-range sums of gamma_Q[k] S_new[k][c]
// are combined in range order.
template <typename T>
__global__ void __launch_bounds__(kDecodeThreads)
    gma_decode(const T* __restrict__ qr, const T* __restrict__ kr, const T* __restrict__ v,
               const float* __restrict__ mu, const double* __restrict__ lam, const double* __restrict__ cst,
               float* __restrict__ state, T* __restrict__ out, float eps, int H, int K, int dr, int dv) {
    __shared__ float sg[2][kDecodeThreads];  // gamma_Q, gamma_K
    __shared__ double sredd[2][kDecodeThreads / 64];
    __shared__ float sred[2][kDecodeThreads / 64];
    __shared__ float spart[kDecodeThreads];
    const int bh = blockIdx.x, h = bh % H, t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    constexpr int NW = kDecodeThreads / 64;

    // 1. log joint (up to a row constant) of the query and key rows, component t
    double lq = -INFINITY, lk = -INFINITY;
    if (t < K) {
        const T* q = qr + (size_t)bh * dr;
        const T* kk = kr + (size_t)bh * dr;
        const float* m = mu + ((size_t)h * K + t) * dr;
        const double* lm = lam + ((size_t)h * K + t) * dr;
        double aq = 0.0, ak = 0.0;
        for (int d = 0; d < dr; ++d) {
            const double dq = (double)Elem<T>::load(q, d) - (double)m[d];
            const double dk = (double)Elem<T>::load(kk, d) - (double)m[d];
            aq = fma(lm[d] * dq, dq, aq);
            ak = fma(lm[d] * dk, dk, ak);
        }
        const double c = cst[(size_t)h * K + t];
        lq = c - 0.5 * aq;
        lk = c - 0.5 * ak;
    }
    // 2. softmax over the components: max in double, exponentials and sums in float
    double mq = wave_max_d(lq), mk = wave_max_d(lk);
    if (lane == 0) {
        sredd[0][wv] = mq;
        sredd[1][wv] = mk;
    }
    __syncthreads();
    mq = sredd[0][0];
    mk = sredd[1][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
        mq = fmax(mq, sredd[0][i]);
        mk = fmax(mk, sredd[1][i]);
    }
    const float eq = t < K ? expf((float)(lq - mq)) : 0.0f;
    const float ek = t < K ? expf((float)(lk - mk)) : 0.0f;
    float sq = wave_sum(eq), sk = wave_sum(ek);
    if (lane == 0) {
        sred[0][wv] = sq;
        sred[1][wv] = sk;
    }
    __syncthreads();
    sq = sred[0][0];
    sk = sred[1][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
        sq += sred[0][i];
        sk += sred[1][i];
    }
    sg[0][t] = eq * (1.0f / sq);
    sg[1][t] = ek * (1.0f / sk);
    __syncthreads();

    // 3. state update + read: P groups of W threads, group p owns components
    //    [p K / P, (p + 1) K / P) of every column
    const int W = dv + 1;
    const int P = W <= kDecodeThreads ? kDecodeThreads / W : 1;
    float* st = state + (size_t)bh * K * W;
    if (t < P * W) {
        const int p = t / W, c = t % W;
        const float vc = c < dv ? (float)Elem<T>::load(v + (size_t)bh * dv, c) : 1.0f;
        const int k0 = (p * K) / P, k1 = ((p + 1) * K) / P;
        float acc = 0.0f;
        for (int k = k0; k < k1; ++k) {
            const float s = st[(size_t)k * W + c] + sg[1][k] * vc;
            st[(size_t)k * W + c] = s;
            acc += sg[0][k] * s;
        }
        spart[t] = acc;
    }
    __syncthreads();
    float den = 0.0f;
    for (int p = 0; p < P; ++p) den += spart[p * W + dv];
    for (int c = t; c < dv; c += kDecodeThreads) {
        float num = 0.0f;
        for (int p = 0; p < P; ++p) num += spart[p * W + c];
        Elem<T>::store(out + (size_t)bh * dv, c, num / (den + eps));
    }
}

}  // namespace

size_t decode_workspace(const gma_desc& d) { return simt_param_bytes(d); }

hipError_t decode_forward(const Args& a) {
    const gma_desc& d = a.d;
    double* lam = reinterpret_cast<double*>(a.ws);
    double* cst = reinterpret_cast<double*>(a.ws + align_up((size_t)d.H * d.K * d.d_r * sizeof(double)));
    hipError_t e = simt_params(a, lam, cst);
    if (e != hipSuccess) return e;
    const int BH = d.B * d.H;
    rec_begin(a, "gma_decode");
    if (d.dtype == GMA_F32)
        gma_decode<float><<<dim3(BH), dim3(kDecodeThreads), 0, a.stream>>>(
            static_cast<const float*>(a.qr), static_cast<const float*>(a.kr), static_cast<const float*>(a.v),
            a.mu, lam, cst, a.state, static_cast<float*>(a.out), a.eps, d.H, d.K, d.d_r, d.d_v);
    else
        gma_decode<bf16_t><<<dim3(BH), dim3(kDecodeThreads), 0, a.stream>>>(
            static_cast<const bf16_t*>(a.qr), static_cast<const bf16_t*>(a.kr), static_cast<const bf16_t*>(a.v),
            a.mu, lam, cst, a.state, static_cast<bf16_t*>(a.out), a.eps, d.H, d.K, d.d_r, d.d_v);
    rec_end(a);
    return hipGetLastError();
}

static bool memory_on_mfma(const gma_desc& d) {
    if (d.algo == GMA_ALGO_SIMT) return false;
    return d.dtype == GMA_BF16 && mfma_supported(d, 0);
}

size_t memory_workspace(const gma_desc& d) {
    return memory_on_mfma(d) ? mfma_memory_workspace(d) : simt_memory_workspace(d);
}

hipError_t memory_forward(const Args& a) { return memory_on_mfma(a.d) ? mfma_memory(a) : simt_memory(a); }

}  // namespace gma
