// Causal memory (prefill) and the single-token decode step of the GMA forward.
//
// Method: Gaussian Mixture Attention (arXiv 2606.18283), "Core mechanism" item 3: the
// causal variant keeps prefix sums of the memory Gamma_K^T V and of the normaliser
// Gamma_K^T 1.  Taken one position at a time this is a recurrence on the state
// [S | z] (K x (d_v + 1) per head): position t adds gamma_K,t (x) [v_t | 1] (the sum is
// inclusive of t) and reads O_t = gamma_Q,t S / (gamma_Q,t . z + eps).
//
//   memory_forward   state after the N positions of a prefix: the write phase over them
//                    on matrix cores for bf16 (the fused write kernel and a split reduction,
//                    or, for coefficient blocks too large for its LDS, the causal
//                    responsibilities and totals kernels and an ordered reduction), the
//                    SIMT write otherwise.
//   decode_forward   one position per (b, h): gma_decode (below), one kernel.
#include <math.h>

#include "gma_internal.h"
#include "gma_numeric.h"

namespace gma {
namespace {

constexpr int kDecodeThreads = 1024;
constexpr int kDimSplit = 4;   // threads per component in the log-joint phase
constexpr int kStateChunk = 32;  // state rows in flight per thread

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

// One workgroup of 1024 threads per (b, h); every phase is a few rounds of independent
// loads, so the step costs a handful of memory latencies.
//   0: log-sum-exp of the head's prior logits (double).
//   1: log joint of this position's query and key rows: kDimSplit threads per component,
//      each over a contiguous quarter of the routing dims, variances (softplus + floor),
//      their log-determinant and the quadratic forms formed on the fly (double for float32
//      inputs, whose parity gate is 1e-5; float for bf16), the quarters combined in a
//      fixed order.
//   2: softmax over the components (workgroup max in double, exponentials and sums in float).
//   3: state update fused with the read: the columns c of [S | z] (the last is z, v_c = 1)
//      are dealt to P = 1024 / (d_v + 1) groups, each taking a contiguous range of
//      components, loaded kStateChunk at a time; the per-range sums of gamma_Q[k] S_new[k][c]
//      are combined in range order.
template <typename T>
__global__ void __launch_bounds__(kDecodeThreads)
    gma_decode(const T* __restrict__ qr, const T* __restrict__ kr, const T* __restrict__ v,
               const float* __restrict__ mu, const float* __restrict__ var_raw, const float* __restrict__ prior,
               float var_floor, float* __restrict__ state, T* __restrict__ out, float eps, int H, int K, int dr,
               int dv) {
    constexpr int NW = kDecodeThreads / 64;
    __shared__ float sg[2][GMA_MAX_K];  // gamma_Q, gamma_K
    __shared__ double sredd[2][NW];
    __shared__ float sred[2][NW];
    __shared__ float spart[kDecodeThreads];
    const int bh = blockIdx.x, h = bh % H, t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6;

    // 0. prior log-sum-exp of this head
    const double p = t < K ? (double)prior[(size_t)h * K + t] : -INFINITY;
    double pm = wave_max_d(p);
    if (lane == 0) sredd[0][wv] = pm;
    __syncthreads();
    pm = sredd[0][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) pm = fmax(pm, sredd[0][i]);
    __syncthreads();
    double pe = t < K ? exp(p - pm) : 0.0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) pe += __shfl_xor(pe, o, 64);
    if (lane == 0) sredd[0][wv] = pe;
    __syncthreads();
    double psum = 0.0;
#pragma unroll
    for (int i = 0; i < NW; ++i) psum += sredd[0][i];
    const double lse = pm + log(psum);
    __syncthreads();

    // 1. log joint (up to a row constant) of the query and key rows
    const int k = t / kDimSplit, part = t % kDimSplit;
    double aq = 0.0, ak = 0.0, lsum = 0.0;
    if (k < K) {
        const T* q = qr + (size_t)bh * dr;
        const T* kk = kr + (size_t)bh * dr;
        const float* m = mu + ((size_t)h * K + k) * dr;
        const float* r = var_raw + ((size_t)h * K + k) * dr;
        const int d0 = (part * dr) / kDimSplit, d1 = ((part + 1) * dr) / kDimSplit;
        if constexpr (sizeof(T) == 4) {
#pragma unroll 16
            for (int d = d0; d < d1; ++d) {
                const double rd = r[d];
                const double var = fmax(rd, 0.0) + log1p(exp(-fabs(rd))) + (double)var_floor;
                lsum += log(var);
                const double lam = 1.0 / var;
                const double dq = (double)Elem<T>::load(q, d) - (double)m[d];
                const double dk = (double)Elem<T>::load(kk, d) - (double)m[d];
                aq = fma(lam * dq, dq, aq);
                ak = fma(lam * dk, dk, ak);
            }
        } else {
            // bf16 rows: float throughout (the bf16 gate is 2e-2; float logits are off by
            // ~1e-7 relative)
            float fq = 0.0f, fk = 0.0f, fl = 0.0f;
#pragma unroll 16
            for (int d = d0; d < d1; ++d) {
                const float rf = r[d];
                const float var = fmaxf(rf, 0.0f) + log1pf(expf(-fabsf(rf))) + var_floor;
                fl += logf(var);
                const float lam = 1.0f / var;
                const float dq = Elem<T>::load(q, d) - m[d];
                const float dk = Elem<T>::load(kk, d) - m[d];
                fq = fmaf(lam * dq, dq, fq);
                fk = fmaf(lam * dk, dk, fk);
            }
            aq = fq;
            ak = fk;
            lsum = fl;
        }
    }
    // quarters combined as (0 + 1) + (2 + 3) on every lane of the group
    aq += __shfl_xor(aq, 1, 64);
    ak += __shfl_xor(ak, 1, 64);
    lsum += __shfl_xor(lsum, 1, 64);
    aq += __shfl_xor(aq, 2, 64);
    ak += __shfl_xor(ak, 2, 64);
    lsum += __shfl_xor(lsum, 2, 64);
    double lq = -INFINITY, lk = -INFINITY;
    if (k < K) {
        const double c = (double)prior[(size_t)h * K + k] - lse - 0.5 * lsum;
        lq = c - 0.5 * aq;
        lk = c - 0.5 * ak;
    }

    // 2. softmax over the components
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
    const bool lead = k < K && part == 0;
    const float eq = lead ? expf((float)(lq - mq)) : 0.0f;
    const float ek = lead ? expf((float)(lk - mk)) : 0.0f;
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
    if (lead) {
        sg[0][k] = eq * (1.0f / sq);
        sg[1][k] = ek * (1.0f / sk);
    }
    __syncthreads();

    // 3. state update + read: group pg owns components [pg K / P, (pg + 1) K / P)
    const int W = dv + 1;
    const int P = kDecodeThreads / W;  // d_v <= 128: P >= 7
    float* st = state + (size_t)bh * K * W;
    if (t < P * W) {
        const int pg = t / W, c = t % W;
        const float vc = c < dv ? (float)Elem<T>::load(v + (size_t)bh * dv, c) : 1.0f;
        const int k0 = (pg * K) / P, k1 = ((pg + 1) * K) / P;
        float acc = 0.0f;
        for (int kb = k0; kb < k1; kb += kStateChunk) {
            float x[kStateChunk];
#pragma unroll
            for (int u = 0; u < kStateChunk; ++u)
                if (kb + u < k1) x[u] = st[(size_t)(kb + u) * W + c];
#pragma unroll
            for (int u = 0; u < kStateChunk; ++u)
                if (kb + u < k1) {
                    const float s = x[u] + sg[1][kb + u] * vc;
                    st[(size_t)(kb + u) * W + c] = s;
                    acc += sg[0][kb + u] * s;
                }
        }
        spart[t] = acc;
    }
    __syncthreads();
    if (t < dv) {
        float num = 0.0f, den = 0.0f;
        for (int pg = 0; pg < P; ++pg) {
            num += spart[pg * W + t];
            den += spart[pg * W + dv];
        }
        Elem<T>::store(out + (size_t)bh * dv, t, num / (den + eps));
    }
}

}  // namespace

size_t decode_workspace(const gma_desc&) { return 0; }

hipError_t decode_forward(const Args& a) {
    const gma_desc& d = a.d;
    const int BH = d.B * d.H;
    rec_begin(a, "gma_decode");
    if (d.dtype == GMA_F32)
        gma_decode<float><<<dim3(BH), dim3(kDecodeThreads), 0, a.stream>>>(
            static_cast<const float*>(a.qr), static_cast<const float*>(a.kr), static_cast<const float*>(a.v),
            a.mu, a.var_raw, a.prior, d.var_floor, a.state, static_cast<float*>(a.out), a.eps, d.H, d.K, d.d_r,
            d.d_v);
    else
        gma_decode<bf16_t><<<dim3(BH), dim3(kDecodeThreads), 0, a.stream>>>(
            static_cast<const bf16_t*>(a.qr), static_cast<const bf16_t*>(a.kr), static_cast<const bf16_t*>(a.v),
            a.mu, a.var_raw, a.prior, d.var_floor, a.state, static_cast<bf16_t*>(a.out), a.eps, d.H, d.K, d.d_r,
            d.d_v);
    rec_end(a);
    return hipGetLastError();
}

static bool memory_on_mfma(const gma_desc& d) {
    if (d.algo == GMA_ALGO_SIMT) return false;
    return d.dtype == GMA_BF16 && mfma_memory_supported(d);
}

size_t memory_workspace(const gma_desc& d) {
    return memory_on_mfma(d) ? mfma_memory_workspace(d) : simt_memory_workspace(d);
}

hipError_t memory_forward(const Args& a) { return memory_on_mfma(a.d) ? mfma_memory(a) : simt_memory(a); }

}  // namespace gma
