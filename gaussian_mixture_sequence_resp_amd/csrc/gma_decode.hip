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
constexpr int kStateChunk = 24;  // state rows in flight per thread

// the two bf16 halves of a 32-bit word as float
__device__ __forceinline__ float lo_f32(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_f32(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// DPP quad permutes [1,0,3,2] and [2,3,0,1] (lane xor 1, xor 2 within each group of four)
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;
template <int CTRL>
__device__ __forceinline__ float quad_perm(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ double quad_perm(double x) {
    const long long b = __double_as_longlong(x);
    const unsigned lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)b, CTRL, 0xf, 0xf, false);
    const unsigned hi = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), CTRL, 0xf, 0xf, false);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
template <typename F>
__device__ __forceinline__ F quad_sum(F x) {
    x = x + quad_perm<kQuadXor1>(x);
    return x + quad_perm<kQuadXor2>(x);
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

// One workgroup of 1024 threads per (b, h); every phase is a few rounds of independent
// loads, so the step costs a handful of memory latencies.
//   1: log joint of this position's query and key rows: kDimSplit threads per component,
//      interleaved over the routing dims (4 dims at a time with VEC, so that the four
//      threads of a component read one contiguous 64-byte piece of its mu and var_raw rows
//      per load), variances (softplus + floor), their log-determinant and the quadratic
//      forms formed on the fly (double for float32 inputs, whose parity gate is 1e-5; float
//      for bf16), the four partial sums combined in a fixed order.  The log prior enters
//      as the raw prior logit: the log-sum-exp over the components is common to every
//      component of a row and cancels in the softmax.
//   2: softmax over the components, by one wave (max in double, exponentials and sums in
//      float).
//   3: state update fused with the read: the columns c of [S | z] (the last is z, v_c = 1)
//      are dealt to P = 1024 / (d_v + 1) groups, each taking a contiguous range of
//      components, loaded kStateChunk at a time (the first chunk at kernel start); the
//      per-range sums of gamma_Q[k] S_new[k][c] are combined in range order.
template <typename T, bool VEC>
__global__ void __launch_bounds__(kDecodeThreads)
    gma_decode(const T* __restrict__ qr, const T* __restrict__ kr, const T* __restrict__ v,
               const float* __restrict__ mu, const float* __restrict__ var_raw, const float* __restrict__ prior,
               float var_floor, float* __restrict__ state, T* __restrict__ out, float eps, int H, int K, int dr,
               int dv) {
    __shared__ float sg[2][GMA_MAX_K];  // gamma_Q, gamma_K
    __shared__ double sl[2][GMA_MAX_K];  // log joints of the query and key rows
    __shared__ float spart[kDecodeThreads];
    const int bh = blockIdx.x, h = bh % H, t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6;

    // the first chunk of this thread's state rows (phase 3) is loaded here, so that its
    // latency overlaps phases 0-2
    const int W = dv + 1;
    const int P = kDecodeThreads / W;  // d_v <= 128: P >= 7
    float* st = state + (size_t)bh * K * W;
    const bool owner = t < P * W;
    const int pg = owner ? t / W : 0, c = owner ? t % W : 0;
    const int k0 = (pg * K) / P, k1 = owner ? ((pg + 1) * K) / P : k0;
    // rows past the range re-read its last row, an empty range (and a thread that owns no
    // column) reads row k0 (< K): no predication, and those values go unused
    const float* srow = st + (size_t)k0 * W + c;
    const int nlast = k1 - k0 > 1 ? k1 - k0 - 1 : 0;
    float x[kStateChunk];
#pragma unroll
    for (int u = 0; u < kStateChunk; ++u) x[u] = srow[(size_t)W * (u < nlast ? u : nlast)];
    const float vc = owner && c < dv ? (float)Elem<T>::load(v + (size_t)bh * dv, c) : 1.0f;

    // 1. log joint (up to a row constant) of the query and key rows
    const int k = t / kDimSplit, part = t % kDimSplit;
    double aq = 0.0, ak = 0.0, lsum = 0.0;
    const double pk = k < K ? (double)prior[(size_t)h * K + k] : 0.0;
    if (k < K) {
        const T* q = qr + (size_t)bh * dr;
        const T* kk = kr + (size_t)bh * dr;
        const float* m = mu + ((size_t)h * K + k) * dr;
        const float* r = var_raw + ((size_t)h * K + k) * dr;
        if constexpr (sizeof(T) == 4) {
            auto term = [&](float rf, float mf, float qf, float kf) {
                const double rd = rf;
                const double var = fmax(rd, 0.0) + log1p(exp(-fabs(rd))) + (double)var_floor;
                lsum += log(var);
                const double lam = 1.0 / var;
                const double dq = (double)qf - (double)mf, dk = (double)kf - (double)mf;
                aq = fma(lam * dq, dq, aq);
                ak = fma(lam * dk, dk, ak);
            };
            if (VEC) {
#pragma unroll 2
                for (int d = 4 * part; d < dr; d += 4 * kDimSplit) {
                    const float4 r4 = *reinterpret_cast<const float4*>(r + d);
                    const float4 m4 = *reinterpret_cast<const float4*>(m + d);
                    const float4 q4 = *reinterpret_cast<const float4*>(q + d);
                    const float4 k4 = *reinterpret_cast<const float4*>(kk + d);
                    term(r4.x, m4.x, q4.x, k4.x);
                    term(r4.y, m4.y, q4.y, k4.y);
                    term(r4.z, m4.z, q4.z, k4.z);
                    term(r4.w, m4.w, q4.w, k4.w);
                }
            } else {
#pragma unroll 4
                for (int d = part; d < dr; d += kDimSplit) term(r[d], m[d], Elem<T>::load(q, d), Elem<T>::load(kk, d));
            }
        } else {
            // bf16 rows: float throughout (the bf16 gate is 2e-2), on the hardware exp2, log2
            // and reciprocal (about 1 ulp each): softplus(r) = max(r, 0) + log1p(e^-|r|) with
            // log1p(x) = log(u) x / (u - 1), u = 1 + x (Goldberg, "What every computer
            // scientist should know about floating-point arithmetic", 1991), which keeps the
            // relative accuracy of small x; the log-determinant is summed in base 2.
            constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
            float fq = 0.0f, fk = 0.0f, fl = 0.0f;
            auto term = [&](float rf, float mf, float qf, float kf) {
                const float e = __builtin_amdgcn_exp2f(-fabsf(rf) * kLog2e);
                const float u = 1.0f + e;
                const float lp = u == 1.0f ? e : __builtin_amdgcn_logf(u) * kLn2 * e * __builtin_amdgcn_rcpf(u - 1.0f);
                const float var = fmaxf(rf, 0.0f) + lp + var_floor;
                fl += __builtin_amdgcn_logf(var);
                const float lam = __builtin_amdgcn_rcpf(var);
                const float dq = qf - mf, dk = kf - mf;
                fq = fmaf(lam * dq, dq, fq);
                fk = fmaf(lam * dk, dk, fk);
            };
            if (VEC) {
#pragma unroll 8
                for (int d = 4 * part; d < dr; d += 4 * kDimSplit) {
                    const float4 r4 = *reinterpret_cast<const float4*>(r + d);
                    const float4 m4 = *reinterpret_cast<const float4*>(m + d);
                    const uint2 qb = *reinterpret_cast<const uint2*>(q + d);
                    const uint2 kb = *reinterpret_cast<const uint2*>(kk + d);
                    term(r4.x, m4.x, lo_f32(qb.x), lo_f32(kb.x));
                    term(r4.y, m4.y, hi_f32(qb.x), hi_f32(kb.x));
                    term(r4.z, m4.z, lo_f32(qb.y), lo_f32(kb.y));
                    term(r4.w, m4.w, hi_f32(qb.y), hi_f32(kb.y));
                }
            } else {
#pragma unroll 8
                for (int d = part; d < dr; d += kDimSplit) term(r[d], m[d], Elem<T>::load(q, d), Elem<T>::load(kk, d));
            }
            aq = fq;
            ak = fk;
            lsum = fl * kLn2;
        }
    }
    // the four partial sums of a component combined as (0 + 1) + (2 + 3) on every lane (DPP
    // quad permutes; float addition commutes, so the four lanes agree bitwise)
    aq = quad_sum(aq);
    ak = quad_sum(ak);
    lsum = quad_sum(lsum);
    // log prior up to the log-sum-exp of the prior logits, which is the same for every
    // component and cancels in the softmax below
    if (k < K && part == 0) {
        const double c = pk - 0.5 * lsum;
        sl[0][k] = c - 0.5 * aq;
        sl[1][k] = c - 0.5 * ak;
    }
    __syncthreads();

    // 2. softmax over the components, by wave 0 (component k = lane + 64 i): max in double,
    //    exponentials and sums in float
    if (wv == 0) {
        double lq[GMA_MAX_K / 64], lk[GMA_MAX_K / 64];
        double mq = -INFINITY, mk = -INFINITY;
#pragma unroll
        for (int i = 0; i < GMA_MAX_K / 64; ++i) {
            const int kc = lane + 64 * i;
            lq[i] = kc < K ? sl[0][kc] : -INFINITY;
            lk[i] = kc < K ? sl[1][kc] : -INFINITY;
            mq = fmax(mq, lq[i]);
            mk = fmax(mk, lk[i]);
        }
        mq = wave_max_d(mq);
        mk = wave_max_d(mk);
        float eq[GMA_MAX_K / 64], ek[GMA_MAX_K / 64];
        float sq = 0.0f, sk = 0.0f;
#pragma unroll
        for (int i = 0; i < GMA_MAX_K / 64; ++i) {
            const bool in = lane + 64 * i < K;
            eq[i] = in ? expf((float)(lq[i] - mq)) : 0.0f;
            ek[i] = in ? expf((float)(lk[i] - mk)) : 0.0f;
            sq += eq[i];
            sk += ek[i];
        }
        const float iq = 1.0f / wave_sum(sq), ik = 1.0f / wave_sum(sk);
#pragma unroll
        for (int i = 0; i < GMA_MAX_K / 64; ++i) {
            const int kc = lane + 64 * i;
            if (kc < K) {
                sg[0][kc] = eq[i] * iq;
                sg[1][kc] = ek[i] * ik;
            }
        }
    }
    __syncthreads();

    // 3. state update + read: group pg owns components [pg K / P, (pg + 1) K / P)
    if (owner) {
        float acc = 0.0f;
        for (int kb = k0; kb < k1; kb += kStateChunk) {
            if (kb != k0) {
#pragma unroll
                for (int u = 0; u < kStateChunk; ++u)
                    if (kb + u < k1) x[u] = st[(size_t)(kb + u) * W + c];
            }
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

template <typename T>
static void launch_decode(const Args& a, bool vec) {
    const gma_desc& d = a.d;
    const int BH = d.B * d.H;
    auto f = vec ? gma_decode<T, true> : gma_decode<T, false>;
    f<<<dim3(BH), dim3(kDecodeThreads), 0, a.stream>>>(
        static_cast<const T*>(a.qr), static_cast<const T*>(a.kr), static_cast<const T*>(a.v), a.mu, a.var_raw,
        a.prior, d.var_floor, a.state, static_cast<T*>(a.out), a.eps, d.H, d.K, d.d_r, d.d_v);
}

hipError_t decode_forward(const Args& a) {
    const gma_desc& d = a.d;
    // 16-byte loads of the parameter rows and 4-dim pieces of the q and k rows: d_r a
    // multiple of 16 and mu, var_raw 16-byte aligned (q, k rows are, given d_r % 16 == 0)
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool vec = d.d_r % 16 == 0 && al16(a.mu) && al16(a.var_raw);
    rec_begin(a, "gma_decode");
    if (d.dtype == GMA_F32)
        launch_decode<float>(a, vec);
    else
        launch_decode<bf16_t>(a, vec);
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
