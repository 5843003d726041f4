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


// ---- prepared parameters and the column-split decode step
//
// The mixture parameters change only when the weights do, so a caller that decodes many
// positions with the same weights prepares them once: gma_decode_prep writes, per head,
// the component means and precisions lambda = 1 / (softplus(var_raw) + var_floor) and the
// constants c_k = prior_logit_k - (1/2) sum_j log var_kj (float64).  The log joint of a
// row x is then c_k - (1/2) sum_j lambda_kj (x_j - mu_kj)^2 up to the row constant that
// cancels in the softmax: three arithmetic operations per element, no transcendental.
//
// Layout of the prepared block: per head, 16-byte vectors [H][NG][K], vector (g, k) holding
// the (mu, lambda) pairs of dims DPV g .. DPV g + DPV - 1 of component k (DPV = 2 float32
// pairs for bf16 inputs, 1 float64 pair for float32 inputs, whose gate is 1e-5; a missing
// last dim is the pair (0, 0), which adds nothing), then the constants [H][K] (float64).
// Lanes of a wave take consecutive components, so each of their 16-byte loads is one
// contiguous kilobyte.

template <typename A>
struct alignas(16) PVec {
    static constexpr int kDims = 16 / (2 * (int)sizeof(A));
    A mu[kDims], lam[kDims];
};

__host__ __device__ constexpr int prep_groups(int dr, int dims) { return (dr + dims - 1) / dims; }

constexpr int kPrepThreads = 64;

// One thread per (h, k): the variances of row k in float64.
template <typename A>
__global__ void __launch_bounds__(kPrepThreads)
    gma_decode_prep(const float* __restrict__ mu, const float* __restrict__ var_raw,
                    const float* __restrict__ prior, float var_floor, PVec<A>* __restrict__ vecs,
                    double* __restrict__ cvec, int H, int K, int dr) {
    constexpr int D = PVec<A>::kDims;
    const int h = blockIdx.y, k = blockIdx.x * kPrepThreads + threadIdx.x;
    if (k >= K) return;
    const float* m = mu + ((size_t)h * K + k) * dr;
    const float* r = var_raw + ((size_t)h * K + k) * dr;
    const int NG = prep_groups(dr, D);
    double lsum = 0.0;
    for (int g = 0; g < NG; ++g) {
        PVec<A> p;
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int j = D * g + i;
            p.mu[i] = 0;
            p.lam[i] = 0;
            if (j < dr) {
                const double rd = r[j];
                const double var = fmax(rd, 0.0) + log1p(exp(-fabs(rd))) + (double)var_floor;
                lsum += log(var);
                p.mu[i] = (A)m[j];
                p.lam[i] = (A)(1.0 / var);
            }
        }
        vecs[((size_t)h * NG + g) * K + k] = p;
    }
    cvec[(size_t)h * K + k] = (double)prior[(size_t)h * K + k] - 0.5 * lsum;
}

// Workgroup barrier that orders LDS only: the global loads and stores in flight (the state
// prefetch, the state stores) are not waited for, as __syncthreads would.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// DPP row rotations by 4 and 8 lanes (within each row of 16)
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128;
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// x + the value of lane l ^ 16 / l ^ 32 (gfx950 lane swaps)
__device__ __forceinline__ float add_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Reduction over the 64 lanes of a wave, the result in every lane: DPP within each row of
// 16 lanes (xor 1, xor 2, rotate 4, rotate 8), then the four row results read from lanes 0,
// 16, 32 and 48 and combined as (r0 . r1) . (r2 . r3).  No LDS round trip (a shuffle costs
// one), and every wave that reduces the same values gets the same bits.
template <typename Op>
__device__ __forceinline__ float wave_reduce(float x, Op op) {
    x = op(x, dpp<kQuadXor1>(x));
    x = op(x, dpp<kQuadXor2>(x));
    x = op(x, dpp<kRowRor4>(x));
    x = op(x, dpp<kRowRor8>(x));
    const int b = __float_as_int(x);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float fmax_op(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float add_op(float a, float b) { return a + b; }

// Sum over the lanes l' = l (mod NQ) of the wave (NQ a power of two), in each of them: a
// butterfly over the lane bits from log2(NQ) up.
template <int NQ>
__device__ __forceinline__ float lane_class_sum(float x) {
    if constexpr (NQ <= 1) x = x + dpp<kQuadXor1>(x);
    if constexpr (NQ <= 2) x = x + dpp<kQuadXor2>(x);
    if constexpr (NQ <= 4) x = x + dpp<kRowRor4>(x);
    if constexpr (NQ <= 8) x = x + dpp<kRowRor8>(x);
    if constexpr (NQ <= 16) x = add_xor16(x);
    if constexpr (NQ <= 32) x = add_xor32(x);
    return x;
}
// the same for a class size known only at run time (the general path)
__device__ __forceinline__ float lane_class_sum_rt(float x, int NQ) {
    if (NQ <= 1) x = x + dpp<kQuadXor1>(x);
    if (NQ <= 2) x = x + dpp<kQuadXor2>(x);
    if (NQ <= 4) x = x + dpp<kRowRor4>(x);
    if (NQ <= 8) x = x + dpp<kRowRor8>(x);
    if (NQ <= 16) x = add_xor16(x);
    if (NQ <= 32) x = add_xor32(x);
    return x;
}

// four floats at 4-byte alignment (the rows of the state are d_v + 1 floats long)
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kSplitThreads = 512;
constexpr int kSplitWaves = kSplitThreads / 64;
constexpr int kVecChunk = 16;  // parameter vectors in flight per thread
constexpr int kXPad = GMA_MAX_DR + 2 * kVecChunk;  // a wave's copy of a row, zero past d_r

// One workgroup per (b, h, column group g): the G workgroups of a (b, h) each form the
// whole softmax of the query and key rows (from the prepared parameters) and then update
// and read only their own value columns [c0, c1) of S; z (column d_v) is read by every
// group and written by the last.  No workgroup needs another's results, so the step is
// one launch with no cross-workgroup reduction, and the groups compute bitwise the same
// responsibilities.  At this size the time is a chain of memory latencies and per-wave
// instruction streams (a wave issues about one instruction per four cycles), so every
// phase is spread over all waves with few instructions and no data-dependent branches,
// and all loads issue first:
//   0: loads, unconditional (indices clamped into range) and in the order they are needed
//      (the global-load counter completes in order): the q, k rows (each wave its own
//      copy, one dim per lane), the parameter vectors of the thread's component and dim
//      part, the constants, the thread's state rows (16 bytes at a time), z, v.
//   1: log joints: wave w takes dim part p = w / (Kc / 64) (S parts, Kc = K rounded up to
//      64) of components 64 (w mod Kc / 64) + lane; the row values come from the wave's own
//      LDS copy (uniform addresses: broadcasts).  Groups past the part's end are masked
//      (lambda taken as 0).  Parts go through LDS.
//   2: softmax over the components of each row: thread (row, k) forms the log joint from
//      the parts and the constant; per-wave maxima and sums of the exponentials are
//      combined in wave order through LDS (every wave reduces the same values in the same
//      order, so the groups agree bitwise).
//   3: state update fused with the read: thread (row range, 4-column block) updates its
//      RC rows (FULL: every block has 4 columns in this group, and rows past the range
//      repeat its last row, whose new value is stored again unchanged) and sums
//      gamma_Q S_new over them; the block sums of a wave are added across its lanes
//      (butterfly), then across the waves in wave order through LDS.  The threads k < K
//      update z[k] and sum gamma_Q z_new the same way.
// Workgroups are numbered so that those of one head run on one XCD where the counts allow
// (consecutive workgroup ids go to different XCDs, eight in turn): the head's parameter
// block, read whole by each of its workgroups, is then fetched into one L2, and z and the
// partly shared cache lines of a (b, h)'s column slices come from that same L2.
template <typename T, typename A, int NQPT>
__global__ void __launch_bounds__(kSplitThreads)
    gma_decode_split(const T* __restrict__ qr, const T* __restrict__ kr, const T* __restrict__ v,
                     const PVec<A>* __restrict__ vecs, const double* __restrict__ cvec,
                     float* __restrict__ state, T* __restrict__ out, float eps, int H, int K, int dr, int dv,
                     int G) {
    constexpr int D = PVec<A>::kDims;
    constexpr int NT = kSplitThreads, NW = kSplitWaves, VC = kVecChunk;
    // NQPT > 0: every group's columns are whole 4-column blocks, NQPT of them rounded up to
    // a power of two, and a range has at most RC = max(1, NQPT / 2) rows (K <= 256);
    // NQPT = 0: the general path (ragged blocks, rows in chunks of 8)
    constexpr bool FULL = NQPT > 0;
    constexpr int RC = NQPT == 0 ? 8 : NQPT / 2 > 1 ? NQPT / 2 : 1;
    __shared__ A swx[NW][2][kXPad];     // each wave's copy of the q, k rows
    __shared__ A sq[NW][2][64];         // dim-part sums: [wave][row][lane]
    __shared__ float sg[2][GMA_MAX_K];  // gamma_Q, gamma_K
    __shared__ float sred[2][2][NW];    // per-wave maxima, sums
    __shared__ float4 scol[NW][64];     // per-wave column-block sums
    __shared__ float sden[NW];
    const int nblk = gridDim.x;
    const int unit = (nblk & 7) == 0 ? (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    // units head-major: the workgroups of one head (all b, all g) are consecutive
    const int B = nblk / (H * G);
    const int h = unit / (B * G), rem = unit - h * (B * G);
    const int bh = (rem / G) * H + h, g = rem % G, t = threadIdx.x;
    const int lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);

    // 0. loads.  The q, k rows: dims lane and 64 + lane ...
    const T* qrow = qr + (size_t)bh * dr;
    const T* krow = kr + (size_t)bh * dr;
    const int j0 = lane < dr ? lane : 0, j1 = lane + 64 < dr ? lane + 64 : 0;
    const T q0 = qrow[j0], k0r = krow[j0], q1 = qrow[j1], k1r = krow[j1];
    // ... the parameter vectors of this wave's (part, component) ...
    const int NG = prep_groups(dr, D);
    const int KB = (K + 63) >> 6;  // waves per part
    const int S = NW / KB;         // K <= 256: S >= 2
    const int p = wv / KB, kq = 64 * (wv % KB) + lane;
    const int g0 = (p * NG) / S, g1 = ((p + 1) * NG) / S;
    const int kqc = kq < K ? kq : K - 1;
    const PVec<A>* vp = vecs + (size_t)h * NG * K + kqc;
    PVec<A> pv[VC];
#pragma unroll
    for (int i = 0; i < VC; ++i) pv[i] = vp[(size_t)K * min(g0 + i, NG - 1)];
    // ... the softmax constant of thread (row, k) = (t / Kc, t mod Kc) ...
    const int Kc = KB * 64;
    const int srow_ = t / Kc, sk = t % Kc;
    const double ck = cvec[(size_t)h * K + min(sk, K - 1)];
    // ... this group's value columns [c0, c1) in blocks of 4 (NQ blocks, NQP rounded up to
    // a power of two: thread t takes block t mod NQP of row range t / NQP) ...
    const int W = dv + 1;
    const int c0 = (g * dv) / G, c1 = ((g + 1) * dv) / G;
    const int n = c1 - c0, NQ = (n + 3) >> 2;
    int NQP = NQPT;
    if (!FULL) {
        NQP = 1;
        while (NQP < NQ) NQP <<= 1;
    }
    const int qi = t & (NQP - 1), pg = t / NQP;
    const bool owner = qi < NQ;
    const int R = (K * NQP + NT - 1) / NT;  // rows per range: ceil(K / P), P = NT / NQP
    const int kr0 = min(pg * R, K), kr1 = min(kr0 + R, K);
    const int cnt = owner ? kr1 - kr0 : 0;
    const int cq = c0 + 4 * qi;      // first column of the block
    const int nv = min(4, c1 - cq);  // its columns in this group (4 but for a ragged last block)
    float* st = state + (size_t)bh * K * W;
    const float* sb = st + (size_t)min(kr0, K - 1) * W + (owner ? cq : c0);
    const int ulast = cnt > 1 ? cnt - 1 : 0;
    float4 xs[RC];
#pragma unroll
    for (int u = 0; u < RC; ++u) {
        const float* e = sb + (size_t)W * (u < ulast ? u : ulast);
        if constexpr (FULL) {
            const f32x4u y = *reinterpret_cast<const f32x4u*>(e);
            xs[u] = make_float4(y.x, y.y, y.z, y.w);
        } else {
            xs[u] = make_float4(e[0], nv > 1 ? e[1] : 0.0f, nv > 2 ? e[2] : 0.0f, nv > 3 ? e[3] : 0.0f);
        }
    }
    // ... z of component t (threads t < K) ...
    const float zt = st[(size_t)(t < K ? t : 0) * W + dv];
    // ... and this block's v values (raw: converted where used, so that no wait lands here)
    T vraw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) vraw[e] = v[(size_t)bh * dv + min(cq + e, dv - 1)];

    // 1. the quadratic forms of dim part p.  The wave's copy of the rows first (written and
    //    read by this wave only: LDS operations of a wave complete in order)
    swx[wv][0][lane] = lane < dr ? (A)Elem<T>::load(&q0, 0) : (A)0;
    swx[wv][1][lane] = lane < dr ? (A)Elem<T>::load(&k0r, 0) : (A)0;
    swx[wv][0][lane + 64] = lane + 64 < dr ? (A)Elem<T>::load(&q1, 0) : (A)0;
    swx[wv][1][lane + 64] = lane + 64 < dr ? (A)Elem<T>::load(&k1r, 0) : (A)0;
    if (lane < kXPad - 128) {
        swx[wv][0][lane + 128] = (A)0;
        swx[wv][1][lane + 128] = (A)0;
    }
    __builtin_amdgcn_wave_barrier();
    {
        A aq = 0, ak = 0;
        for (int gb = g0; gb < g1; gb += VC) {
            if (gb != g0) {
#pragma unroll
                for (int i = 0; i < VC; ++i) pv[i] = vp[(size_t)K * min(gb + i, NG - 1)];
            }
            // the chunk's row values, read together (one LDS round trip, not one per group);
            // dims past d_r read the zero padding, and their lambda is 0 (prepared)
            A xq[VC * D], xk[VC * D];
#pragma unroll
            for (int j = 0; j < VC * D; ++j) {
                xq[j] = swx[wv][0][D * gb + j];
                xk[j] = swx[wv][1][D * gb + j];
            }
#pragma unroll
            for (int i = 0; i < VC; ++i) {
                const A m = gb + i < g1 ? (A)1 : (A)0;
#pragma unroll
                for (int e = 0; e < D; ++e) {
                    const A dq = xq[D * i + e] - pv[i].mu[e], dk = xk[D * i + e] - pv[i].mu[e];
                    const A lam = pv[i].lam[e] * m;
                    aq = fma(lam * dq, dq, aq);
                    ak = fma(lam * dk, dk, ak);
                }
            }
        }
        sq[wv][0][lane] = aq;
        sq[wv][1][lane] = ak;
    }
    lds_barrier();

    // 2. softmax: thread (row, k), row = t / Kc, over the lanes with k < K
    const bool lead = srow_ < 2 && sk < K;
    const int r = srow_ < 2 ? srow_ : 0;
    A l = 0;
    {
        const int wb = sk >> 6;  // the waves holding component sk's parts: wb + KB p
        A qf = 0;
        for (int pp = 0; pp < S; ++pp) qf += sq[wb + KB * pp][r][lane];
        l = (A)ck - (A)0.5 * qf;
        const float m_w = wave_reduce(lead ? (float)l : -INFINITY, fmax_op);
        if (lane == 0) sred[0][r][wv] = m_w;  // waves past the two rows write row 0's slots unread
    }
    lds_barrier();
    float e = 0.0f;
    {
        // the row's waves are r KB .. r KB + KB - 1; the shift only has to be common to the
        // row and near its maximum: the float maximum of the (rounded) log joints serves
        float m = -INFINITY;
        for (int w = 0; w < KB; ++w) m = fmaxf(m, sred[0][r][r * KB + w]);
        e = lead ? expf((float)(l - (A)m)) : 0.0f;
        const float s_w = wave_reduce(e, add_op);
        if (lane == 0) sred[1][r][wv] = s_w;
    }
    lds_barrier();
    {
        float s = 0.0f;
        for (int w = 0; w < KB; ++w) s += sred[1][r][r * KB + w];
        if (lead) sg[r][sk] = e * (1.0f / s);
    }
    lds_barrier();

    // 3. state update + read: this thread's rows of its column block ...
    float vv[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) vv[e2] = owner && e2 < nv ? (float)Elem<T>::load(&vraw[e2], 0) : 0.0f;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if constexpr (FULL) {
        if (cnt > 0) {
#pragma unroll
            for (int u = 0; u < RC; ++u) {
                const int kk = kr0 + (u < ulast ? u : ulast);
                const float wk = sg[1][kk], wq = u < cnt ? sg[0][kk] : 0.0f;
                const float4 s4 = make_float4(fmaf(wk, vv[0], xs[u].x), fmaf(wk, vv[1], xs[u].y),
                                              fmaf(wk, vv[2], xs[u].z), fmaf(wk, vv[3], xs[u].w));
                *reinterpret_cast<f32x4u*>(st + (size_t)kk * W + cq) = f32x4u{s4.x, s4.y, s4.z, s4.w};
                acc.x = fmaf(wq, s4.x, acc.x);
                acc.y = fmaf(wq, s4.y, acc.y);
                acc.z = fmaf(wq, s4.z, acc.z);
                acc.w = fmaf(wq, s4.w, acc.w);
            }
        }
    } else {
        for (int ub = 0; ub < cnt; ub += RC) {
            if (ub != 0) {
#pragma unroll
                for (int u = 0; u < RC; ++u) {
                    const float* e2 = sb + (size_t)W * min(ub + u, ulast);
                    xs[u] = make_float4(e2[0], nv > 1 ? e2[1] : 0.0f, nv > 2 ? e2[2] : 0.0f, nv > 3 ? e2[3] : 0.0f);
                }
            }
#pragma unroll
            for (int u = 0; u < RC; ++u) {
                const int kk = kr0 + min(ub + u, ulast);
                const float wk = sg[1][kk], wq = sg[0][kk];
                float4 s4;
                s4.x = fmaf(wk, vv[0], xs[u].x);
                s4.y = fmaf(wk, vv[1], xs[u].y);
                s4.z = fmaf(wk, vv[2], xs[u].z);
                s4.w = fmaf(wk, vv[3], xs[u].w);
                if (ub + u < cnt) {
                    float* d2 = st + (size_t)kk * W + cq;
                    d2[0] = s4.x;
                    if (nv > 1) d2[1] = s4.y;
                    if (nv > 2) d2[2] = s4.z;
                    if (nv > 3) d2[3] = s4.w;
                    acc.x = fmaf(wq, s4.x, acc.x);
                    acc.y = fmaf(wq, s4.y, acc.y);
                    acc.z = fmaf(wq, s4.z, acc.z);
                    acc.w = fmaf(wq, s4.w, acc.w);
                }
            }
        }
    }
    // ... z of component t, and gamma_Q . z_new
    float dz = 0.0f;
    if (t < K) {
        const float zn = zt + sg[1][t];
        if (g == G - 1) st[(size_t)t * W + dv] = zn;
        dz = sg[0][t] * zn;
    }
    // block sums over the wave's row ranges (lanes of one block), then over the waves
    if constexpr (FULL) {
        acc.x = lane_class_sum<NQPT>(acc.x);
        acc.y = lane_class_sum<NQPT>(acc.y);
        acc.z = lane_class_sum<NQPT>(acc.z);
        acc.w = lane_class_sum<NQPT>(acc.w);
    } else {
        acc.x = lane_class_sum_rt(acc.x, NQP);
        acc.y = lane_class_sum_rt(acc.y, NQP);
        acc.z = lane_class_sum_rt(acc.z, NQP);
        acc.w = lane_class_sum_rt(acc.w, NQP);
    }
    dz = wave_reduce(dz, add_op);
    if (lane < NQP) scol[wv][lane] = acc;
    if (lane == 0) sden[wv] = dz;
    lds_barrier();
    if (t < n) {
        // column c0 + t is component t & 3 of block t >> 2: word t of a wave's block sums
        const float* sc = reinterpret_cast<const float*>(&scol[0][0]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            num += sc[w * 256 + t];
            den += sden[w];
        }
        Elem<T>::store(out + (size_t)bh * dv, c0 + t, num / (den + eps));
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

size_t decode_prepared_bytes(const gma_desc& d) {
    const int D = d.dtype == GMA_F32 ? PVec<double>::kDims : PVec<float>::kDims;
    return (size_t)d.H * prep_groups(d.d_r, D) * d.K * 16 + (size_t)d.H * d.K * sizeof(double);
}

// Column groups per (b, h) for the prepared step: the most (up to 4) that keep one
// workgroup per CU and at least 8 value columns per group.
static int cu_count() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
    }
    return cus;
}

int decode_groups(const gma_desc& d) {
    const long bh = (long)d.B * d.H;
    int g = 1;
    while (g < 4 && bh * g * 2 <= cu_count() && d.d_v / (2 * g) >= 8) g *= 2;
    return g;
}

template <typename A>
static void launch_prep(const Args& a) {
    const gma_desc& d = a.d;
    const int NG = prep_groups(d.d_r, PVec<A>::kDims);
    auto* vecs = reinterpret_cast<PVec<A>*>(a.ws);
    auto* cv = reinterpret_cast<double*>(a.ws + (size_t)d.H * NG * d.K * sizeof(PVec<A>));
    gma_decode_prep<A><<<dim3((d.K + kPrepThreads - 1) / kPrepThreads, d.H), dim3(kPrepThreads), 0, a.stream>>>(
        a.mu, a.var_raw, a.prior, d.var_floor, vecs, cv, d.H, d.K, d.d_r);
}

hipError_t decode_prepare(const Args& a) {
    rec_begin(a, "gma_decode_prep");
    if (a.d.dtype == GMA_F32)
        launch_prep<double>(a);
    else
        launch_prep<float>(a);
    rec_end(a);
    return hipGetLastError();
}

template <typename T, typename A, int NQPT>
static void launch_split_nq(const Args& a, int G, const PVec<A>* vecs, const double* cv) {
    const gma_desc& d = a.d;
    gma_decode_split<T, A, NQPT><<<dim3(d.B * d.H * G), dim3(kSplitThreads), 0, a.stream>>>(
        static_cast<const T*>(a.qr), static_cast<const T*>(a.kr), static_cast<const T*>(a.v), vecs, cv, a.state,
        static_cast<T*>(a.out), a.eps, d.H, d.K, d.d_r, d.d_v, G);
}

// The whole-block kernels when every group's columns are whole 4-column blocks (d_v a
// multiple of 4 G), specialised on the block count rounded up to a power of two; the
// general kernel otherwise.
template <typename T, typename A>
static void launch_split(const Args& a, int G) {
    const gma_desc& d = a.d;
    const int NG = prep_groups(d.d_r, PVec<A>::kDims);
    const auto* vecs = reinterpret_cast<const PVec<A>*>(a.ws);
    const auto* cv = reinterpret_cast<const double*>(a.ws + (size_t)d.H * NG * d.K * sizeof(PVec<A>));
    const int NQ = (d.d_v / G + 3) / 4;
    int NQP = 1;
    while (NQP < NQ) NQP <<= 1;
    if (d.d_v % (4 * G) != 0) return launch_split_nq<T, A, 0>(a, G, vecs, cv);
    switch (NQP) {
        case 1: return launch_split_nq<T, A, 1>(a, G, vecs, cv);
        case 2: return launch_split_nq<T, A, 2>(a, G, vecs, cv);
        case 4: return launch_split_nq<T, A, 4>(a, G, vecs, cv);
        case 8: return launch_split_nq<T, A, 8>(a, G, vecs, cv);
        case 16: return launch_split_nq<T, A, 16>(a, G, vecs, cv);
        default: return launch_split_nq<T, A, 32>(a, G, vecs, cv);
    }
}

hipError_t decode_prepared_forward(const Args& a, int groups) {
    const int G = groups > 0 ? groups : decode_groups(a.d);
    rec_begin(a, "gma_decode_split");
    if (a.d.dtype == GMA_F32)
        launch_split<float, double>(a, G);
    else
        launch_split<bf16_t, float>(a, G);
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
