// Responsibility statistics of one set of routing rows, per head.
//
// Method: Gaussian Mixture Attention (arXiv 2606.18283).  The pages analyse the learned
// responsibilities by component usage (how many of the K components receive rows, and the
// entropy of that usage) and by hard assignments compared with token categories.  Computed
// here for the rows x [B,H,N,d_r] (queries or keys), per head h pooled over (b, n):
//   hard[b,h,n]  argmax_k gamma (the lowest k among equal maxima)
//   counts[h,k]  number of rows whose hard assignment is k
//   usage[h,k]   sum over the rows of gamma_k (soft usage)
//   used[h]      number of k with counts > 0
//   entropy[h]   -sum_k p_k ln p_k / ln K, p_k = counts / (B N)  (0 when K = 1 or no rows)
//
// Kernels (caller's stream, in this order):
//   bf16, matrix cores: gma_prep and gma_causal_resp<..., STATS> (hard assignments from the
//     fp32 logits; the soft usage summed inside the kernel, one partial per workgroup, so
//     Gamma never leaves the chip);
//   SIMT: params_kernel and resp_kernel (Gamma rows in float32, hard assignments from the
//     double logits), then gma_stats_usage_rows (per chunk of rows, partial soft usage);
//   both: gma_stats_hist (per chunk of rows: histogram of the hard assignments in LDS with
//     integer atomics, so the counts do not depend on the order of arrival), then
//     gma_stats_finish (one workgroup per head: the chunk histograms and the usage partials
//     summed in a fixed order; components used and the entropy).
// Every floating-point sum has a fixed order: the results are deterministic.
#include <math.h>

#include "gma_internal.h"
#include "gma_mfma_common.h"
#include "gma_mfma_geo.h"
#include "gma_numeric.h"

namespace gma {
namespace {

constexpr int kHistChunks = 16;  // count partials per head
constexpr int kFinishThreads = 1024;

// Partial histogram of the hard assignments of chunk c of head h's rows u = b N + n (integer
// atomics in LDS: the counts do not depend on the order of arrival).
__global__ void __launch_bounds__(1024)
    gma_stats_hist(const int* __restrict__ hard, int* __restrict__ cpart, int H, int B, int N, int K,
                   int per_chunk) {
    __shared__ int hist[GMA_MAX_K];
    const int h = blockIdx.x, c = blockIdx.y, t = threadIdx.x;
    for (int k = t; k < K; k += blockDim.x) hist[k] = 0;
    __syncthreads();
    const int total = B * N;
    const int u0 = c * per_chunk, u1 = min(total, u0 + per_chunk);
    for (int u = u0 + t; u < u1; u += blockDim.x) {
        const int b = u / N, n = u % N;
        const int k = hard[(size_t)(b * H + h) * N + n];
        if ((unsigned)k < (unsigned)K) atomicAdd(&hist[k], 1);
    }
    __syncthreads();
    for (int k = t; k < K; k += blockDim.x) cpart[((size_t)h * kHistChunks + c) * K + k] = hist[k];
}

// Partial soft usage of chunk c of head h from float32 Gamma rows [B H][N][K]: thread k sums
// gamma[row][k] over the chunk's rows in order (rows u = b N + n).
__global__ void __launch_bounds__(256)
    gma_stats_usage_rows(const float* __restrict__ gamma, float* __restrict__ part, int H, int B, int N, int K, int C,
                         int per_chunk) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    const int h = blockIdx.y, c = blockIdx.z;
    if (k >= K) return;
    const int total = B * N;
    const int u0 = c * per_chunk, u1 = min(total, u0 + per_chunk);
    float s = 0.0f;
    for (int u = u0; u < u1; ++u) {
        const int b = u / N, n = u % N;
        s += gamma[((size_t)(b * H + h) * N + n) * K + k];
    }
    part[((size_t)h * C + c) * K + k] = s;
}

// One workgroup per head: counts (the chunk histograms summed), usage (the C partials of the
// head in order: rows h C + c of part when P = 0 (the SIMT chunks), rows
// (b H + h) P + p for c = b P + p otherwise (the matrix-core workgroups: batch element b,
// part p)), used, entropy.
__global__ void __launch_bounds__(kFinishThreads)
    gma_stats_finish(const int* __restrict__ cpart, const float* __restrict__ part, int* __restrict__ counts,
                     float* __restrict__ usage, int* __restrict__ used, float* __restrict__ entropy, int H, int B,
                     int N, int K, int CH, int C, int pstride, int P) {
    __shared__ int hist[GMA_MAX_K];
    const int h = blockIdx.x, t = threadIdx.x;
    const int total = B * N;
    // (partials loaded 16 at a time, then added in chunk order)
    for (int k = t; k < K; k += kFinishThreads) {
        int v[kHistChunks];
#pragma unroll
        for (int c = 0; c < kHistChunks; ++c) v[c] = c < CH ? cpart[((size_t)h * kHistChunks + c) * K + k] : 0;
        int n = 0;
#pragma unroll
        for (int c = 0; c < kHistChunks; ++c) n += v[c];
        hist[k] = n;
    }
    __syncthreads();
    for (int k = t; k < K; k += kFinishThreads) {
        counts[(size_t)h * K + k] = hist[k];
        auto prow = [&](int c) -> size_t {
            return P == 0 ? (size_t)h * C + c : ((size_t)(c / P) * H + h) * P + c % P;
        };
        float s = 0.0f;
        for (int c0 = 0; c0 < C; c0 += 16) {
            float v[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) v[c] = c0 + c < C ? part[prow(c0 + c) * pstride + k] : 0.0f;
#pragma unroll
            for (int c = 0; c < 16; ++c)
                if (c0 + c < C) s += v[c];
        }
        usage[(size_t)h * K + k] = s;
    }
    if (t < 64) {
        // components used and -sum p ln p over lanes k = t + 64 i, then across the wave
        const double rows = (double)total;
        int nu = 0;
        double ent = 0.0;
        for (int k = t; k < K; k += 64) {
            const int n = hist[k];
            if (n > 0) {
                ++nu;
                const double p = (double)n / rows;
                ent -= p * log(p);
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            nu += __shfl_xor(nu, o, 64);
            ent += __shfl_xor(ent, o, 64);
        }
        if (t == 0) {
            used[h] = nu;
            entropy[h] = (K > 1 && total > 0) ? (float)(ent / log((double)K)) : 0.0f;
        }
    }
}

struct StatsLayout {
    size_t lam, cst, gamma, W, C, hard, part, cpart, total;
    int Kp, chunks, per_chunk, parts, hchunks, hper;
};

StatsLayout stats_layout(const gma_desc& d) {
    StatsLayout L{};
    const int BH = d.B * d.H;
    size_t off = 0;
    if (stats_on_mfma(d)) {
        const mf::Geo g = mf::geometry(d);
        L.Kp = g.Kp;
        // one usage partial per workgroup of the responsibilities kernel: (b, part) per head
        L.parts = d.N > 0 ? mf::resp_parts(BH, mf::stats_np(d), nullptr) : 0;
        L.chunks = d.B * L.parts;
        L.W = off;
        off += align_up((size_t)d.H * g.Kp * 4 * g.Dp * sizeof(bf16_t));
        L.C = off;
        off += align_up((size_t)d.H * g.Kp * sizeof(float));
        L.part = off;
        off += align_up((size_t)BH * (L.parts ? L.parts : 1) * g.Kp * sizeof(float));
    } else {
        L.Kp = d.K;
        // row chunks: about 256 workgroups over the heads
        const int rows = d.B * d.N;
        int c = (256 + d.H - 1) / d.H;
        if (c > rows) c = rows;
        L.chunks = rows > 0 ? c : 0;
        L.per_chunk = L.chunks ? (rows + L.chunks - 1) / L.chunks : 0;
        L.lam = off;
        off += simt_param_bytes(d);
        L.gamma = off;
        off += align_up((size_t)BH * d.N * d.K * sizeof(float));
        L.part = off;
        off += align_up((size_t)d.H * (L.chunks ? L.chunks : 1) * d.K * sizeof(float));
    }
    L.hard = off;
    off += align_up((size_t)BH * d.N * sizeof(int));
    const int rows = d.B * d.N;
    L.hchunks = rows > 0 ? (rows < kHistChunks ? rows : kHistChunks) : 0;
    L.hper = L.hchunks ? (rows + L.hchunks - 1) / L.hchunks : 0;
    L.cpart = off;
    off += align_up((size_t)d.H * kHistChunks * d.K * sizeof(int));
    L.total = off;
    return L;
}

}  // namespace

bool stats_on_mfma(const gma_desc& d) { return d.algo != GMA_ALGO_SIMT && mf::stats_supported(d); }

size_t stats_workspace(const gma_desc& d) { return stats_layout(d).total; }

hipError_t stats_forward(const Args& a) {
    const gma_desc& d = a.d;
    const StatsLayout L = stats_layout(d);
    int* hard = a.hard ? a.hard : reinterpret_cast<int*>(a.ws + L.hard);
    float* part = reinterpret_cast<float*>(a.ws + L.part);
    int* cpart = reinterpret_cast<int*>(a.ws + L.cpart);
    const bool mfma = stats_on_mfma(d);
    hipError_t e;
    if (d.N > 0) {
        if (mfma) {
            bf16_t* W = reinterpret_cast<bf16_t*>(a.ws + L.W);
            float* cvec = reinterpret_cast<float*>(a.ws + L.C);
            if ((e = mf::stats_resp(a, W, cvec, part, hard)) != hipSuccess) return e;
        } else {
            double* lam = reinterpret_cast<double*>(a.ws + L.lam);
            double* cst = reinterpret_cast<double*>(a.ws + L.lam + align_up((size_t)d.H * d.K * d.d_r * sizeof(double)));
            float* gamma = reinterpret_cast<float*>(a.ws + L.gamma);
            if ((e = simt_params(a, lam, cst)) != hipSuccess) return e;
            // the rows as the key side (no query rows)
            Args ka = a;
            ka.d.N = 0;
            ka.Nk = d.N;
            ka.qr = a.kr;
            if ((e = simt_gamma(ka, gamma, lam, cst, hard)) != hipSuccess) return e;
            rec_begin(a, "gma_stats_usage_rows");
            gma_stats_usage_rows<<<dim3((d.K + 255) / 256, d.H, L.chunks), dim3(256), 0, a.stream>>>(
                gamma, part, d.H, d.B, d.N, d.K, L.chunks, L.per_chunk);
            rec_end(a);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        rec_begin(a, "gma_stats_hist");
        gma_stats_hist<<<dim3(d.H, L.hchunks), dim3(1024), 0, a.stream>>>(hard, cpart, d.H, d.B, d.N, d.K, L.hper);
        rec_end(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    rec_begin(a, "gma_stats_finish");
    gma_stats_finish<<<dim3(d.H), dim3(kFinishThreads), 0, a.stream>>>(
        cpart, part, a.counts, a.usage, a.used, a.entropy, d.H, d.B, d.N, d.K, L.hchunks, L.chunks,
        mfma ? L.Kp : d.K, mfma ? L.parts : 0);
    rec_end(a);
    return hipGetLastError();
}

}  // namespace gma
