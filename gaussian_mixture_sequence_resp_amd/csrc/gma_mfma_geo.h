// Geometry and shared device helpers of the MFMA kernel families (bidirectional, causal).
#pragma once

#include "gma_internal.h"
#include "gma_mfma_common.h"
#include "gma_numeric.h"

namespace gma {
namespace mf {

struct Geo {
    int Kp, MT;        // components padded to 32 * MT (MT in {1, 2, 4, 8})
    int Dp, NC;        // routing dims padded to 16 * NC (NC in {1, 2, 4, 8})
    int Dvp, NT;       // value dims padded to 32 * NT (NT in {1, 2, 4})
    int wstride;       // bytes per coefficient row in LDS
};

inline int pow2_tiles(int n, int unit) {
    int t = 1;
    while (t * unit < n) t <<= 1;
    return t;
}

inline Geo geometry(const gma_desc& d) {
    Geo g;
    g.MT = pow2_tiles(d.K, 32);
    g.Kp = 32 * g.MT;
    g.NC = pow2_tiles(d.d_r, 16);
    g.Dp = 16 * g.NC;
    g.NT = pow2_tiles(d.d_v, 32);
    g.Dvp = 32 * g.NT;
    g.wstride = 8 * g.Dp + 16;  // 4 pieces x Dp bf16, +16 B so rows rotate over the banks
    return g;
}

constexpr size_t kLdsMax = 160 * 1024 - 256;  // leave room for static LDS

// Coefficient block [ah | al | bh | bl] (Kp rows of 8 Dp bytes) and c of head h, staged into
// LDS (rows padded to wstride) by a workgroup of THREADS threads: load() issues this thread's
// first batch of global loads (up to 16 vectors), store() writes it to LDS and stages any
// remaining batches, so a caller can put its other prologue loads in flight in between.
template <int MT, int NC, int THREADS>
struct CoefRegs {
    static constexpr int Kp = 32 * MT, Dp = 16 * NC;
    static constexpr int VPR = (8 * Dp) / 16;  // 16-byte vectors per row
    static constexpr int TOTAL = Kp * VPR;
    static constexpr int PER = (TOTAL + THREADS - 1) / THREADS;
    static constexpr int BATCH = PER < 16 ? PER : 16;
    static constexpr int CPER = (Kp + THREADS - 1) / THREADS;
    bf16x8 v[BATCH];
    float c[CPER];
    const unsigned char* src;

    __device__ __forceinline__ void load_batch(int u0) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int i = threadIdx.x + (u0 + u) * THREADS;
            if (u0 + u < PER && i < TOTAL) v[u] = *reinterpret_cast<const bf16x8*>(src + 16 * (size_t)i);
        }
    }
    __device__ __forceinline__ void store_batch(unsigned char* sW, int wstride, int u0) const {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int i = threadIdx.x + (u0 + u) * THREADS;
            if (u0 + u < PER && i < TOTAL)
                *reinterpret_cast<bf16x8*>(sW + (size_t)(i / VPR) * wstride + 16 * (i % VPR)) = v[u];
        }
    }
    __device__ __forceinline__ void load(const bf16_t* W, const float* cvec, int h) {
        src = reinterpret_cast<const unsigned char*>(W + (size_t)h * Kp * 4 * Dp);
        load_batch(0);
#pragma unroll
        for (int u = 0; u < CPER; ++u) {
            const int i = threadIdx.x + u * THREADS;
            if (i < Kp) c[u] = cvec[(size_t)h * Kp + i];
        }
    }
    __device__ __forceinline__ void store(unsigned char* sW, float* sC, int wstride) {
        store_batch(sW, wstride, 0);
#pragma unroll
        for (int u = 0; u < CPER; ++u) {
            const int i = threadIdx.x + u * THREADS;
            if (i < Kp) sC[i] = c[u];
        }
        for (int u0 = BATCH; u0 < PER; u0 += BATCH) {
            load_batch(u0);
            store_batch(sW, wstride, u0);
        }
    }
};

// Map a linear block index to (head, part) so that the parts of one head run on one XCD
// (blocks are dealt round-robin to the 8 XCDs): they then share the head's coefficients
// and memory in that XCD's L2.
__device__ __forceinline__ void head_part(int b, int heads, int parts, int& head, int& part) {
    const int total = heads * parts;
    if ((heads & 7) == 0 && total == (int)gridDim.x) {
        const int x = b & 7, y = b >> 3;
        head = x + 8 * (y / parts);
        part = y % parts;
    } else {
        head = b / parts;
        part = b % parts;
    }
}

// Parameter prep (coefficients [ah|al|bh|bl] per head in bf16, c_k in float); defined with
// the bidirectional kernels.
hipError_t launch_prep(const Args& a, const Geo& g, bf16_t* W, float* cvec);

// Causal forward with the responsibilities kept on chip (gma_causal_fused.hip): eight
// component tiles (128 < K <= 256), d_r <= 64, d_v <= 64.
bool fused_causal_supported(const gma_desc& d);
size_t fused_causal_workspace(const gma_desc& d);
hipError_t fused_causal_forward(const Args& a);

// Causal family (defined in gma_mfma_causal.hip).
bool causal_supported(const gma_desc& d);
size_t causal_workspace(const gma_desc& d);
hipError_t causal_forward(const Args& a);
size_t causal_memory_workspace(const gma_desc& d);
hipError_t causal_memory(const Args& a);
// Position parts per (b, h) of the responsibilities kernel (and the part length).
int resp_parts(int BH, int Np, int* part_len);
// Responsibility statistics: hard assignments of the rows a.kr and the soft usage partials
// [B H parts][Kp] of the responsibilities kernel's workgroups (Np = stats_np(d)).
bool stats_supported(const gma_desc& d);
int stats_np(const gma_desc& d);
hipError_t stats_resp(const Args& a, bf16_t* W, float* cvec, float* upart, int* hard);
// Responsibilities of both sides as float32 rows [2][B H][N][K] (the backward's layout).
hipError_t resp_rows(const Args& a, bf16_t* W, float* cvec, float* gamma);

}  // namespace mf
}  // namespace gma
