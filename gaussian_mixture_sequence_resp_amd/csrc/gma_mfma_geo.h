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

// Copy the coefficient block and c of head h into LDS (rows padded to g.wstride).  Loads
// are issued in batches of 8 per thread before their LDS stores, so their latencies overlap.
__device__ __forceinline__ void stage_coefficients(unsigned char* sW, float* sC, const bf16_t* W, const float* cvec,
                                                   int h, int Kp, int Dp, int wstride) {
    const int vec_per_row = (8 * Dp) / 16;  // 16-byte vectors per row
    const int total = Kp * vec_per_row;
    const unsigned char* src = reinterpret_cast<const unsigned char*>(W + (size_t)h * Kp * 4 * Dp);
    for (int i0 = threadIdx.x; i0 < total; i0 += 8 * blockDim.x) {
        bf16x8 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * blockDim.x;
            if (i < total) v[u] = *reinterpret_cast<const bf16x8*>(src + 16 * (size_t)i);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * blockDim.x;
            if (i < total)
                *reinterpret_cast<bf16x8*>(sW + (size_t)(i / vec_per_row) * wstride + 16 * (i % vec_per_row)) = v[u];
        }
    }
    for (int i = threadIdx.x; i < Kp; i += blockDim.x) sC[i] = cvec[(size_t)h * Kp + i];
}

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

// Causal family (defined in gma_mfma_causal.hip).
bool causal_supported(const gma_desc& d);
size_t causal_workspace(const gma_desc& d);
hipError_t causal_forward(const Args& a);

}  // namespace mf
}  // namespace gma
