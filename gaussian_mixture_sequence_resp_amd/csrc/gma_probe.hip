// Device peak probe for the benchmark (not part of the GMA C ABI in include/gma.h): a loop of
// the bf16 matrix-core instruction the GMA kernels use (v_mfma_f32_32x32x16_bf16), four
// independent accumulators per wave, no memory traffic in the loop, so that its rate is the
// practical MFMA ceiling of the device at the clock it holds under this load.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__global__ void __launch_bounds__(256) mfma_loop(float* __restrict__ out, int iters) {
    const int l = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (short)(0x3f80 + ((l + j) & 7));  // bf16 values near 1
        b[j] = (short)(0x3c00 + ((l * 3 + j) & 7));
    }
    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    for (int i = 0; i < iters; ++i) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc2, 0, 0, 0);
        acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc0[e] + acc1[e] + acc2[e] + acc3[e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the loop live
}

}  // namespace

// blocks x 256 threads (4 waves), each wave 4 * iters MFMAs of 32 x 32 x 16 (32768 flops).
// out: blocks * 256 floats.  Returns a hipError_t value (0 = success).
extern "C" int gma_probe_mfma(int blocks, int iters, float* out, hipStream_t stream) {
    if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
    mfma_loop<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(out, iters);
    return (int)hipGetLastError();
}
