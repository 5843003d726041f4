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

// The same loop with each MFMA's A operand read from LDS (one 16-byte fragment per lane, i.e.
// 1 KB per wave per MFMA, rotating over 16 fragments of a 16 KB block), as the logits loops
// of the GMA kernels stream their coefficient operand: its rate against the register-only
// loop shows what the LDS operand stream costs the matrix cores.
__global__ void __launch_bounds__(256) mfma_lds_loop(float* __restrict__ out, int iters) {
    __shared__ __align__(16) unsigned char lds[16 * 1024];
    const int l = threadIdx.x & 63;
    for (int i = threadIdx.x; i < 16 * 1024 / 2; i += 256)
        reinterpret_cast<short*>(lds)[i] = (short)(0x3f80 + (i & 7));
    __syncthreads();
    bf16x8 b;
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = (short)(0x3c00 + ((l * 3 + j) & 7));
    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    const unsigned char* base = lds + 16 * l;
    for (int i = 0; i < iters; ++i) {
        const int f = (4 * i) & 15;
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(base + 1024 * f);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(base + 1024 * (f + 1));
        const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(base + 1024 * (f + 2));
        const bf16x8 a3 = *reinterpret_cast<const bf16x8*>(base + 1024 * (f + 3));
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b, acc2, 0, 0, 0);
        acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b, acc3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc0[e] + acc1[e] + acc2[e] + acc3[e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Both operands of each MFMA read from LDS (2 KB per wave per MFMA): with the one-operand loop
// above, the LDS bandwidth the matrix cores can be fed at.
__global__ void __launch_bounds__(256) mfma_lds2_loop(float* __restrict__ out, int iters) {
    __shared__ __align__(16) unsigned char lds[16 * 1024];
    const int l = threadIdx.x & 63;
    for (int i = threadIdx.x; i < 16 * 1024 / 2; i += 256)
        reinterpret_cast<short*>(lds)[i] = (short)(0x3f80 + (i & 7));
    __syncthreads();
    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    const unsigned char* base = lds + 16 * l;
    for (int i = 0; i < iters; ++i) {
        const int f = (8 * i) & 15;
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(base + 1024 * f);
        const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(base + 1024 * (f + 1));
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(base + 1024 * (f + 2));
        const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(base + 1024 * (f + 3));
        const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(base + 1024 * (f + 4));
        const bf16x8 b2 = *reinterpret_cast<const bf16x8*>(base + 1024 * (f + 5));
        const bf16x8 a3 = *reinterpret_cast<const bf16x8*>(base + 1024 * (f + 6));
        const bf16x8 b3 = *reinterpret_cast<const bf16x8*>(base + 1024 * (f + 7));
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b2, acc2, 0, 0, 0);
        acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b3, acc3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc0[e] + acc1[e] + acc2[e] + acc3[e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// The two-operand LDS variant (mfma_lds2_loop), same launch and output contract.
extern "C" int gma_probe_mfma_lds2(int blocks, int iters, float* out, hipStream_t stream) {
    if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
    mfma_lds2_loop<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(out, iters);
    return (int)hipGetLastError();
}

// The LDS-operand variant (mfma_lds_loop), same launch and output contract.
extern "C" int gma_probe_mfma_lds(int blocks, int iters, float* out, hipStream_t stream) {
    if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
    mfma_lds_loop<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(out, iters);
    return (int)hipGetLastError();
}

// blocks x 256 threads (4 waves), each wave 4 * iters MFMAs of 32 x 32 x 16 (32768 flops).
// out: blocks * 256 floats.  Returns a hipError_t value (0 = success).
extern "C" int gma_probe_mfma(int blocks, int iters, float* out, hipStream_t stream) {
    if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
    mfma_loop<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(out, iters);
    return (int)hipGetLastError();
}
