// Dense bf16 and fp32 matrix-core loops: the measured peaks the benchmark
// quotes beside the datasheet figures.  Each wave runs four independent accumulator chains
// (enough to keep the matrix pipe busy across the instruction's latency) on
// operands that stay in registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_bf16_loop(float *out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (lane + e));
        b[e] = (__bf16)(0.002f * (lane - e));
    }
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, b, c3, 0, 0, 0);
    }
    const f32x4 s = c0 + c1 + c2 + c3;
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

__global__ __launch_bounds__(256) void mfma_f32_loop(float *out, int iters) {
    const int lane = threadIdx.x & 63;
    const float a = 0.001f * lane, b = 0.002f * (64 - lane);
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x4f32(b, b, c3, 0, 0, 0);
    }
    const f32x4 s = c0 + c1 + c2 + c3;
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

}  // namespace

extern "C" int32_t gdn_probe_mfma_f32(float *out, int32_t n_blocks, int32_t iters, void *stream) {
    if (!out || n_blocks < 1 || iters < 1) return 1;
    hipLaunchKernelGGL(mfma_f32_loop, dim3((unsigned)n_blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int32_t gdn_probe_mfma_bf16(float *out, int32_t n_blocks, int32_t iters, void *stream) {
    if (!out || n_blocks < 1 || iters < 1) return 1;
    hipLaunchKernelGGL(mfma_bf16_loop, dim3((unsigned)n_blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
