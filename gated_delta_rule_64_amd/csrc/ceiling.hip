// Measured ceilings for the benchmark (not part of the KDA library): a kernel that keeps
// the bf16 matrix cores as busy as a plain instruction stream can, so the chunk path's
// matrix-core fraction can be read against a measured rate as well as the published peak.
//
//   int kda_ceiling_mfma_bf16(int blocks, int iters, float* out, hipStream_t stream)
//     launches `blocks` workgroups of 256 threads (four waves); every wave issues
//     iters x 8 independent v_mfma_f32_16x16x32_bf16 (16,384 flops each) and writes one
//     float per lane to out[blocks * 256] so nothing is optimised away. Returns a
//     hipError_t value (0 on success).
#include <hip/hip_runtime.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__global__ __launch_bounds__(256) void mfma_loop(float* out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f + 1e-3f * (float)((lane + e) & 7));
        b[e] = (__bf16)(1e-3f * (float)((lane * 3 + e) & 15));
    }
    // eight accumulation chains with distinct starting values (chains that start equal
    // are the same computation, which the compiler would merge into one)
    const float x = (float)lane;
    f32x4 c0 = {x, 0.f, 0.f, 0.f}, c1 = {x, 1.f, 0.f, 0.f}, c2 = {x, 2.f, 0.f, 0.f},
          c3 = {x, 3.f, 0.f, 0.f}, c4 = {x, 4.f, 0.f, 0.f}, c5 = {x, 5.f, 0.f, 0.f},
          c6 = {x, 6.f, 0.f, 0.f}, c7 = {x, 7.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c4, 0, 0, 0);
        c5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c5, 0, 0, 0);
        c6 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c6, 0, 0, 0);
        c7 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c7, 0, 0, 0);
    }
    const f32x4 t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    const float s = (t[0] + t[1]) + (t[2] + t[3]);
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" int kda_ceiling_mfma_bf16(int blocks, int iters, float* out, hipStream_t stream) {
    if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_loop, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
    return (int)hipGetLastError();
}
