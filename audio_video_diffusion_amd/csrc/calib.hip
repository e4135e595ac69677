// Matrix-core calibration for measurement: the sustained bf16 MFMA rate of
// this GPU under its own power and clock limits.  Not part of the attention
// path; the benchmark times it beside the forward so that the forward's rate
// can be read against the sustained rate as well as against the data-sheet
// peak.
//
// Launch shape as the forward: 512-thread work-groups, two waves per SIMD.
// Each wave runs `iters` x 16 v_mfma_f32_32x32x16_bf16 on four independent
// accumulators (no dependency stalls) from register operands; nothing but the
// final sums touches memory.
#include "common.h"
#include "params.h"

namespace h3 {

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_calib_kernel(float* out, int iters, float seed) {
    const int tid = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(tid + i));
        b[i] = (__bf16)(seed * (float)(tid - i));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += (c0[i] + c1[i]) + (c2[i] + c3[i]);
    out[(int64_t)blockIdx.x * 512 + tid] = s;
}

hipError_t launch_mfma_calib(float* out, int blocks, int iters, hipStream_t stream) {
    (void)hipGetLastError();     // clear an error left by an earlier, unrelated call
    hipLaunchKernelGGL(mfma_calib_kernel, dim3(blocks), dim3(512), 0, stream, out, iters, 1e-3f);
    return hipGetLastError();
}

}  // namespace h3
