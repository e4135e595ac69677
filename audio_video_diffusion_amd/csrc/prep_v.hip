// FP8 V staging for the FP8 P V product, gfx950.
//
// V (bf16, token-major NHD strided view) becomes OCP E4M3 codes with one fp32
// scale per (head, channel) over all N tokens: the V scale/FP8 quantization
// step of the SageAttention2 path ("H3 Runtime Current State", Owned
// Performance Kernels: V transpose/pad and V scale/FP8 quantization; the owned
// V-preparation study emits E4M3 V plus FP32 per-channel scales).
//
//   a_c = max_n |v[n, c]|, s_c = a_c / 448, inv_c = 448 / a_c (fp32, nearest),
//   code = E4M3(clamp(v * inv_c, -448, 448)), nearest with ties to even;
//   a_c = 0 gives s_c = 0 and zero codes.  448 is E4M3's largest finite value.
//
// Output layout, per head: N_pad/64 tiles of 64 keys, each tile d-major
// [128 d][64 keys] (8 KB, key contiguous), pad keys zero.  This is the V^T
// operand order of the FP8 matrix-core product, so the forward reads it with
// plain 128-bit LDS loads.
//
// Four launches on one stream: clear the 128 x H absmax words (a fill kernel,
// not a memset), absmax over tokens (atomic max of the non-negative fp32 bit
// patterns: order-independent, so the result is deterministic), quantise and
// transpose, then turn each absmax into its scale in place.
#include "common.h"
#include "params.h"

namespace h3 {

__global__ void __launch_bounds__(256) vfp8_clear(uint32_t* amax, int count) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < count) amax[i] = 0u;
}

// One work-group per 64-token block: thread (head-chunk, channel) scans the
// block's tokens.  Grid (npad / 64, ceil(H * 128 / 256)).
__global__ void __launch_bounds__(256) vfp8_absmax(PrepVParams P) {
    const int hc = blockIdx.y * 256 + threadIdx.x;       // head * 128 + channel
    if (hc >= P.h * 128) return;
    const int head = hc >> 7, ch = hc & 127;
    const int t0 = blockIdx.x * 64;
    const int t1 = min(t0 + 64, P.n);
    float a = 0.f;
    for (int t = t0; t < t1; ++t) {
        const uint16_t b = P.v[(int64_t)t * P.v_st + (int64_t)head * P.v_sh + ch];
        a = fmaxf(a, fabsf(__uint_as_float((uint32_t)b << 16)));
    }
    if (a > 0.f) atomicMax(reinterpret_cast<unsigned int*>(P.scales) + hc, __float_as_uint(a));
}

// One work-group per (64-token tile, head): 64 tokens x 128 channels.
// Thread t handles channel pair 2*(t & 63) (+1) for 16 tokens (t >> 6) + 4i;
// codes go through LDS to leave d-major.
__global__ void __launch_bounds__(256) vfp8_quant(PrepVParams P) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[128][64 + 4];                 // [d][key], padded rows
    const int tid = threadIdx.x;
    const int head = blockIdx.y;
    const int t0 = blockIdx.x * 64;
    const int cp = tid & 63, tq = tid >> 6;
    const int c0 = 2 * cp;
    const float* amax = P.scales + (int64_t)head * 128;
    const float a0 = amax[c0], a1 = amax[c0 + 1];
    const float inv0 = a0 > 0.f ? 448.0f / a0 : 0.f;
    const float inv1 = a1 > 0.f ? 448.0f / a1 : 0.f;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
        const int key = tq + 4 * i;
        const int tok = t0 + key;
        uint32_t w = 0;
        if (tok < P.n) {
            const uint32_t two =
                *reinterpret_cast<const uint32_t*>(P.v + (int64_t)tok * P.v_st + (int64_t)head * P.v_sh + c0);
            const float x0 = fminf(fmaxf(__uint_as_float(two << 16) * inv0, -448.f), 448.f);
            const float x1 = fminf(fmaxf(__uint_as_float(two & 0xffff0000u) * inv1, -448.f), 448.f);
            w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
        }
        tile[c0][key] = (uint8_t)(w & 0xff);
        tile[c0 + 1][key] = (uint8_t)((w >> 8) & 0xff);
    }
    __syncthreads();
    // 8 KB out: thread t writes 32 bytes = half a d-row
    uint8_t* out = P.out + ((int64_t)head * P.npad + t0) * 128;
    const int row = tid >> 1, half = tid & 1;
    // rows are 68 bytes apart: every 4-byte word of a row is aligned
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&tile[row][32 * half]);
    u32x4 lo, hi;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        lo[k] = src[k];
        hi[k] = src[4 + k];
    }
    st16(out + row * 64 + 32 * half, lo);
    st16(out + row * 64 + 32 * half + 16, hi);
}

__global__ void __launch_bounds__(256) vfp8_finalize(float* scales, int count) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < count) scales[i] = scales[i] / 448.0f;
}

hipError_t launch_prep_v(const PrepVParams& P, hipStream_t stream) {
    (void)hipGetLastError();     // clear an error left by an earlier, unrelated call
    const int count = P.h * 128;
    const int cb = (count + 255) / 256;
    hipLaunchKernelGGL(vfp8_clear, dim3(cb), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(P.scales), count);
    hipLaunchKernelGGL(vfp8_absmax, dim3(P.npad / 64, cb), dim3(256), 0, stream, P);
    hipLaunchKernelGGL(vfp8_quant, dim3(P.npad / 64, P.h), dim3(256), 0, stream, P);
    hipLaunchKernelGGL(vfp8_finalize, dim3(cb), dim3(256), 0, stream, P.scales, count);
    return hipGetLastError();
}

}  // namespace h3
