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
// not a memset), absmax over tokens (partial maxima per 512-token block, then
// an atomic max of the non-negative fp32 bit patterns: order-independent, so
// the result is deterministic), quantise and transpose, then turn each absmax
// into its scale in place.
#include "common.h"
#include "params.h"

namespace h3 {

__global__ void __launch_bounds__(256) vfp8_clear(uint32_t* amax, int count) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < count) amax[i] = 0u;
}

// Channel absmax: one work-group per (512-token block, 64 groups of 8
// channels).  Thread (g, q) = (tid % 64, tid / 64) reads 16 bytes (8 channels)
// of every 4th token of the block, so a wave covers 1 KB of one token row per
// load; the four token phases meet in LDS and one atomic max per channel
// leaves the work-group.  Grid (ceil(N / 512), ceil(H * 16 / 64)).
constexpr int kAbsTokens = 512;

__global__ void __launch_bounds__(256) vfp8_absmax(PrepVParams P) {
    __shared__ float part[4][64][9];                 // [token phase][group][channel], padded
    const int g = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int c8 = blockIdx.y * 64 + g;              // head * 16 + channel group
    const bool live = c8 < P.h * 16;
    const int head = c8 >> 4, ch0 = (c8 & 15) * 8;
    const int t0 = blockIdx.x * kAbsTokens;
    const int t1 = min(t0 + kAbsTokens, P.n);
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = 0.f;
    if (live) {
        const uint16_t* base = P.v + (int64_t)head * P.v_sh + ch0;
#pragma unroll 8
        for (int t = t0 + q; t < t1; t += 4) {
            const u32x4 w = ld16(base + (int64_t)t * P.v_st);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                a[2 * k] = fmaxf(a[2 * k], fabsf(bf16lo_to_f32(w[k])));
                a[2 * k + 1] = fmaxf(a[2 * k + 1], fabsf(bf16hi_to_f32(w[k])));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[q][g][i] = a[i];
    __syncthreads();
    if (q == 0 && live) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float m = fmaxf(fmaxf(part[0][g][i], part[1][g][i]), fmaxf(part[2][g][i], part[3][g][i]));
            if (m > 0.f)
                atomicMax(reinterpret_cast<unsigned int*>(P.scales) + head * 128 + ch0 + i, __float_as_uint(m));
        }
    }
}

// One work-group per (64-token tile, head): 64 tokens x 128 channels.
// Thread t handles the 8 channels 8 * (t & 15) of the tokens (t >> 4) + 16i,
// i < 4, with 16-byte loads (a wave reads four 256-byte token rows); codes go
// through LDS to leave d-major.
__global__ void __launch_bounds__(256) vfp8_quant(PrepVParams P) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[128][64 + 4];                 // [d][key], padded rows
    const int tid = threadIdx.x;
    const int head = blockIdx.y;
    const int t0 = blockIdx.x * 64;
    const int c0 = 8 * (tid & 15), tq = tid >> 4;
    const float* amax = P.scales + (int64_t)head * 128 + c0;
    float inv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = amax[i];
        inv[i] = a > 0.f ? 448.0f / a : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = tq + 16 * i;
        const int tok = t0 + key;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (tok < P.n) w = ld16(P.v + (int64_t)tok * P.v_st + (int64_t)head * P.v_sh + c0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float x0 = fminf(fmaxf(bf16lo_to_f32(w[k]) * inv[2 * k], -448.f), 448.f);
            const float x1 = fminf(fmaxf(bf16hi_to_f32(w[k]) * inv[2 * k + 1], -448.f), 448.f);
            const uint32_t b = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
            tile[c0 + 2 * k][key] = (uint8_t)(b & 0xff);
            tile[c0 + 2 * k + 1][key] = (uint8_t)((b >> 8) & 0xff);
        }
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
    hipLaunchKernelGGL(vfp8_absmax, dim3((P.n + kAbsTokens - 1) / kAbsTokens, (P.h * 16 + 63) / 64), dim3(256), 0,
                       stream, P);
    hipLaunchKernelGGL(vfp8_quant, dim3(P.npad / 64, P.h), dim3(256), 0, stream, P);
    hipLaunchKernelGGL(vfp8_finalize, dim3(cb), dim3(256), 0, stream, P.scales, count);
    return hipGetLastError();
}

}  // namespace h3
