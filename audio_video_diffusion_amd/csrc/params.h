// Launch parameters of the gfx950 kernels (shared by the C-ABI layer and the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

struct PrepParams {
    const uint16_t* q; int64_t q_st, q_sh;      // bf16 NHD views (element strides)
    const uint16_t* k; int64_t k_st, k_sh;
    const uint16_t* gq; const uint16_t* gk; int64_t g_sh;
    const int32_t* pos;                          // [N][3]
    void* q_out; void* k_out;                    // [H][npad][128] bf16 or int8
    float* q_scales; float* k_scales;            // [H][nblk] (int8 only)
    float* k_mean;                               // [H][128] K smoothing means (K smoothing only)
    int n, h, npad, nblk;
    float eps;
    double rho0, rho1, rho2;   // theta^(-2/s) of the t, h and w sections (fp64, from the host)
    int sec0, sec1, sec2;
};

struct PrepVParams {
    const uint16_t* v; int64_t v_st, v_sh;      // bf16 NHD view (element strides)
    uint8_t* out;                                // [H][npad/64][128][64] E4M3 codes
    float* scales;                               // [H][128]: absmax, then scale
    int n, h, npad;
};

struct FwdParams {
    const void* q;          // [H][npad][128] bf16 or int8
    const void* k;
    const float* qs;        // [H][nblk] (int8 only)
    const float* ks;
    const uint16_t* v; int64_t v_st, v_sh;      // bf16 V view, or E4M3 V tiles (fp8v)
    const float* vs;                             // [H][128] V channel scales (fp8v only)
    // fused-Q forward only: raw Q (bf16 NHD view), gamma_q, positions and RoPE / RMSNorm parameters
    const uint16_t* qraw; int64_t q_st, q_sh;
    const uint16_t* gq; int64_t g_sh;
    const int32_t* pos;
    float eps;
    double rho0, rho1, rho2;   // theta^(-2/s) of the t, h and w sections (fp64, from the host)
    int sec0, sec1, sec2;
    uint16_t* o; int64_t o_st, o_sh;
    int n, h, npad, nblk;
    int qtiles;             // ceil(N / forward_tile_rows(...))
    int total;              // H * qtiles
    int per_xcd;            // ceil(total / 8)
    float c;                // softmax_scale * log2(e)
    // int32 scores hook only: window [s_row0, +s_nrows) x [s_col0, +s_ncols) of
    // head s_head into s_out (row-major); query tiles s_qt0 .. s_qt0 + total - 1,
    // key tiles kt0 .. kt1
    int32_t* s_out;
    int s_head, s_row0, s_nrows, s_col0, s_ncols, s_qt0, kt0, kt1;
};

hipError_t launch_prep(const PrepParams& P, bool int8, hipStream_t stream);
hipError_t launch_prep_k(const PrepParams& P, bool int8, hipStream_t stream);
hipError_t launch_prep_ksmooth(const PrepParams& P, hipStream_t stream);
hipError_t launch_forward(const FwdParams& P, bool int8, bool fp8v, hipStream_t stream);
// query rows per work-group of that forward (FwdParams::qtiles counts tiles of this size)
int forward_tile_rows(bool int8);
// RoPE section widths that are multiples of 16: each lane's 8-element chunk of a
// first half pairs with one whole chunk of the second half (the fast prep form,
// and the only one the fused-Q forwards build)
inline bool sections_are_chunks(int s0, int s1, int s2) { return s0 % 16 == 0 && s1 % 16 == 0 && s2 % 16 == 0; }
// bf16 Q'/K', V through its view, Q' computed from raw Q in the prologue
hipError_t launch_forward_fused_q(const FwdParams& P, bool int8, hipStream_t stream);
hipError_t launch_prep_v(const PrepVParams& P, hipStream_t stream);
// the int8 forward's Q'K'^T path writing the exact int32 scores of a window
hipError_t launch_scores_i8(const FwdParams& P, bool fp8v_layout, hipStream_t stream);
hipError_t launch_mfma_calib(float* out, int blocks, int iters, hipStream_t stream);

}  // namespace h3
