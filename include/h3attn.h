/*
 * h3attn.h - C ABI of the packed joint-attention library for MI355X (gfx950).
 *
 * One H3 denoiser block attends over a single packed sequence of video, audio
 * and text tokens with one softmax per query row and no padding of semantic
 * tokens ("H3 Blackwell Runtime Plan", Architecture and Non-Negotiable
 * Validation).  In front of the attention, Q and K get a per-head RMSNorm and
 * a 3-axis (t, h, w) split-half RoPE ("H3 Runtime Current State", Owned
 * Performance Kernels: the entry fusion of strided-NHD Q/K RMSNorm, split-half
 * RoPE and Q quantisation; "H3 Blackwell Runtime Plan", 2026-08-15 Handoff:
 * fused Q/K RMS + RoPE + HND layout).
 *
 * Two calls carry the path:
 *   h3attn_prep     RMSNorm + RoPE of Q and K, written head-major (HND),
 *                   either as bf16 or as int8 codes with per-64-token scales.
 *   h3attn_forward  softmax(Q' K'^T * scale) V, written token-major (NHD).
 * Around them: h3attn_prep_k + h3attn_forward_fused_q (bf16) and
 * h3attn_prep_k_i8 + h3attn_forward_fused_q_i8 (int8) move the Q half of the
 * prep into the forward; h3attn_prep_ksmooth, h3attn_prep_v_fp8 and
 * h3attn_forward_fp8v complete the quantised path (K smoothing, E4M3 P V);
 * h3attn_debug_scores_i32 is a test hook and h3attn_calibrate_mfma_bf16 a
 * measuring aid.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers (memory of the current HIP
 *   device); the problem descriptor is a HOST pointer.
 * - The caller owns every buffer.  The library never allocates, never frees,
 *   never synchronises and keeps no state between calls; calls on different
 *   streams may run concurrently.  `stream` is a hipStream_t (NULL = the
 *   default stream), passed as void* so that this header needs no HIP header
 *   and the library can be called from plain C.  Work is enqueued on `stream`;
 *   results are ready when the stream reaches that point.
 * - Strides are in ELEMENTS of the tensor's type, the last (head-dim) axis is
 *   contiguous.  Q/K/V inputs are strided NHD views, e.g. slices of an
 *   interleaved QKV projection output ("H3 Runtime Current State", Owned
 *   Performance Kernels: Q/K/V stay strided views and the attention emits
 *   contiguous token-major NHD output).
 * - Every argument is checked on the host before anything is enqueued; a
 *   rejected call enqueues nothing and returns a negative h3attn_status.
 *   There is no fallback path: unsupported input is an error.
 * - Numbers: bf16 is IEEE binary32 truncated to 16 bits (8-bit exponent);
 *   rounding to bf16 is to nearest, ties to even.
 */
#ifndef H3ATTN_H
#define H3ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3ATTN_ABI_VERSION 8

typedef enum {
    H3ATTN_OK = 0,
    H3ATTN_E_NULL = -1,         /* a required pointer is NULL                         */
    H3ATTN_E_SHAPE = -2,        /* bad N/H/sections/strides/window/scale value         */
    H3ATTN_E_UNSUPPORTED = -3,  /* head_dim != 128, unknown format, V token stride > 2^24,
                                   fused-Q forward with sections not /16              */
    H3ATTN_E_ALIGN = -4,        /* pointer not 16-byte aligned or stride not /8 (/16) */
    H3ATTN_E_ALIAS = -5,        /* an output byte range overlaps another buffer        */
    H3ATTN_E_HIP = -6           /* the HIP runtime reported an error on launch         */
} h3attn_status;

/* Storage of the prepped Q'/K' tensors. */
typedef enum {
    H3ATTN_QK_BF16 = 0,         /* bf16 values                                          */
    H3ATTN_QK_I8_BLK64 = 1      /* int8 codes + one fp32 scale per 64 tokens per head   */
} h3attn_qk_format;

/* Problem descriptor (host memory). */
typedef struct {
    int32_t n_tokens;           /* N >= 1: packed video + audio + text tokens           */
    int32_t n_heads;            /* H >= 1                                               */
    int32_t head_dim;           /* d: must be 128                                       */
    int32_t rope_sections[3];   /* widths of the t, h, w slices of d, in this order:
                                   contiguous [0,s0), [s0,s0+s1), [s0+s1,d); each even
                                   and >= 0, summing to d (e.g. 32, 48, 48); E_SHAPE
                                   otherwise.  Split-half RoPE pairs element j of a
                                   section's first half with j of its second half.
                                   With every width a multiple of 16 each lane's
                                   8-element chunk of a first half pairs with a whole
                                   chunk of the second half (the fast form); other
                                   even widths take a prep form that pairs elements
                                   through LDS (slower, same arithmetic per element),
                                   and the fused-Q forwards, which build only the chunk
                                   form, return H3ATTN_E_UNSUPPORTED for them          */
    float rope_theta;           /* RoPE base, > 0 (e.g. 10000)                          */
    float rms_eps;              /* RMSNorm epsilon, >= 0 (e.g. 1e-6)                    */
    int32_t qk_format;          /* h3attn_qk_format                                     */
} h3attn_problem;

/* Rows per head of the prepped Q'/K' buffers: N rounded up to a multiple of
 * 256.  Rows N..N_pad-1 are written by h3attn_prep (zeros) and never form
 * part of any softmax.  Returns 0 for an invalid descriptor. */
int64_t h3attn_padded_tokens(const h3attn_problem* p);

/* Bytes of ONE prepped tensor (Q' or K'): H * N_pad * 128 * (2 for bf16,
 * 1 for int8).  Returns 0 for an invalid descriptor. */
size_t h3attn_prepped_qk_bytes(const h3attn_problem* p);

/* Bytes of ONE scale array (Q' or K') in int8 format: H * ceil(N/64) * 4,
 * fp32 [H][ceil(N/64)]; 0 in bf16 format or for an invalid descriptor. */
size_t h3attn_scales_bytes(const h3attn_problem* p);

/* Bytes of the E4M3 V tiles that h3attn_prep_v_fp8 writes: H * N_pad * 128. */
size_t h3attn_prepped_v_bytes(const h3attn_problem* p);

/* Bytes of the fp32 V channel scales that h3attn_prep_v_fp8 writes: H * 128 * 4. */
size_t h3attn_v_scales_bytes(const h3attn_problem* p);

/*
 * h3attn_prep - per-head RMSNorm, then 3-axis split-half RoPE, of Q and K.
 *
 * For every token n < N, head h and tensor X in {Q, K}, with x = X[n, h, :]
 * widened from bf16 to fp32:
 *   y = x / sqrt(mean_c(x_c^2) + eps) * gamma_X[h, :]
 * then, for each section a in (t, h, w) at offset o of width s, each j < s/2:
 *   phi = pos_thw[n][a] * theta^(-2j/s)
 *   (y[o+j], y[o+j+s/2]) <- (y[o+j] cos phi - y[o+j+s/2] sin phi,
 *                            y[o+j+s/2] cos phi + y[o+j] sin phi)
 * ("H3 Runtime Current State", Owned Performance Kernels: Q/K RMSNorm and
 * split-half RoPE; "H3 Blackwell Runtime Plan", Architecture: 3-axis RoPE).
 * Arithmetic is fp32; the result is rounded once to bf16.  phi is formed and
 * reduced in fp64 (theta^(-2j/s) as the j-th power of theta^(-2/s), reduction
 * by multiples of pi/2) and cos/sin are evaluated in fp32 from their Taylor
 * series on |r| <= pi/4: absolute error about 1e-7.
 *
 * bf16 format: q_out/k_out are bf16 [H][N_pad][128] (HND, row stride 128).
 * int8 format: the bf16-rounded values of each head are grouped in blocks of
 *   64 tokens from token 0 (the last block may be partial); with a = max|y|
 *   over the block (fp32), scale = a/127 and inv = 127/a (IEEE fp32 division,
 *   round to nearest even) and code = clamp(rint(y * inv), -127, 127) (fp32
 *   product, rint ties-to-even); a == 0 gives scale 0 and zero codes.
 *   q_out/k_out are int8 [H][N_pad][128]; q_scales/k_scales are fp32
 *   [H][ceil(N/64)].  This is the int8 Q/K step of the quantised attention
 *   path ("H3 Runtime Current State", Owned Performance Kernels: Q
 *   quantization and K quantization), without K-mean smoothing.
 * Rows n >= N of q_out/k_out are written as zeros in both formats.
 *
 * q, k:      bf16 views, element (n,h,c) at base + n*stride_tok + h*stride_head + c;
 *            16-byte aligned, strides >= 0 and multiples of 8.
 * gamma_q/k: bf16; element (h,c) at base + h*gamma_head_stride + c;
 *            gamma_head_stride = 0 shares one [128] vector by all heads;
 *            16-byte aligned, stride >= 0 and a multiple of 8.
 * pos_thw:   int32 [N][3] (t, h, w) positions, 4-byte aligned.
 * q_out/k_out: h3attn_prepped_qk_bytes(p) bytes each, 16-byte aligned.
 * q_scales/k_scales: h3attn_scales_bytes(p) bytes each (4-byte aligned) in
 *            int8 format; must be NULL in bf16 format.
 * Outputs must not overlap each other or any input.
 * Errors: E_NULL, E_SHAPE, E_UNSUPPORTED, E_ALIGN, E_ALIAS (nothing is
 * enqueued), E_HIP (launch failure).
 */
int h3attn_prep(const h3attn_problem* p,
                const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                const void* gamma_q, const void* gamma_k, int64_t gamma_head_stride,
                const int32_t* pos_thw,
                void* q_out, void* k_out, float* q_scales, float* k_scales,
                void* stream);

/*
 * h3attn_prep_ksmooth - h3attn_prep in the int8 format with K smoothing: the
 * per-head, per-channel mean of K' over all tokens is subtracted before K' is
 * quantised, the K-mean step of the quantised path ("H3 Runtime Current
 * State", Owned Performance Kernels: K mean, then K quantization).  Every
 * score of a query row shifts by the same q . mean, so the attention is
 * unchanged up to quantisation, while the int8 K codes resolve the spread
 * around the mean instead of a common offset.
 *   mean[h][c] = S / N in fp32, where S adds, in block order, the fp32 sums
 *                of each 64-token block taken in token order (one rounding
 *                per addition) over the bf16-rounded K'[n,h,c];
 *   K codes/scales = the int8 quantiser of h3attn_prep applied to
 *                fl32(K'[n,h,c] - mean[h][c]) (rows n >= N stay zero).
 * Q' codes/scales are exactly those of h3attn_prep.  Feed the outputs to
 * h3attn_forward / h3attn_forward_fp8v as int8 Q'/K' (mean is not needed).
 * k_mean: device fp32 [H][128], 4-byte aligned, written; must not overlap the
 *         other arguments.  k_out also serves as scratch during the call.
 * Requires qk_format == H3ATTN_QK_I8_BLK64 (E_UNSUPPORTED otherwise).  Three
 * kernels on `stream`; nothing is allocated.  Other arguments and errors: as
 * for h3attn_prep.
 */
int h3attn_prep_ksmooth(const h3attn_problem* p,
                        const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                        const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                        const void* gamma_q, const void* gamma_k, int64_t gamma_head_stride,
                        const int32_t* pos_thw,
                        void* q_out, void* k_out, float* q_scales, float* k_scales,
                        float* k_mean, void* stream);

/*
 * h3attn_forward - non-causal attention over the whole packed sequence.
 *
 * For every head h and query n < N:
 *   O[n, h, :] = sum_m softmax_m(softmax_scale * <Q'[h,n,:], K'[h,m,:]>) V[m, h, :]
 * over all m < N: one softmax per row, no mask, no padding keys ("H3 Blackwell
 * Runtime Plan", Architecture: ragged Ulysses runs attention on the full packed
 * tokens; Non-Negotiable Validation: never pad semantic tokens).
 * In int8 format the logit is S_int * s_q[h, n/64] * s_k[h, m/64] *
 * softmax_scale with S_int the exact int32 dot product of the codes.
 * Accumulation is fp32; the probabilities are rounded to bf16 for the P V
 * product; the output is rounded once to bf16.
 *
 * q_prep/k_prep: the outputs of h3attn_prep for the same descriptor
 *            (bf16 or int8 [H][N_pad][128]); q_scales/k_scales as written
 *            by h3attn_prep (int8 format) or NULL (bf16 format).
 * v:         bf16 view [N][H][128] with strides as for q in h3attn_prep;
 *            v_stride_tok above 2^24 elements returns H3ATTN_E_UNSUPPORTED.
 * o:         bf16 output view; element (n,h,c) at o + n*o_stride_tok +
 *            h*o_stride_head + c; 16-byte aligned, strides multiples of 8,
 *            and the view must not overlap itself (either o_stride_head >= 128
 *            and o_stride_tok >= (H-1)*o_stride_head + 128, or o_stride_tok >=
 *            128 and o_stride_head >= (N-1)*o_stride_tok + 128).  Only rows
 *            n < N are written.
 * softmax_scale: finite and > 0 (e.g. 1/sqrt(128)).
 * o must not overlap any input.
 * Errors: as for h3attn_prep.
 */
int h3attn_forward(const h3attn_problem* p,
                   const void* q_prep, const void* k_prep,
                   const float* q_scales, const float* k_scales,
                   const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                   void* o, int64_t o_stride_tok, int64_t o_stride_head,
                   float softmax_scale, void* stream);

/*
 * h3attn_prep_v_fp8 - V to OCP E4M3 with one fp32 scale per (head, channel),
 * the V preparation of the FP8 P V path ("H3 Runtime Current State", Owned
 * Performance Kernels: V transpose/pad and V scale/FP8 quantization; the owned
 * V-preparation study emits E4M3 V plus FP32 per-channel scales).
 *
 * For every head h and channel c, over all N tokens:
 *   a = max_n |V[n,h,c]|, s = a / 448, inv = 448 / a   (fp32, nearest-even),
 *   code = E4M3(clamp(V[n,h,c] * inv, -448, 448))       (nearest, ties to even;
 *                                                        subnormals kept),
 *   a == 0 gives s = 0 and zero codes.
 * v:        bf16 view [N][H][128], strides as for q in h3attn_prep.
 * v_codes:  h3attn_prepped_v_bytes(p) bytes, 16-byte aligned.  Per head,
 *           N_pad/64 tiles of 64 keys; each tile d-major: byte
 *           v_codes[((h*N_pad/64 + m/64)*128 + c)*64 + m%64] is the code of
 *           V[m,h,c]; keys m >= N are 0.
 * v_scales: fp32 [H][128], 4-byte aligned: s per (head, channel).
 * Outputs must not overlap v or each other.  The descriptor's qk_format is
 * ignored.  Four kernels on `stream`; nothing is allocated.
 * Errors: as for h3attn_prep.
 */
int h3attn_prep_v_fp8(const h3attn_problem* p,
                      const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                      void* v_codes, float* v_scales, void* stream);

/*
 * h3attn_forward_fp8v - h3attn_forward with the P V product on the FP8 matrix
 * cores: V comes as E4M3 codes with per-channel scales (h3attn_prep_v_fp8) and
 * the probabilities are rounded to E4M3 for the product (the FP8-PV half of the
 * SageAttention2 path, "H3 Runtime Current State", Owned Performance Kernels:
 * INT8 QK and FP8 PV).  Q'/K' in either qk_format, as for h3attn_forward.
 *   O[n,h,c] = s[h,c] * sum_m E4M3(a * P[n,m]) code[m,h,c] / sum_m a * P[n,m]
 * where P[n,m] = 2^(log2(e) * scale * (S[n,m] - M)) are the fp32 softmax
 * numerators against a running row maximum M that the kernel raises only when
 * a score exceeds it by more than 8 / (log2(e) * scale), so P <= 2^8, and
 * a = 2^0.8 keeps a * P below 448; a cancels in the quotient.  The rounding
 * is nearest-even with subnormals, as in h3attn_prep_v_fp8.
 * v_codes/v_scales: as written by h3attn_prep_v_fp8 for the same descriptor.
 * Other arguments and errors: as for h3attn_forward.
 */
int h3attn_forward_fp8v(const h3attn_problem* p,
                        const void* q_prep, const void* k_prep,
                        const float* q_scales, const float* k_scales,
                        const void* v_codes, const float* v_scales,
                        void* o, int64_t o_stride_tok, int64_t o_stride_head,
                        float softmax_scale, void* stream);

/*
 * h3attn_prep_k - the K half of h3attn_prep in the bf16 format: writes K'
 * (bf16 [H][N_pad][128], rows n >= N zero) exactly as h3attn_prep does, and
 * no Q'.  It supplies h3attn_forward_fused_q, which prepares Q itself.
 * k, gamma_k, pos_thw, k_out: as for h3attn_prep; k_out must not overlap an
 * input.  Requires qk_format == H3ATTN_QK_BF16 (E_UNSUPPORTED otherwise).
 * Errors: as for h3attn_prep.
 */
int h3attn_prep_k(const h3attn_problem* p,
                  const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                  const void* gamma_k, int64_t gamma_head_stride,
                  const int32_t* pos_thw, void* k_out, void* stream);

/*
 * h3attn_forward_fused_q - h3attn_forward in the bf16 format with the Q half
 * of h3attn_prep moved into the forward: each work-group computes the Q' rows
 * it owns from raw Q (RMSNorm + 3-axis RoPE with the arithmetic of
 * h3attn_prep) while its first K'/V tiles load, so Q' is never written to or
 * read from memory.  This removes the prep -> forward boundary for Q, the
 * entry-fusion step of the quantised path ("H3 Runtime Current State", Owned
 * Performance Kernels: the fused entry kernel that the pages measured and the
 * direct-layout boundary-removal target).  Since Q' stays inside the kernel,
 * it is rounded to bf16 once with the base-2 logit factor
 * softmax_scale * log2(e) already applied (one rounding, as for h3attn_prep's
 * Q'), and the running row max enters as the start value of each Q'K'^T
 * product; the output therefore agrees with h3attn_prep + h3attn_forward to
 * within bf16 rounding of Q', not bit for bit.
 * q, gamma_q, pos_thw: as for h3attn_prep (raw Q view, its RMSNorm weight,
 *            the (t, h, w) positions).
 * k_prep:    bf16 K' from h3attn_prep_k (or h3attn_prep) for the same descriptor.
 * v, o, softmax_scale: as for h3attn_forward; o must not overlap any input.
 * Requires qk_format == H3ATTN_QK_BF16 and RoPE section widths that are
 * multiples of 16 (E_UNSUPPORTED otherwise).
 * Errors: as for h3attn_prep.
 */
int h3attn_forward_fused_q(const h3attn_problem* p,
                           const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                           const void* gamma_q, int64_t gamma_head_stride, const int32_t* pos_thw,
                           const void* k_prep,
                           const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                           void* o, int64_t o_stride_tok, int64_t o_stride_head,
                           float softmax_scale, void* stream);

/*
 * h3attn_prep_k_i8 - the K half of h3attn_prep in the int8 format: writes the
 * K' codes (int8 [H][N_pad][128], rows n >= N zero) and their per-64-token
 * block scales (fp32 [H][N_pad / 64]) exactly as h3attn_prep does, and no Q'
 * ("H3 Runtime Current State", Owned Performance Kernels: K quantization).  It
 * supplies h3attn_forward_fused_q_i8, which prepares and quantises Q itself.
 * k, gamma_k, pos_thw: as for h3attn_prep.  k_out, k_scales: device buffers of
 * h3attn_prepped_qk_bytes and h3attn_scales_bytes; neither may overlap an input
 * or the other.  Requires qk_format == H3ATTN_QK_I8_BLK64 (E_UNSUPPORTED
 * otherwise).  Errors: as for h3attn_prep.
 */
int h3attn_prep_k_i8(const h3attn_problem* p,
                     const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                     const void* gamma_k, int64_t gamma_head_stride,
                     const int32_t* pos_thw, void* k_out, float* k_scales, void* stream);

/*
 * h3attn_forward_fused_q_i8 - h3attn_forward in the int8 format with the Q
 * half of h3attn_prep moved into the forward (the entry fusion of the
 * quantised path, "H3 Runtime Current State", Owned Performance Kernels: the
 * fused entry kernel; Q quantization): each work-group computes its 384 Q' rows
 * from raw Q with the prep's arithmetic, rounds them to bf16, and quantises
 * each 64-row block with the prep's absmax, scale and rounding, so its codes
 * and scales are those h3attn_prep would write, and the output is that of
 * h3attn_prep + h3attn_forward bit for bit.  Q' never reaches memory.
 * q, gamma_q, pos_thw: as for h3attn_prep (raw Q view, its RMSNorm weight,
 *            the (t, h, w) positions).
 * k_codes, k_scales: from h3attn_prep_k_i8 (or h3attn_prep) for the same
 *            descriptor.
 * v, o, softmax_scale: as for h3attn_forward (bf16 V view); o must not
 *            overlap any input.
 * Requires qk_format == H3ATTN_QK_I8_BLK64 and RoPE section widths that are
 * multiples of 16 (E_UNSUPPORTED otherwise).
 * Errors: as for h3attn_prep.
 */
int h3attn_forward_fused_q_i8(const h3attn_problem* p,
                              const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                              const void* gamma_q, int64_t gamma_head_stride, const int32_t* pos_thw,
                              const void* k_codes, const float* k_scales,
                              const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                              void* o, int64_t o_stride_tok, int64_t o_stride_head,
                              float softmax_scale, void* stream);

/*
 * h3attn_debug_scores_i32 - test hook for the int8 format: the exact int32
 * Q'K'^T of one head over a window, computed by the int8 forward's own
 * kernel ("H3 Runtime Current State", Owned Performance Kernels: the INT8 QK
 * mainloop, held to byte-exactness there).  The kernel is h3attn_forward's
 * int8 kernel instantiated to stop after the Q'K'^T products: the same Q'
 * operand registers, the same buffer -> LDS stream of K' tiles with its row
 * permutation and chunk swizzle, the same int8 matrix-core chain started from
 * the bit pattern of 1.5 * 2^23; it writes the accumulators minus that start
 * in place of the softmax (V is not read).
 *   out[r][c] = sum_d q_codes[head][row0 + r][d] * k_codes[head][col0 + c][d]
 * for r < nrows, c < ncols (out is int32 [nrows][ncols], row-major, device).
 * fp8v_layout: 0 = the form h3attn_forward runs, 1 = the form
 *            h3attn_forward_fp8v runs with int8 Q'/K' (the K' row order of the
 *            FP8 P V product); both run twelve waves, 384 query rows per
 *            work-group.
 * Requires the int8 format, 0 <= head < H, nrows, ncols >= 1,
 * 0 <= row0, row0 + nrows <= N, 0 <= col0, col0 + ncols <= N,
 * fp8v_layout in {0, 1} (E_SHAPE otherwise).
 * Errors: as for h3attn_prep.
 */
int h3attn_debug_scores_i32(const h3attn_problem* p,
                            const void* q_codes, const void* k_codes,
                            int32_t head, int32_t row0, int32_t nrows,
                            int32_t col0, int32_t ncols, int32_t fp8v_layout,
                            int32_t* out, void* stream);

/* Static description of a status code (never NULL). */
const char* h3attn_status_string(int status);

/*
 * h3attn_calibrate_mfma_bf16 - measurement aid, not part of the attention
 * path: `blocks` work-groups of 512 threads (two waves per SIMD, as the
 * forward) each run `iters` x 16 bf16 32x32x16 matrix-core products per wave
 * on register operands, i.e. blocks * 8 * iters * 16 * 32768 FLOP, so that a
 * caller timing it on `stream` gets the sustained bf16 MFMA rate of this GPU
 * under its power and clock limits.
 * out: device, fp32 [blocks * 512], 4-byte aligned (written with the sums).
 * Errors: E_NULL, E_ALIGN; E_SHAPE unless 1 <= blocks, iters <= 2^20; E_HIP.
 */
int h3attn_calibrate_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream);

/* H3ATTN_ABI_VERSION of the built library. */
int h3attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H */
