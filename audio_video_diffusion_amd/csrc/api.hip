// C ABI of the packed-attention library: argument validation and launches.
//
// Every check runs on the host before anything is enqueued, so a rejected
// call has no side effect.  The library keeps no state, never allocates and
// never synchronises.
#include <math.h>
#include <string.h>

#include "../../include/h3attn.h"
#include "params.h"


namespace {

constexpr int64_t kMaxTokens = (int64_t)1 << 30;   // keeps every int32 index in range
// The forward addresses the 64 V rows of a tile with 32-bit byte offsets.
constexpr int64_t kMaxVStrideTok = (int64_t)1 << 24;

struct Range {
    uintptr_t lo, hi;    // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Byte extent of a strided [N][H][d] view.
Range view_range(const void* p, int64_t n, int64_t h, int64_t st, int64_t sh, int64_t d, int64_t elt) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return {b, b + (uintptr_t)(((n - 1) * st + (h - 1) * sh + d) * elt)};
}
Range span(const void* p, size_t bytes) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return {b, b + bytes};
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_problem(const h3attn_problem* p) {
    if (!p) return H3ATTN_E_NULL;
    if (p->head_dim != 128) return H3ATTN_E_UNSUPPORTED;
    if (p->qk_format != H3ATTN_QK_BF16 && p->qk_format != H3ATTN_QK_I8_BLK64) return H3ATTN_E_UNSUPPORTED;
    if (p->n_tokens < 1 || p->n_tokens > kMaxTokens || p->n_heads < 1) return H3ATTN_E_SHAPE;
    // the head-major prepped tensors are indexed with 64-bit offsets, but keep H*N_pad*d sane
    const int64_t npad = ((int64_t)p->n_tokens + 255) / 256 * 256;
    if ((int64_t)p->n_heads * npad > ((int64_t)1 << 40)) return H3ATTN_E_SHAPE;
    int sum = 0;
    for (int a = 0; a < 3; ++a) {
        const int s = p->rope_sections[a];
        if (s < 0 || s % 2) return H3ATTN_E_SHAPE;
        sum += s;
    }
    if (sum != p->head_dim) return H3ATTN_E_SHAPE;
    if (!(p->rope_theta > 0.f) || !isfinite(p->rope_theta)) return H3ATTN_E_SHAPE;
    if (!(p->rms_eps >= 0.f) || !isfinite(p->rms_eps)) return H3ATTN_E_SHAPE;
    return H3ATTN_OK;
}

int64_t npad_of(const h3attn_problem* p) { return ((int64_t)p->n_tokens + 255) / 256 * 256; }

// theta^(-2/s) of RoPE section a in fp64: the kernels take the inverse
// frequencies theta^(-2j/s) as its powers (1 for an empty section).
double rope_ratio(const h3attn_problem* p, int a) {
    const int s = p->rope_sections[a];
    return s > 0 ? pow((double)p->rope_theta, -2.0 / (double)s) : 1.0;
}
int64_t nblk_of(const h3attn_problem* p) { return ((int64_t)p->n_tokens + 63) / 64; }

// strides of an input view: non-negative multiples of 8 elements
int check_in_view(const void* ptr, int64_t st, int64_t sh) {
    if (!ptr) return H3ATTN_E_NULL;
    if (st < 0 || sh < 0) return H3ATTN_E_SHAPE;
    if (!aligned(ptr, 16) || (st % 8) || (sh % 8)) return H3ATTN_E_ALIGN;
    return H3ATTN_OK;
}

}  // namespace

extern "C" {

int h3attn_abi_version(void) { return H3ATTN_ABI_VERSION; }

const char* h3attn_status_string(int s) {
    switch (s) {
        case H3ATTN_OK: return "ok";
        case H3ATTN_E_NULL: return "a required pointer is NULL";
        case H3ATTN_E_SHAPE: return "invalid shape, stride, window or scalar argument";
        case H3ATTN_E_UNSUPPORTED: return "unsupported head_dim, format or RoPE section widths";
        case H3ATTN_E_ALIGN: return "pointer or stride misaligned";
        case H3ATTN_E_ALIAS: return "an output overlaps another buffer";
        case H3ATTN_E_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int64_t h3attn_padded_tokens(const h3attn_problem* p) {
    return check_problem(p) == H3ATTN_OK ? npad_of(p) : 0;
}

size_t h3attn_prepped_qk_bytes(const h3attn_problem* p) {
    if (check_problem(p) != H3ATTN_OK) return 0;
    const size_t elt = p->qk_format == H3ATTN_QK_BF16 ? 2 : 1;
    return (size_t)p->n_heads * (size_t)npad_of(p) * 128 * elt;
}

size_t h3attn_scales_bytes(const h3attn_problem* p) {
    if (check_problem(p) != H3ATTN_OK || p->qk_format != H3ATTN_QK_I8_BLK64) return 0;
    return (size_t)p->n_heads * (size_t)nblk_of(p) * sizeof(float);
}

size_t h3attn_prepped_v_bytes(const h3attn_problem* p) {
    if (check_problem(p) != H3ATTN_OK) return 0;
    return (size_t)p->n_heads * (size_t)npad_of(p) * 128;
}

size_t h3attn_v_scales_bytes(const h3attn_problem* p) {
    if (check_problem(p) != H3ATTN_OK) return 0;
    return (size_t)p->n_heads * 128 * sizeof(float);
}

}  // extern "C"

namespace {

// Shared by h3attn_prep, h3attn_prep_ksmooth (int8 with K smoothing) and
// h3attn_prep_k (bf16 K' alone: q, gamma_q and q_out are unused and NULL).
int prep_common(const h3attn_problem* p,
                const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                const void* gamma_q, const void* gamma_k, int64_t gamma_head_stride,
                const int32_t* pos_thw,
                void* q_out, void* k_out, float* q_scales, float* k_scales,
                float* k_mean, bool smooth, bool k_only, bool k_only_i8, void* stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    const bool i8 = p->qk_format == H3ATTN_QK_I8_BLK64;
    if (smooth && !i8) return H3ATTN_E_UNSUPPORTED;
    if (k_only && i8 != k_only_i8) return H3ATTN_E_UNSUPPORTED;
    if (smooth && !k_mean) return H3ATTN_E_NULL;
    if (smooth && !aligned(k_mean, 4)) return H3ATTN_E_ALIGN;
    if (k_only) {
        // placeholders for the absent Q side: the same buffers as K, never read or written
        q = k; q_stride_tok = k_stride_tok; q_stride_head = k_stride_head;
        gamma_q = gamma_k;
        q_out = k_out;
        q_scales = k_scales;
    }
    if ((rc = check_in_view(q, q_stride_tok, q_stride_head))) return rc;
    if ((rc = check_in_view(k, k_stride_tok, k_stride_head))) return rc;
    if ((rc = check_in_view(gamma_q, 0, gamma_head_stride))) return rc;
    if ((rc = check_in_view(gamma_k, 0, gamma_head_stride))) return rc;
    if (!pos_thw || !q_out || !k_out) return H3ATTN_E_NULL;
    if (i8 && (!q_scales || !k_scales)) return H3ATTN_E_NULL;
    if (!i8 && (q_scales || k_scales)) return H3ATTN_E_SHAPE;
    if (!aligned(pos_thw, 4) || !aligned(q_out, 16) || !aligned(k_out, 16)) return H3ATTN_E_ALIGN;
    if (i8 && (!aligned(q_scales, 4) || !aligned(k_scales, 4))) return H3ATTN_E_ALIGN;

    const int64_t n = p->n_tokens, h = p->n_heads;
    const size_t out_b = h3attn_prepped_qk_bytes(p), sc_b = h3attn_scales_bytes(p);
    const Range ins[5] = {view_range(q, n, h, q_stride_tok, q_stride_head, 128, 2),
                          view_range(k, n, h, k_stride_tok, k_stride_head, 128, 2),
                          view_range(gamma_q, 1, h, 0, gamma_head_stride, 128, 2),
                          view_range(gamma_k, 1, h, 0, gamma_head_stride, 128, 2),
                          span(pos_thw, (size_t)n * 3 * sizeof(int32_t))};
    Range outs[5] = {span(q_out, out_b), span(k_out, out_b), {0, 0}, {0, 0}, {0, 0}};
    int nout = smooth ? 5 : i8 ? 4 : 2;
    if (i8) {
        outs[2] = span(q_scales, sc_b);
        outs[3] = span(k_scales, sc_b);
    }
    if (k_only) {                // K' (and its scales) only
        outs[0] = outs[1];
        outs[1] = outs[3];
        nout = i8 ? 2 : 1;
    }
    if (smooth) outs[4] = span(k_mean, (size_t)h * 128 * sizeof(float));
    for (int o = 0; o < nout; ++o) {
        for (const Range& r : ins)
            if (overlap(outs[o], r)) return H3ATTN_E_ALIAS;
        for (int o2 = o + 1; o2 < nout; ++o2)
            if (overlap(outs[o], outs[o2])) return H3ATTN_E_ALIAS;
    }

    h3::PrepParams P{};
    P.q = static_cast<const uint16_t*>(q); P.q_st = q_stride_tok; P.q_sh = q_stride_head;
    P.k = static_cast<const uint16_t*>(k); P.k_st = k_stride_tok; P.k_sh = k_stride_head;
    P.gq = static_cast<const uint16_t*>(gamma_q); P.gk = static_cast<const uint16_t*>(gamma_k);
    P.g_sh = gamma_head_stride;
    P.pos = pos_thw;
    P.q_out = q_out; P.k_out = k_out; P.q_scales = q_scales; P.k_scales = k_scales;
    P.n = (int)n; P.h = (int)h; P.npad = (int)npad_of(p); P.nblk = (int)nblk_of(p);
    P.eps = p->rms_eps;
    P.rho0 = rope_ratio(p, 0); P.rho1 = rope_ratio(p, 1); P.rho2 = rope_ratio(p, 2);
    P.sec0 = p->rope_sections[0]; P.sec1 = p->rope_sections[1]; P.sec2 = p->rope_sections[2];
    P.k_mean = k_mean;
    if (k_only) {
        P.q = nullptr; P.gq = nullptr; P.q_out = nullptr; P.q_scales = nullptr;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = smooth ? h3::launch_prep_ksmooth(P, st) : k_only ? h3::launch_prep_k(P, i8, st)
                                                                          : h3::launch_prep(P, i8, st);
    if (e != hipSuccess) return H3ATTN_E_HIP;
    return H3ATTN_OK;
}

}  // namespace

extern "C" {

int h3attn_prep(const h3attn_problem* p,
                const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                const void* gamma_q, const void* gamma_k, int64_t gamma_head_stride,
                const int32_t* pos_thw,
                void* q_out, void* k_out, float* q_scales, float* k_scales,
                void* stream) {
    return prep_common(p, q, q_stride_tok, q_stride_head, k, k_stride_tok, k_stride_head, gamma_q, gamma_k,
                       gamma_head_stride, pos_thw, q_out, k_out, q_scales, k_scales, nullptr, false, false, false,
                       stream);
}

int h3attn_prep_k(const h3attn_problem* p, const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                  const void* gamma_k, int64_t gamma_head_stride, const int32_t* pos_thw, void* k_out,
                  void* stream) {
    return prep_common(p, nullptr, 0, 0, k, k_stride_tok, k_stride_head, nullptr, gamma_k, gamma_head_stride,
                       pos_thw, nullptr, k_out, nullptr, nullptr, nullptr, false, true, false, stream);
}

int h3attn_prep_k_i8(const h3attn_problem* p, const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                     const void* gamma_k, int64_t gamma_head_stride, const int32_t* pos_thw, void* k_out,
                     float* k_scales, void* stream) {
    return prep_common(p, nullptr, 0, 0, k, k_stride_tok, k_stride_head, nullptr, gamma_k, gamma_head_stride,
                       pos_thw, nullptr, k_out, nullptr, k_scales, nullptr, false, true, true, stream);
}

int h3attn_prep_ksmooth(const h3attn_problem* p,
                        const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                        const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                        const void* gamma_q, const void* gamma_k, int64_t gamma_head_stride,
                        const int32_t* pos_thw,
                        void* q_out, void* k_out, float* q_scales, float* k_scales,
                        float* k_mean, void* stream) {
    return prep_common(p, q, q_stride_tok, q_stride_head, k, k_stride_tok, k_stride_head, gamma_q, gamma_k,
                       gamma_head_stride, pos_thw, q_out, k_out, q_scales, k_scales, k_mean, true, false, false,
                       stream);
}

}  // extern "C"

namespace {

// Raw-Q inputs of h3attn_forward_fused_q and h3attn_forward_fused_q_i8.
struct RawQ {
    const void* q;
    int64_t st, sh;
    const void* gamma;
    int64_t g_sh;
    const int32_t* pos;
    bool int8;           // the entry point's format
};

// Shared by h3attn_forward (bf16 V view), h3attn_forward_fp8v (staged E4M3 V)
// and h3attn_forward_fused_q (raw Q in place of q_prep, bf16 only).
int forward_common(const h3attn_problem* p, const void* q_prep, const void* k_prep,
                   const float* q_scales, const float* k_scales, bool fp8v, const void* v,
                   int64_t v_stride_tok, int64_t v_stride_head, const float* v_scales, void* o,
                   int64_t o_stride_tok, int64_t o_stride_head, float softmax_scale, const RawQ* rq,
                   void* stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    const bool i8 = p->qk_format == H3ATTN_QK_I8_BLK64;
    if (rq) {
        if (i8 != rq->int8 || fp8v) return H3ATTN_E_UNSUPPORTED;
        // the fused prologue pairs whole 8-element chunks only
        if (!h3::sections_are_chunks(p->rope_sections[0], p->rope_sections[1], p->rope_sections[2]))
            return H3ATTN_E_UNSUPPORTED;
        if ((rc = check_in_view(rq->q, rq->st, rq->sh))) return rc;
        if ((rc = check_in_view(rq->gamma, 0, rq->g_sh))) return rc;
        if (!rq->pos) return H3ATTN_E_NULL;
        if (!aligned(rq->pos, 4)) return H3ATTN_E_ALIGN;
        q_prep = k_prep;     // placeholders for the checks below; never read
        if (i8) q_scales = k_scales;
    }
    if (!q_prep || !k_prep) return H3ATTN_E_NULL;
    if (!aligned(q_prep, 16) || !aligned(k_prep, 16)) return H3ATTN_E_ALIGN;
    if (i8 && (!q_scales || !k_scales)) return H3ATTN_E_NULL;
    if (!i8 && (q_scales || k_scales)) return H3ATTN_E_SHAPE;
    if (i8 && (!aligned(q_scales, 4) || !aligned(k_scales, 4))) return H3ATTN_E_ALIGN;
    const int64_t n = p->n_tokens, h = p->n_heads;
    Range vrng;
    if (fp8v) {
        if (!v || !v_scales) return H3ATTN_E_NULL;
        if (!aligned(v, 16) || !aligned(v_scales, 4)) return H3ATTN_E_ALIGN;
        vrng = span(v, h3attn_prepped_v_bytes(p));
    } else {
        if ((rc = check_in_view(v, v_stride_tok, v_stride_head))) return rc;
        if (v_stride_tok > kMaxVStrideTok) return H3ATTN_E_UNSUPPORTED;
        vrng = view_range(v, n, h, v_stride_tok, v_stride_head, 128, 2);
    }
    if ((rc = check_in_view(o, o_stride_tok, o_stride_head))) return rc;
    if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return H3ATTN_E_SHAPE;

    // the output view must not overlap itself
    const bool nhd_ok = o_stride_head >= 128 && o_stride_tok >= (h - 1) * o_stride_head + 128;
    const bool hnd_ok = o_stride_tok >= 128 && o_stride_head >= (n - 1) * o_stride_tok + 128;
    if (!(nhd_ok || hnd_ok)) return H3ATTN_E_SHAPE;

    const size_t in_b = h3attn_prepped_qk_bytes(p), sc_b = h3attn_scales_bytes(p);
    const Range orng = view_range(o, n, h, o_stride_tok, o_stride_head, 128, 2);
    if (overlap(orng, span(q_prep, in_b)) || overlap(orng, span(k_prep, in_b)) || overlap(orng, vrng))
        return H3ATTN_E_ALIAS;
    if (i8 && (overlap(orng, span(q_scales, sc_b)) || overlap(orng, span(k_scales, sc_b))))
        return H3ATTN_E_ALIAS;
    if (fp8v && overlap(orng, span(v_scales, h3attn_v_scales_bytes(p)))) return H3ATTN_E_ALIAS;
    if (rq && (overlap(orng, view_range(rq->q, n, h, rq->st, rq->sh, 128, 2)) ||
               overlap(orng, view_range(rq->gamma, 1, h, 0, rq->g_sh, 128, 2)) ||
               overlap(orng, span(rq->pos, (size_t)n * 3 * sizeof(int32_t)))))
        return H3ATTN_E_ALIAS;

    h3::FwdParams P{};
    P.q = q_prep; P.k = k_prep; P.qs = q_scales; P.ks = k_scales;
    P.v = static_cast<const uint16_t*>(v); P.v_st = fp8v ? 0 : v_stride_tok; P.v_sh = fp8v ? 0 : v_stride_head;
    P.vs = v_scales;
    P.o = static_cast<uint16_t*>(o); P.o_st = o_stride_tok; P.o_sh = o_stride_head;
    P.n = (int)n; P.h = (int)h; P.npad = (int)npad_of(p); P.nblk = (int)nblk_of(p);
    const int tile_rows = h3::forward_tile_rows(i8);
    P.qtiles = (int)((n + tile_rows - 1) / tile_rows);
    const int64_t total = h * P.qtiles;
    if (total > ((int64_t)1 << 28)) return H3ATTN_E_SHAPE;
    P.total = (int)total;
    P.per_xcd = (int)((total + 7) / 8);
    P.c = (float)((double)softmax_scale * 1.4426950408889634);
    if (rq) {
        P.q = nullptr;
        P.qs = nullptr;
        P.qraw = static_cast<const uint16_t*>(rq->q); P.q_st = rq->st; P.q_sh = rq->sh;
        P.gq = static_cast<const uint16_t*>(rq->gamma); P.g_sh = rq->g_sh;
        P.pos = rq->pos;
        P.eps = p->rms_eps;
        P.rho0 = rope_ratio(p, 0); P.rho1 = rope_ratio(p, 1); P.rho2 = rope_ratio(p, 2);
        P.sec0 = p->rope_sections[0]; P.sec1 = p->rope_sections[1]; P.sec2 = p->rope_sections[2];
        if (h3::launch_forward_fused_q(P, i8, static_cast<hipStream_t>(stream)) != hipSuccess) return H3ATTN_E_HIP;
        return H3ATTN_OK;
    }
    if (h3::launch_forward(P, i8, fp8v, static_cast<hipStream_t>(stream)) != hipSuccess) return H3ATTN_E_HIP;
    return H3ATTN_OK;
}

}  // namespace

extern "C" {

int h3attn_forward(const h3attn_problem* p,
                   const void* q_prep, const void* k_prep,
                   const float* q_scales, const float* k_scales,
                   const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                   void* o, int64_t o_stride_tok, int64_t o_stride_head,
                   float softmax_scale, void* stream) {
    return forward_common(p, q_prep, k_prep, q_scales, k_scales, false, v, v_stride_tok, v_stride_head,
                          nullptr, o, o_stride_tok, o_stride_head, softmax_scale, nullptr, stream);
}

int h3attn_forward_fused_q(const h3attn_problem* p,
                           const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                           const void* gamma_q, int64_t gamma_head_stride, const int32_t* pos_thw,
                           const void* k_prep,
                           const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                           void* o, int64_t o_stride_tok, int64_t o_stride_head,
                           float softmax_scale, void* stream) {
    const RawQ rq{q, q_stride_tok, q_stride_head, gamma_q, gamma_head_stride, pos_thw, false};
    return forward_common(p, nullptr, k_prep, nullptr, nullptr, false, v, v_stride_tok, v_stride_head, nullptr,
                          o, o_stride_tok, o_stride_head, softmax_scale, &rq, stream);
}

int h3attn_forward_fused_q_i8(const h3attn_problem* p,
                              const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                              const void* gamma_q, int64_t gamma_head_stride, const int32_t* pos_thw,
                              const void* k_codes, const float* k_scales,
                              const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                              void* o, int64_t o_stride_tok, int64_t o_stride_head,
                              float softmax_scale, void* stream) {
    const RawQ rq{q, q_stride_tok, q_stride_head, gamma_q, gamma_head_stride, pos_thw, true};
    return forward_common(p, nullptr, k_codes, nullptr, k_scales, false, v, v_stride_tok, v_stride_head, nullptr,
                          o, o_stride_tok, o_stride_head, softmax_scale, &rq, stream);
}

int h3attn_forward_fp8v(const h3attn_problem* p,
                        const void* q_prep, const void* k_prep,
                        const float* q_scales, const float* k_scales,
                        const void* v_codes, const float* v_scales,
                        void* o, int64_t o_stride_tok, int64_t o_stride_head,
                        float softmax_scale, void* stream) {
    return forward_common(p, q_prep, k_prep, q_scales, k_scales, true, v_codes, 0, 0, v_scales, o,
                          o_stride_tok, o_stride_head, softmax_scale, nullptr, stream);
}

int h3attn_prep_v_fp8(const h3attn_problem* p, const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                      void* v_codes, float* v_scales, void* stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if ((rc = check_in_view(v, v_stride_tok, v_stride_head))) return rc;
    if (!v_codes || !v_scales) return H3ATTN_E_NULL;
    if (!aligned(v_codes, 16) || !aligned(v_scales, 4)) return H3ATTN_E_ALIGN;
    const int64_t n = p->n_tokens, h = p->n_heads;
    const Range vin = view_range(v, n, h, v_stride_tok, v_stride_head, 128, 2);
    const Range cod = span(v_codes, h3attn_prepped_v_bytes(p));
    const Range sc = span(v_scales, h3attn_v_scales_bytes(p));
    if (overlap(cod, vin) || overlap(sc, vin) || overlap(cod, sc)) return H3ATTN_E_ALIAS;
    h3::PrepVParams P{};
    P.v = static_cast<const uint16_t*>(v); P.v_st = v_stride_tok; P.v_sh = v_stride_head;
    P.out = static_cast<uint8_t*>(v_codes); P.scales = v_scales;
    P.n = (int)n; P.h = (int)h; P.npad = (int)npad_of(p);
    if (h3::launch_prep_v(P, static_cast<hipStream_t>(stream)) != hipSuccess) return H3ATTN_E_HIP;
    return H3ATTN_OK;
}

int h3attn_calibrate_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream) {
    if (!out) return H3ATTN_E_NULL;
    if (!aligned(out, 4)) return H3ATTN_E_ALIGN;
    if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20)) return H3ATTN_E_SHAPE;
    if (h3::launch_mfma_calib(out, blocks, iters, static_cast<hipStream_t>(stream)) != hipSuccess)
        return H3ATTN_E_HIP;
    return H3ATTN_OK;
}

int h3attn_debug_scores_i32(const h3attn_problem* p, const void* q_codes, const void* k_codes,
                            int32_t head, int32_t row0, int32_t nrows, int32_t col0, int32_t ncols,
                            int32_t fp8v_layout, int32_t* out, void* stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (p->qk_format != H3ATTN_QK_I8_BLK64) return H3ATTN_E_UNSUPPORTED;
    if (!q_codes || !k_codes || !out) return H3ATTN_E_NULL;
    if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(out, 4)) return H3ATTN_E_ALIGN;
    const int64_t n = p->n_tokens;
    if (head < 0 || head >= p->n_heads || nrows < 1 || ncols < 1 || row0 < 0 || col0 < 0 ||
        (int64_t)row0 + nrows > n || (int64_t)col0 + ncols > n || (fp8v_layout != 0 && fp8v_layout != 1))
        return H3ATTN_E_SHAPE;
    const size_t in_b = h3attn_prepped_qk_bytes(p);
    const Range orng = span(out, (size_t)nrows * (size_t)ncols * sizeof(int32_t));
    if (overlap(orng, span(q_codes, in_b)) || overlap(orng, span(k_codes, in_b))) return H3ATTN_E_ALIAS;

    // the int8 forward's own parameters (no scales, V or output are read)
    h3::FwdParams P{};
    P.q = q_codes; P.k = k_codes;
    P.n = (int)n; P.h = p->n_heads; P.npad = (int)npad_of(p); P.nblk = (int)nblk_of(p);
    const int tile_rows = h3::forward_tile_rows(true);
    P.qtiles = (int)((n + tile_rows - 1) / tile_rows);
    P.s_out = out;
    P.s_head = head; P.s_row0 = row0; P.s_nrows = nrows; P.s_col0 = col0; P.s_ncols = ncols;
    P.s_qt0 = row0 / tile_rows;
    P.total = (row0 + nrows - 1) / tile_rows - P.s_qt0 + 1;
    P.per_xcd = (P.total + 7) / 8;
    P.kt0 = col0 / 64;
    P.kt1 = (col0 + ncols - 1) / 64;
    if (h3::launch_scores_i8(P, fp8v_layout != 0, static_cast<hipStream_t>(stream)) != hipSuccess)
        return H3ATTN_E_HIP;
    return H3ATTN_OK;
}

}  // extern "C"
