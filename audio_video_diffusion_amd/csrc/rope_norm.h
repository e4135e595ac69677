// Per-row Q/K RMSNorm + 3-axis split-half RoPE shared by the prep kernel and
// the forward's fused-Q prologue, so both produce the same bits.
//
// Eight threads own one (token, head) row: thread slot p holds the 16-byte
// chunk a(p) of the first half of a RoPE section and its partner chunk b(p) of
// the second half ("H3 Blackwell Runtime Plan", Architecture: 3-axis RoPE;
// "H3 Runtime Current State", Owned Performance Kernels: split-half RoPE), so
// the rotation is thread-local and only the sum of squares crosses lanes.
#pragma once

#include "common.h"

namespace h3 {

struct Slot {
    int a, b;       // chunk index (of 16) of the first-half chunk and its partner
    int axis;       // 0 = t, 1 = h, 2 = w
    int j0;         // frequency index of element 0 of chunk a inside its section
    int width;      // section width s
};

__device__ __forceinline__ Slot slot_of(int p, int s0, int s1, int s2) {
    const int w[3] = {s0, s1, s2};
    int off = 0;
    Slot r{0, 0, 0, 0, 16};
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) {
        const int cnt = w[ax] / 16;          // first-half chunks of this section
        if (p >= 0 && p < cnt) {
            r.a = off / 8 + p;
            r.b = r.a + cnt;
            r.axis = ax;
            r.j0 = 8 * p;
            r.width = w[ax];
        }
        p -= cnt;
        off += w[ax];
    }
    return r;
}

// Any even section widths (the prep only): slot p takes the first-half
// elements k = 8p .. 8p+7 of the 64 that the three sections' first halves hold
// in order (t, then h, then w), and their partners.  Element i of the slot is
// head-dim index e1[i], angle index j[i] of section ax[i]; its partner is
// e1[i] + s/2.
struct GenSlot {
    int e1[8], e2[8], ax[8], j[8];
};

__device__ __forceinline__ GenSlot gen_slot_of(int p, int s0, int s1, int s2) {
    GenSlot g;
    const int h0 = s0 / 2, h1 = s1 / 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int k = 8 * p + i;
        const int ax = k < h0 ? 0 : k < h0 + h1 ? 1 : 2;
        const int j = ax == 0 ? k : ax == 1 ? k - h0 : k - h0 - h1;
        const int off = ax == 0 ? 0 : ax == 1 ? s0 : s0 + s1;
        const int half = (ax == 0 ? s0 : ax == 1 ? s1 : s2) / 2;
        g.e1[i] = off + j;
        g.e2[i] = off + j + half;
        g.ax[i] = ax;
        g.j[i] = j;
    }
    return g;
}

__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16lo_to_f32(v[i]);
        f[2 * i + 1] = bf16hi_to_f32(v[i]);
    }
}

// Sum over the 8-lane group of the calling lane (all 64 lanes active): lane
// swaps by DPP, l^1 and l^2 inside each quad, then the other quad of the
// group (row_half_mirror: any of its lanes holds the same quad sum).
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf,
                                                                 false));
}
__device__ __forceinline__ float sum8lanes(float v) {
    v += dpp<0xb1>(v);      // quad_perm [1,0,3,2]
    v += dpp<0x4e>(v);      // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);     // row_half_mirror
    return v;
}

// RMSNorm + rotation of one (token, head) pair of chunks; result rounded to bf16
// and returned both as packed words and as the rounded fp32 values.  Every
// rounding is spelled out (no contraction), so the prep kernel and the
// forward's prologue produce the same bits from the same inputs.  With
// kPostScale the fp32 result is multiplied by `post` before the one bf16
// rounding (the forward's fused prologue folds the logit scale in there).
template <bool kPostScale = false>
__device__ __forceinline__ void norm_rotate(const float* xa, const float* xb, const float* ga,
                                            const float* gb, const float* cs, const float* sn,
                                            float eps, u32x4& oa, u32x4& ob, float* ra, float* rb,
                                            float post = 1.0f) {
#pragma clang fp contract(off)
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ss = __builtin_fmaf(xa[i], xa[i], ss);
        ss = __builtin_fmaf(xb[i], xb[i], ss);
    }
    ss = sum8lanes(ss);
    const float rinv = rsqrtf(__builtin_fmaf(ss, 1.0f / kHeadDim, eps));
    float ya[8], yb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float u = (xa[i] * rinv) * ga[i];
        const float w = (xb[i] * rinv) * gb[i];
        ya[i] = __builtin_fmaf(u, cs[i], -(w * sn[i]));
        yb[i] = __builtin_fmaf(w, cs[i], u * sn[i]);
        if constexpr (kPostScale) {
            ya[i] = ya[i] * post;
            yb[i] = yb[i] * post;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        oa[i] = pack_bf16x2(ya[2 * i], ya[2 * i + 1]);
        ob[i] = pack_bf16x2(yb[2 * i], yb[2 * i + 1]);
        ra[2 * i] = bf16lo_to_f32(oa[i]);
        ra[2 * i + 1] = bf16hi_to_f32(oa[i]);
        rb[2 * i] = bf16lo_to_f32(ob[i]);
        rb[2 * i + 1] = bf16hi_to_f32(ob[i]);
    }
}

// Inverse frequencies theta^(-2j/s) of the slot's 8 angle indices j = j0 ..
// j0+7, as powers of rho = theta^(-2/s) (rho0..2: the t, h, w sections,
// computed once on the host in fp64): rho^j0 by binary powering, then one
// multiplication per step.  Relative error ~1e-15, far below what reaches
// the bf16 output; fixed operation order, so every kernel gets the same bits.
__device__ __forceinline__ void rope_freqs(const Slot& sl, double rho0, double rho1, double rho2, double* f) {
#pragma clang fp contract(off)
    const double rho = sl.axis == 0 ? rho0 : sl.axis == 1 ? rho1 : rho2;
    double acc = 1.0, b = rho;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {            // j0 < 64
        if ((sl.j0 >> bit) & 1) acc = acc * b;
        b = b * b;
    }
    f[0] = acc;
#pragma unroll
    for (int i = 1; i < 8; ++i) f[i] = f[i - 1] * rho;
}

// The generic slot's 8 inverse frequencies theta^(-2j/s): rho^j of each
// element's own section by binary powering.
__device__ __forceinline__ void rope_freqs_gen(const GenSlot& g, double rho0, double rho1, double rho2, double* f) {
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double rho = g.ax[i] == 0 ? rho0 : g.ax[i] == 1 ? rho1 : rho2;
        double acc = 1.0, b = rho;
#pragma unroll
        for (int bit = 0; bit < 6; ++bit) {        // j < 64
            if ((g.j[i] >> bit) & 1) acc = acc * b;
            b = b * b;
        }
        f[i] = acc;
    }
}

// cos/sin of the angles phi = pos * f[i].  phi is formed and reduced in fp64
// (with positions in the thousands an fp32 product alone is off by ~1e-4
// rad): k = rint(phi * 2/pi), r = phi - k pi/2 with one fused multiply-add,
// the Cody-Waite quadrant reduction with |r| <= pi/4; then r is rounded to
// fp32 and sin r, cos r come from their Taylor series through r^9 and r^10
// (truncation below 2e-9 on |r| <= pi/4, under fp32 rounding), evaluated by
// Horner's rule, and the quadrant k mod 4 swaps and negates them.
// kPerElement: pv holds one position per element (the generic slots, whose
// elements may belong to different sections).
template <bool kPerElement = false>
__device__ __forceinline__ void rope_angles_t(const double* pv, const double* f, float* cs, float* sn) {
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double phi = pv[kPerElement ? i : 0] * f[i];
        const double k = rint(phi * 0.636619772367581343076);                 // 2 / pi
        const float r = (float)__builtin_fma(-k, 1.57079632679489661923, phi); // pi / 2
        const int q = (int)__builtin_fma(-4.0, floor(k * 0.25), k);           // k mod 4, exact
        const float r2 = r * r;
        float sp = -1.0f / 362880.0f;
        sp = __builtin_fmaf(r2, sp, 1.0f / 5040.0f);
        sp = __builtin_fmaf(r2, sp, -1.0f / 120.0f);
        sp = __builtin_fmaf(r2, sp, 1.0f / 6.0f);
        const float s = __builtin_fmaf(-(r * r2), sp, r);   // r - r^3/6 + r^5/120 - ...
        float cp = -1.0f / 3628800.0f;
        cp = __builtin_fmaf(r2, cp, 1.0f / 40320.0f);
        cp = __builtin_fmaf(r2, cp, -1.0f / 720.0f);
        cp = __builtin_fmaf(r2, cp, 1.0f / 24.0f);
        cp = __builtin_fmaf(r2, cp, -0.5f);
        const float c = __builtin_fmaf(r2, cp, 1.0f);
        // sin/cos of r + q pi/2: odd q swaps them; sin is negated for q = 2, 3
        // and cos for q = 1, 2 (sign-bit flips)
        const bool odd = (q & 1) != 0;
        const uint32_t neg_s = (uint32_t)(q & 2) << 30, neg_c = (uint32_t)((q + 1) & 2) << 30;
        sn[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, odd ? c : s) ^ neg_s);
        cs[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, odd ? s : c) ^ neg_c);
    }
}
__device__ __forceinline__ void rope_angles(double pv, const double* f, float* cs, float* sn) {
    rope_angles_t<false>(&pv, f, cs, sn);
}

// The int8 code of each of v[0..3] at reciprocal scale inv (round to nearest
// even, clamped to [-127, 127]), packed little-endian: the per-block absmax
// quantiser of the int8 Q/K path ("H3 Runtime Current State", Owned
// Performance Kernels: Q quantization, K quantization), shared by the prep and
// the int8 forward's Q prologue so that both produce the same codes.
__device__ __forceinline__ uint32_t quant4(const float* v, float inv) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float c = __builtin_rintf(v[i] * inv);
        c = fminf(fmaxf(c, -127.f), 127.f);
        w |= (uint32_t)((int)c & 0xff) << (8 * i);
    }
    return w;
}

}  // namespace h3
