// Q/K RMSNorm + 3-axis split-half RoPE + head-major layout (+ optional int8 block
// quantisation) for gfx950.
//
// What is computed is the entry step of the packed-attention block: per-head
// RMSNorm then split-half RoPE of strided-NHD Q and K ("H3 Runtime Current
// State", Owned Performance Kernels: the fused entry kernel; "H3 Blackwell
// Runtime Plan", 2026-08-15 Handoff: fused Q/K RMS + RoPE + HND layout), with
// the int8 Q/K quantisation of the quantised attention path as an option
// ("H3 Runtime Current State", Owned Performance Kernels: Q quantization,
// K quantization).
//
// The step is HBM-bound (read Q and K once, write Q' and K' once).  Mapping:
// one 256-thread work-group owns a 64-token block for ALL heads.  Eight
// threads own one token row of a head: thread slot p holds the 16-byte chunk
// a(p) of the first half of a RoPE section and its partner chunk b(p) of the
// second half, so the rotation is thread-local and only the sum of squares
// is reduced across the eight lanes.  cos/sin of the thread's 8 angles are
// computed once per token and reused for every head and for both Q and K.
// The 64-token block is exactly one int8 scale block, so the block absmax is a
// work-group reduction.
//
// With K smoothing (the K-mean step of the same quantised path) the per-head,
// per-channel mean of K' is subtracted before K is quantised, in three passes
// (see PrepMode).
//
// Section widths that are even but not multiples of 16 (kGen) split chunks
// between section halves, so a lane's partner elements lie in other lanes'
// chunks.  Then each eight-lane group passes its row through LDS: the lanes
// load chunks p and p + 8 as usual and store them there, each lane gathers
// the 8 first-half elements of its generic slot (gen_slot_of) and their
// partners, normalises and rotates them with the same routine, scatters the
// bf16 results back, and reads chunks p and p + 8 of the result; from there
// on (stores, quantisation, K sums) the kernel runs as with chunk slots
// a = p, b = p + 8.
#include "common.h"
#include "params.h"
#include "rope_norm.h"

namespace h3 {



// kPrepI8Sums and kPrepI8Smooth are the first and last pass of K smoothing:
// the first writes Q' codes as kPrepI8 does, and for K' the per-block channel
// sums of its bf16 values (into the K code buffer, used as scratch); after
// ksum_reduce has turned them into the channel means, the last recomputes K'
// alone and quantises fl32(k - mean).
// kPrepBf16K and kPrepI8K write K' alone, bf16 or int8 codes + scales (for the
// forwards that compute Q' in their prologue).
enum PrepMode { kPrepBf16 = 0, kPrepI8 = 1, kPrepI8Sums = 2, kPrepI8Smooth = 3, kPrepBf16K = 4, kPrepI8K = 5 };

template <int kMode, bool kGen = false>
__global__ void __launch_bounds__(256) prep_kernel(PrepParams P) {
    constexpr bool kInt8 = kMode == kPrepI8 || kMode == kPrepI8Sums || kMode == kPrepI8Smooth || kMode == kPrepI8K;
    // Q' produced in this pass
    constexpr bool kDoQ = kMode != kPrepI8Smooth && kMode != kPrepBf16K && kMode != kPrepI8K;
    constexpr bool kQuantK = kMode == kPrepI8 || kMode == kPrepI8Smooth || kMode == kPrepI8K;
    const int tid = threadIdx.x;
    const int row = tid >> 3;            // 0..31
    const int p = tid & 7;               // slot
    const int t0 = blockIdx.x * 64;
    const Slot sl = kGen ? Slot{p, p + 8, 0, 0, 0} : slot_of(p, P.sec0, P.sec1, P.sec2);
    const GenSlot gs = gen_slot_of(p, P.sec0, P.sec1, P.sec2);     // kGen only

    int tok[2];
    bool valid[2];
    float cs[2][8], sn[2][8];
    double freq[8];
    if constexpr (kGen)
        rope_freqs_gen(gs, P.rho0, P.rho1, P.rho2, freq);
    else
        rope_freqs(sl, P.rho0, P.rho1, P.rho2, freq);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        tok[t] = t0 + row + 32 * t;
        valid[t] = tok[t] < P.n;
        if constexpr (kGen) {
            double pv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) pv[i] = valid[t] ? (double)P.pos[(int64_t)tok[t] * 3 + gs.ax[i]] : 0.0;
            rope_angles_t<true>(pv, freq, cs[t], sn[t]);
        } else {
            const double pv = valid[t] ? (double)P.pos[(int64_t)tok[t] * 3 + sl.axis] : 0.0;
            rope_angles(pv, freq, cs[t], sn[t]);
        }
    }

    // gamma of the slot's elements: chunks a and b, or (kGen) the generic
    // slot's first-half elements and their partners
    float gqa[8], gqb[8], gka[8], gkb[8];
    auto load_gamma = [&](int h) {
        if constexpr (kGen) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (kDoQ) {
                    gqa[i] = bf16_to_f32(P.gq[h * P.g_sh + gs.e1[i]]);
                    gqb[i] = bf16_to_f32(P.gq[h * P.g_sh + gs.e2[i]]);
                }
                gka[i] = bf16_to_f32(P.gk[h * P.g_sh + gs.e1[i]]);
                gkb[i] = bf16_to_f32(P.gk[h * P.g_sh + gs.e2[i]]);
            }
        } else {
            if constexpr (kDoQ) {        // gamma_q is absent (NULL) when Q' is not produced
                unpack8(ld16(P.gq + h * P.g_sh + 8 * sl.a), gqa);
                unpack8(ld16(P.gq + h * P.g_sh + 8 * sl.b), gqb);
            }
            unpack8(ld16(P.gk + h * P.g_sh + 8 * sl.a), gka);
            unpack8(ld16(P.gk + h * P.g_sh + 8 * sl.b), gkb);
        }
    };
    load_gamma(0);

    // kGen: the row of this eight-lane group (bf16 bits), for the gather and
    // scatter; the lanes of a group are one wave's, whose LDS accesses run in
    // program order (the waits below also order them for the compiler)
    __shared__ uint16_t grow[kGen ? 32 : 1][kGen ? kHeadDim : 1];
    auto rot = [&](u32x4 ca, u32x4 cb, const float* ga, const float* gb, const float* c8, const float* s8,
                   u32x4& oa, u32x4& ob, float* ra, float* rb) {
        if constexpr (kGen) {
            uint16_t* rw = grow[row];
            *reinterpret_cast<u32x4*>(rw + 8 * sl.a) = ca;
            *reinterpret_cast<u32x4*>(rw + 8 * sl.b) = cb;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            float xa[8], xb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xa[i] = bf16_to_f32(rw[gs.e1[i]]);
                xb[i] = bf16_to_f32(rw[gs.e2[i]]);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            u32x4 ga4, gb4;
            float fa[8], fb[8];
            norm_rotate(xa, xb, ga, gb, c8, s8, P.eps, ga4, gb4, fa, fb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rw[gs.e1[2 * i]] = (uint16_t)(ga4[i] & 0xffff);
                rw[gs.e1[2 * i + 1]] = (uint16_t)(ga4[i] >> 16);
                rw[gs.e2[2 * i]] = (uint16_t)(gb4[i] & 0xffff);
                rw[gs.e2[2 * i + 1]] = (uint16_t)(gb4[i] >> 16);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            oa = *reinterpret_cast<const u32x4*>(rw + 8 * sl.a);
            ob = *reinterpret_cast<const u32x4*>(rw + 8 * sl.b);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            unpack8(oa, ra);
            unpack8(ob, rb);
        } else {
            float xa[8], xb[8];
            unpack8(ca, xa);
            unpack8(cb, xb);
            norm_rotate(xa, xb, ga, gb, c8, s8, P.eps, oa, ob, ra, rb);
        }
    };

    __shared__ float red[2][2][4];      // [head parity][q/k][wave]
    // K smoothing, first pass: one head's bf16 K' block as fp32, [token][channel]
    __shared__ float ksum_tile[kMode == kPrepI8Sums ? 64 : 1][kMode == kPrepI8Sums ? kHeadDim + 1 : 1];
    const int wave = tid >> 6;

    for (int h = 0; h < P.h; ++h) {
        if (P.g_sh != 0 && h > 0) load_gamma(h);
        u32x4 qa[2], qb[2], ka[2], kb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (valid[t]) {
                const uint16_t* qr = P.q + (int64_t)tok[t] * P.q_st + (int64_t)h * P.q_sh;
                const uint16_t* kr = P.k + (int64_t)tok[t] * P.k_st + (int64_t)h * P.k_sh;
                if constexpr (kDoQ) {
                    qa[t] = ld16(qr + 8 * sl.a);
                    qb[t] = ld16(qr + 8 * sl.b);
                } else {
                    qa[t] = qb[t] = u32x4{0, 0, 0, 0};
                }
                ka[t] = ld16(kr + 8 * sl.a);
                kb[t] = ld16(kr + 8 * sl.b);
            } else {
                qa[t] = qb[t] = ka[t] = kb[t] = u32x4{0, 0, 0, 0};
            }
        }
        float rq[2][16], rk[2][16];
        u32x4 oqa[2], oqb[2], oka[2], okb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if constexpr (kDoQ) {
                rot(qa[t], qb[t], gqa, gqb, cs[t], sn[t], oqa[t], oqb[t], rq[t], rq[t] + 8);
            } else {
                oqa[t] = oqb[t] = u32x4{0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < 16; ++i) rq[t][i] = 0.f;
            }
            rot(ka[t], kb[t], gka, gkb, cs[t], sn[t], oka[t], okb[t], rk[t], rk[t] + 8);
            if (!valid[t]) {
                oqa[t] = oqb[t] = oka[t] = okb[t] = u32x4{0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < 16; ++i) rq[t][i] = rk[t][i] = 0.f;
            }
        }
        const int64_t head_base = (int64_t)h * P.npad;
        if constexpr (!kInt8) {
            uint16_t* qo = static_cast<uint16_t*>(P.q_out);
            uint16_t* ko = static_cast<uint16_t*>(P.k_out);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int64_t r = (head_base + tok[t]) * kHeadDim;
                if constexpr (kDoQ) {
                    st16(qo + r + 8 * sl.a, oqa[t]);
                    st16(qo + r + 8 * sl.b, oqb[t]);
                }
                st16(ko + r + 8 * sl.a, oka[t]);
                st16(ko + r + 8 * sl.b, okb[t]);
            }
        } else {
            if constexpr (kMode == kPrepI8Smooth) {
                // quantiser input fl32(k - mean); rows past N stay zero
                float mu[16];
                const float* mh = P.k_mean + (int64_t)h * kHeadDim;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    mu[i] = mh[8 * sl.a + i];
                    mu[8 + i] = mh[8 * sl.b + i];
                }
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    if (valid[t])
#pragma unroll
                        for (int i = 0; i < 16; ++i) rk[t][i] = rk[t][i] - mu[i];
            }
            if constexpr (kMode == kPrepI8Sums) {
                // per-channel sum of the block's bf16 K' in token order, one fp32
                // addition at a time (the order the smoothing mean is defined in)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        ksum_tile[row + 32 * t][8 * sl.a + i] = rk[t][i];
                        ksum_tile[row + 32 * t][8 * sl.b + i] = rk[t][8 + i];
                    }
                __syncthreads();
                if (tid < kHeadDim && t0 < P.n) {
                    const int cnt = min(64, P.n - t0);
                    float acc = 0.f;
                    for (int i = 0; i < cnt; ++i) acc += ksum_tile[i][tid];
                    float* sums = static_cast<float*>(P.k_out);
                    sums[((int64_t)h * P.nblk + blockIdx.x) * kHeadDim + tid] = acc;
                }
                __syncthreads();
            }
            float mq = 0.f, mk = 0.f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    mq = fmaxf(mq, fabsf(rq[t][i]));
                    mk = fmaxf(mk, fabsf(rk[t][i]));
                }
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) {
                mq = fmaxf(mq, __shfl_xor(mq, s));
                mk = fmaxf(mk, __shfl_xor(mk, s));
            }
            if ((tid & 63) == 0) {
                red[h & 1][0][wave] = mq;
                red[h & 1][1][wave] = mk;
            }
            __syncthreads();
            float aq = red[h & 1][0][0], ak = red[h & 1][1][0];
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                aq = fmaxf(aq, red[h & 1][0][w]);
                ak = fmaxf(ak, red[h & 1][1][w]);
            }
            // IEEE fp32 divisions (correctly rounded: the library is compiled without fast-math)
            const float sq = aq / 127.0f, sk = ak / 127.0f;
            const float iq = aq > 0.f ? 127.0f / aq : 0.f;
            const float ik = ak > 0.f ? 127.0f / ak : 0.f;
            if (tid == 0 && t0 < P.n) {
                if constexpr (kDoQ) P.q_scales[(int64_t)h * P.nblk + blockIdx.x] = sq;
                if constexpr (kQuantK) P.k_scales[(int64_t)h * P.nblk + blockIdx.x] = sk;
            }
            int8_t* qo = static_cast<int8_t*>(P.q_out);
            int8_t* ko = static_cast<int8_t*>(P.k_out);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int64_t r = (head_base + tok[t]) * kHeadDim;
                if constexpr (kDoQ) {
                    st8(qo + r + 8 * sl.a, u32x2{quant4(rq[t], iq), quant4(rq[t] + 4, iq)});
                    st8(qo + r + 8 * sl.b, u32x2{quant4(rq[t] + 8, iq), quant4(rq[t] + 12, iq)});
                }
                if constexpr (kQuantK) {
                    st8(ko + r + 8 * sl.a, u32x2{quant4(rk[t], ik), quant4(rk[t] + 4, ik)});
                    st8(ko + r + 8 * sl.b, u32x2{quant4(rk[t] + 8, ik), quant4(rk[t] + 12, ik)});
                }
            }
        }
    }
}

// K smoothing, middle pass: mean[h][c] = (sum over blocks in order of the
// block sums) / N, one fp32 addition at a time; one thread per (head, channel)
__global__ void __launch_bounds__(256) ksum_reduce(const float* sums, float* mean, int h, int nblk, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= h * kHeadDim) return;
    const int head = i / kHeadDim, c = i % kHeadDim;
    const float* s = sums + (int64_t)head * nblk * kHeadDim + c;
    float acc = 0.f;
    int b = 0;
    // loads run ahead in groups of 16; the additions stay in block order
    for (; b + 16 <= nblk; b += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = s[(int64_t)(b + u) * kHeadDim];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += v[u];
    }
    for (; b < nblk; ++b) acc += s[(int64_t)b * kHeadDim];
    mean[i] = acc / (float)n;       // IEEE division (the library is compiled without fast-math)
}

// one prep pass in the chunk-slot form, or the generic one when a section
// width is not a multiple of 16
template <int kMode>
void launch_mode(const PrepParams& P, dim3 grid, hipStream_t stream) {
    if (sections_are_chunks(P.sec0, P.sec1, P.sec2))
        hipLaunchKernelGGL((prep_kernel<kMode, false>), grid, dim3(256), 0, stream, P);
    else
        hipLaunchKernelGGL((prep_kernel<kMode, true>), grid, dim3(256), 0, stream, P);
}

hipError_t launch_prep(const PrepParams& P, bool int8, hipStream_t stream) {
    (void)hipGetLastError();     // clear an error left by an earlier, unrelated call
    const dim3 grid(P.npad / 64);
    if (int8)
        launch_mode<kPrepI8>(P, grid, stream);
    else
        launch_mode<kPrepBf16>(P, grid, stream);
    return hipGetLastError();
}

hipError_t launch_prep_k(const PrepParams& P, bool int8, hipStream_t stream) {
    (void)hipGetLastError();     // clear an error left by an earlier, unrelated call
    const dim3 grid(P.npad / 64);
    if (int8)
        launch_mode<kPrepI8K>(P, grid, stream);
    else
        launch_mode<kPrepBf16K>(P, grid, stream);
    return hipGetLastError();
}

hipError_t launch_prep_ksmooth(const PrepParams& P, hipStream_t stream) {
    (void)hipGetLastError();     // clear an error left by an earlier, unrelated call
    const dim3 grid(P.npad / 64), block(256);
    launch_mode<kPrepI8Sums>(P, grid, stream);
    hipLaunchKernelGGL(ksum_reduce, dim3((P.h * kHeadDim + 255) / 256), block, 0, stream,
                       static_cast<const float*>(P.k_out), P.k_mean, P.h, P.nblk, P.n);
    launch_mode<kPrepI8Smooth>(P, grid, stream);
    return hipGetLastError();
}

}  // namespace h3
