// Non-causal flash-style attention over the packed joint sequence, gfx950.
//
// Computes O = softmax(Q' K'^T * scale) V for every head over all N packed
// tokens, one softmax per query row, no padding keys ("H3 Blackwell Runtime
// Plan", Architecture and Non-Negotiable Validation).  Q'/K' come head-major
// from the prep step (bf16, or int8 codes with per-64-token fp32 scales as in
// the int8-QK path of "H3 Runtime Current State", Owned Performance Kernels);
// V is read through its token-major strides and O is written token-major.
//
// Work decomposition (one 256-thread work-group = 4 wave64s, one per SIMD):
// * a work-group owns 256 query rows of one head; each wave owns 64 rows as
//   two 32-row MFMA blocks and keeps its Q' rows in registers;
// * the work-group streams K'/V in tiles of 64 keys through double-buffered
//   LDS: K' as [key][d] rows (permuted, see kperm), V transposed to [d][key];
// * everything is computed transposed so that one lane owns one query column:
//     S^T (keys x queries) = K' Q'^T     with v_mfma_f32_32x32x16_bf16
//                                        (int8: v_mfma_i32_32x32x32_i8)
//     O^T (d x queries)   += V^T P^T     with v_mfma_f32_32x32x16_bf16
//   The row max and row sum of a query are then in-lane reductions plus one
//   exchange between lane l and l^32, and the rescale of O touches only the
//   lane's own accumulators;
// * K' rows are placed in LDS so that the 32x32 accumulator layout of S^T
//   (lane half h holds rows 8i+4h+j) directly yields, per lane, 8 consecutive
//   keys for each 16-key step of the P V product: P needs no lane movement;
// * online softmax in base 2 with the scale*log2(e) folded into one FMA; the
//   running max is only raised when it grows by more than 2^8 (exact: the
//   stale max cancels between numerator and denominator, P stays <= 256);
// * the blockIdx -> (head, query tile) map keeps the work-groups that one XCD
//   runs at a time on adjacent query tiles of one head, so K'/V tiles are
//   shared through that XCD's L2.
#include "common.h"
#include "params.h"

namespace h3 {


constexpr int kBM = 256;            // query rows per work-group
constexpr int kBN = 64;             // keys per tile
constexpr int kXcds = 8;
constexpr float kRescaleLog2 = 8.0f;

// LDS row pitches in bytes (16-byte pad keeps ds_read_b128 row groups conflict free)
template <bool kInt8> struct Lds {
    static constexpr int kRow = (kInt8 ? 128 : 256) + 16;    // K' row
    static constexpr int kBytes = kBN * kRow;
    static constexpr int vRow = kBN * 2 + 16;                 // V^T row (64 keys)
    static constexpr int vBytes = kHeadDim * vRow;
    static constexpr int stage = kBytes + vBytes;
};

// LDS row of key (0..63) of a tile: inverse of the accumulator row order, so
// that accumulator element 8s+e of lane half h is key 16s + 8h + e of its block.
__device__ __forceinline__ int kperm(int key) {
    const int blk = key >> 5, kk = key & 31;
    const int i = 2 * (kk >> 4) + ((kk >> 2) & 1);
    const int hh = (kk >> 3) & 1;
    return 32 * blk + 8 * i + 4 * hh + (kk & 3);
}

// ---- staging of one K'/V tile: global -> registers -> LDS ------------------

template <bool kInt8> struct Stage {
    u32x4 kreg[kInt8 ? 2 : 4];
    u32x4 vreg[4];
};

template <bool kInt8>
__device__ __forceinline__ void stage_load(Stage<kInt8>& st, const FwdParams& P, const uint8_t* khead,
                                           const uint16_t* vhead, int key0, int tid) {
    constexpr int rowB = kInt8 ? 128 : 256;
#pragma unroll
    for (int r = 0; r < (kInt8 ? 2 : 4); ++r) {
        const int g = tid + 256 * r;             // 16-byte chunk of the contiguous tile
        st.kreg[r] = ld16(khead + (int64_t)key0 * rowB + (int64_t)g * 16);
    }
    const int kg = tid & 15, dc = tid >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int key = key0 + 4 * kg + r;
        st.vreg[r] = key < P.n ? ld16(vhead + (int64_t)key * P.v_st + 8 * dc) : u32x4{0, 0, 0, 0};
    }
}

template <bool kInt8>
__device__ __forceinline__ void stage_store(const Stage<kInt8>& st, uint8_t* lds, int tid) {
    using L = Lds<kInt8>;
    constexpr int chunks = kInt8 ? 8 : 16;      // 16-byte chunks per K' row
#pragma unroll
    for (int r = 0; r < (kInt8 ? 2 : 4); ++r) {
        const int g = tid + 256 * r;
        const int key = g / chunks, ch = g % chunks;
        *reinterpret_cast<u32x4*>(lds + kperm(key) * L::kRow + ch * 16) = st.kreg[r];
    }
    uint8_t* vt = lds + L::kBytes;
    const int kg = tid & 15, dc = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // column pair (2i, 2i+1) of the chunk for keys 4kg..4kg+3
        const uint32_t a0 = st.vreg[0][i], a1 = st.vreg[1][i], a2 = st.vreg[2][i], a3 = st.vreg[3][i];
        const u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        const u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        const int d = 8 * dc + 2 * i;
        *reinterpret_cast<u32x2*>(vt + d * L::vRow + kg * 8) = lo;
        *reinterpret_cast<u32x2*>(vt + (d + 1) * L::vRow + kg * 8) = hi;
    }
}

// ---- S^T = K' Q'^T for one tile: S[kb][qb] is keys 32kb.. x queries 32qb.. --

__device__ __forceinline__ void qk_tile_bf16(const uint8_t* klds, const bf16x8 (&qreg)[2][8],
                                             f32x16 (&S)[2][2], int n32, int hh) {
    using L = Lds<false>;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        S[kb][0] = f32x16{};
        S[kb][1] = f32x16{};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(klds + (32 * kb + n32) * L::kRow + 32 * t + 16 * hh);
            S[kb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[0][t], S[kb][0], 0, 0, 0);
            S[kb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[1][t], S[kb][1], 0, 0, 0);
        }
    }
}

__device__ __forceinline__ void qk_tile_i8(const uint8_t* klds, const i32x4 (&qreg)[2][4],
                                           i32x16 (&S)[2][2], int n32, int hh) {
    using L = Lds<true>;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        S[kb][0] = i32x16{};
        S[kb][1] = i32x16{};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const i32x4 a = *reinterpret_cast<const i32x4*>(klds + (32 * kb + n32) * L::kRow + 32 * t + 16 * hh);
            S[kb][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[0][t], S[kb][0], 0, 0, 0);
            S[kb][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[1][t], S[kb][1], 0, 0, 0);
        }
    }
}

// Q' rows of one wave as MFMA B operands: lane (n32, hh) holds row q0+32qb+n32.
__device__ __forceinline__ void load_q_bf16(const uint8_t* qhead, int q0, int n32, int hh, bf16x8 (&qreg)[2][8]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int t = 0; t < 8; ++t)
            qreg[qb][t] = __builtin_bit_cast(bf16x8, ld16(qhead + (int64_t)(q0 + 32 * qb + n32) * 256 + 32 * t + 16 * hh));
}

__device__ __forceinline__ void load_q_i8(const uint8_t* qhead, int q0, int n32, int hh, i32x4 (&qreg)[2][4]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            qreg[qb][t] = __builtin_bit_cast(i32x4, ld16(qhead + (int64_t)(q0 + 32 * qb + n32) * 128 + 32 * t + 16 * hh));
}

// acc *= alpha with acc pinned to the accumulation registers (AGPRs): the rare
// rescale of the running output then never forces O into arch VGPRs.
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
    float tmp;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float x = acc[e];
        asm volatile("v_accvgpr_read_b32 %1, %0\n\t"
                     "v_mul_f32 %1, %1, %2\n\t"
                     "v_accvgpr_write_b32 %0, %1"
                     : "+a"(x), "=&v"(tmp) : "v"(alpha));
        acc[e] = x;
    }
}

// ---- online softmax + P V of one tile --------------------------------------

template <bool kMask>
__device__ __forceinline__ void softmax_pv(f32x16 (&S)[2][2], float coef, const uint8_t* vt,
                                           f32x16 (&O)[2][4], float (&m)[2], float (&l)[2],
                                           int key0, int n, int n32, int hh) {
    using L = Lds<false>;
    bf16x8 Pb[2][2][2];      // [qb][kb][s]
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        if constexpr (kMask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = key0 + 32 * kb + 16 * (e >> 3) + 8 * hh + (e & 7);
                    if (key >= n) S[kb][qb][e] = -INFINITY;
                }
        }
        float mx = S[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, S[kb][qb][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = mx * coef;
        if (__any(mnew > m[qb] + kRescaleLog2)) {
            const float mm = fmaxf(m[qb], mnew);
            const float alpha = __builtin_amdgcn_exp2f(m[qb] - mm);
            m[qb] = mm;
            l[qb] *= alpha;
#pragma unroll
            for (int c = 0; c < 4; ++c) scale_acc(O[qb][c], alpha);
        }
        const float mq = m[qb];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float p[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][qb][e], coef, -mq));
                if constexpr (kMask) {
                    // keys >= N: probability exactly 0 (also when coef == 0)
                    const int key = key0 + 32 * kb + 16 * (e >> 3) + 8 * hh + (e & 7);
                    if (key >= n) p[e] = 0.f;
                }
                rs += p[e];
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                u32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(p[8 * s + 2 * i], p[8 * s + 2 * i + 1]);
                Pb[qb][kb][s] = __builtin_bit_cast(bf16x8, w);
            }
        }
        l[qb] += rs;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (32 * c + n32) * L::vRow + 2 * (32 * kb + 16 * s + 8 * hh));
                O[0][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, Pb[0][kb][s], O[0][c], 0, 0, 0);
                O[1][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, Pb[1][kb][s], O[1][c], 0, 0, 0);
            }
}

__device__ __forceinline__ void s_to_float(const i32x16 (&Si)[2][2], f32x16 (&S)[2][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int e = 0; e < 16; ++e) S[kb][qb][e] = (float)Si[kb][qb][e];
}

template <bool kInt8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
fwd_kernel(FwdParams P) {
    using L = Lds<kInt8>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::stage];

    const int vb = (blockIdx.x % kXcds) * P.per_xcd + blockIdx.x / kXcds;
    if (vb >= P.total) return;                     // whole work-group, before any barrier
    const int head = vb / P.qtiles;
    const int qt = vb % P.qtiles;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n32 = lane & 31, hh = lane >> 5;
    const int q0 = qt * kBM + wave * 64;

    constexpr int elt = kInt8 ? 1 : 2;
    const uint8_t* qhead = static_cast<const uint8_t*>(P.q) + (int64_t)head * P.npad * kHeadDim * elt;
    const uint8_t* khead = static_cast<const uint8_t*>(P.k) + (int64_t)head * P.npad * kHeadDim * elt;
    const uint16_t* vhead = P.v + (int64_t)head * P.v_sh;

    bf16x8 qb16[2][8];
    i32x4 qi8[2][4];
    float qscale = 0.f;
    if constexpr (kInt8) {
        load_q_i8(qhead, q0, n32, hh, qi8);
        qscale = q0 < P.n ? P.qs[(int64_t)head * P.nblk + q0 / kQuantBlock] : 0.f;
    } else {
        load_q_bf16(qhead, q0, n32, hh, qb16);
    }

    f32x16 O[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int c = 0; c < 4; ++c) O[qb][c] = f32x16{};
    float m[2] = {-INFINITY, -INFINITY};
    float l[2] = {0.f, 0.f};

    const int ntiles = (P.n + kBN - 1) / kBN;
    const bool ragged = (P.n % kBN) != 0;

    Stage<kInt8> st;
    stage_load<kInt8>(st, P, khead, vhead, 0, tid);
    stage_store<kInt8>(st, lds, tid);
    __syncthreads();

    // S^T of one tile (bf16 or dequantised int8) and its logit coefficient
    auto scores = [&](const uint8_t* cur, int kt, f32x16 (&S)[2][2]) -> float {
        if constexpr (kInt8) {
            i32x16 Si[2][2];
            qk_tile_i8(cur, qi8, Si, n32, hh);
            s_to_float(Si, S);
            return P.c * qscale * P.ks[(int64_t)head * P.nblk + kt];
        } else {
            qk_tile_bf16(cur, qb16, S, n32, hh);
            return P.c;
        }
    };

    // all full tiles but the last: no key mask; the next tile is prefetched
    for (int kt = 0; kt + 1 < ntiles; ++kt) {
        uint8_t* cur = lds + (kt & 1) * L::stage;
        stage_load<kInt8>(st, P, khead, vhead, (kt + 1) * kBN, tid);
        f32x16 S[2][2];
        const float coef = scores(cur, kt, S);
        softmax_pv<false>(S, coef, cur + L::kBytes, O, m, l, kt * kBN, P.n, n32, hh);
        stage_store<kInt8>(st, lds + ((kt + 1) & 1) * L::stage, tid);
        __syncthreads();
    }
    // last tile: keys >= N are masked when N is not a multiple of the tile
    {
        const int kt = ntiles - 1;
        uint8_t* cur = lds + (kt & 1) * L::stage;
        f32x16 S[2][2];
        const float coef = scores(cur, kt, S);
        if (ragged)
            softmax_pv<true>(S, coef, cur + L::kBytes, O, m, l, kt * kBN, P.n, n32, hh);
        else
            softmax_pv<false>(S, coef, cur + L::kBytes, O, m, l, kt * kBN, P.n, n32, hh);
    }

    // epilogue: O^T / l -> bf16, lane (n32, hh) holds d = 32c + 8i + 4hh + j of its query
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = l[qb] + __shfl_xor(l[qb], 32);
        const float inv = 1.0f / lt;
        const int q = q0 + 32 * qb + n32;
        if (q < P.n) {
            uint16_t* orow = P.o + (int64_t)q * P.o_st + (int64_t)head * P.o_sh;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x2 w = {pack_bf16x2(O[qb][c][4 * i] * inv, O[qb][c][4 * i + 1] * inv),
                                     pack_bf16x2(O[qb][c][4 * i + 2] * inv, O[qb][c][4 * i + 3] * inv)};
                    st8(orow + 32 * c + 8 * i + 4 * hh, w);
                }
        }
    }
}

// ---- exact int32 scores of the int8 path (test hook), same tile routine -----


__global__ void __launch_bounds__(256) scores_i8_kernel(ScoreParams P) {
    using L = Lds<true>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[L::kBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n32 = lane & 31, hh = lane >> 5;
    const int qbase = (P.row0 / kBM) * kBM + blockIdx.y * kBM;
    const int kbase = (P.col0 / kBN) * kBN + blockIdx.x * kBN;
    const int q0 = qbase + wave * 64;

    i32x4 qreg[2][4];
    load_q_i8(P.qhead, q0, n32, hh, qreg);
    for (int r = 0; r < 2; ++r) {                    // same placement as the forward staging
        const int g = tid + 256 * r;
        const int key = g / 8, ch = g % 8;
        *reinterpret_cast<u32x4*>(lds + kperm(key) * L::kRow + ch * 16) =
            ld16(P.khead + (int64_t)(kbase + key) * 128 + ch * 16);
    }
    __syncthreads();
    i32x16 S[2][2];
    qk_tile_i8(lds, qreg, S, n32, hh);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int q = q0 + 32 * qb + n32;
                const int key = kbase + 32 * kb + 16 * (e >> 3) + 8 * hh + (e & 7);
                const int r = q - P.row0, c = key - P.col0;
                if (r >= 0 && r < P.nrows && c >= 0 && c < P.ncols)
                    P.out[(int64_t)r * P.ncols + c] = S[kb][qb][e];
            }
}

hipError_t launch_forward(const FwdParams& P, bool int8, hipStream_t stream) {
    (void)hipGetLastError();     // clear an error left by an earlier, unrelated call
    dim3 grid(kXcds * P.per_xcd), block(256);
    if (int8)
        hipLaunchKernelGGL(fwd_kernel<true>, grid, block, 0, stream, P);
    else
        hipLaunchKernelGGL(fwd_kernel<false>, grid, block, 0, stream, P);
    return hipGetLastError();
}

hipError_t launch_scores_i8(const ScoreParams& P, hipStream_t stream) {
    (void)hipGetLastError();     // clear an error left by an earlier, unrelated call
    const int r_lo = (P.row0 / kBM) * kBM, c_lo = (P.col0 / kBN) * kBN;
    const int ry = (P.row0 + P.nrows - r_lo + kBM - 1) / kBM;
    const int cx = (P.col0 + P.ncols - c_lo + kBN - 1) / kBN;
    hipLaunchKernelGGL(scores_i8_kernel, dim3(cx, ry), dim3(256), 0, stream, P);
    return hipGetLastError();
}

}  // namespace h3
