// Non-causal flash-style attention over the packed joint sequence, gfx950.
//
// Computes O = softmax(Q' K'^T * scale) V for every head over all N packed
// tokens, one softmax per query row, no padding keys ("H3 Blackwell Runtime
// Plan", Architecture and Non-Negotiable Validation).  Q'/K' come head-major
// from the prep step (bf16, or int8 codes with per-64-token fp32 scales as in
// the int8-QK path of "H3 Runtime Current State", Owned Performance Kernels);
// V is read through its token-major strides and O is written token-major.
//
// Work decomposition (fwd8_kernel, bf16 and int8 Q/K):
// * a work-group of eight wave64s owns 256 query rows of one head; each wave
//   owns one 32-row block and keeps its Q' rows in registers.  Waves w and
//   w+4 share a SIMD: per wave the state is small (O^T in 64 AGPRs), so two
//   waves fit each SIMD's register file and the hardware overlaps one wave's
//   softmax with the other's matrix-core work.  The int8 forms run twelve
//   waves and 384 rows instead, three waves per SIMD (see kW);
// * the work-group streams K'/V in tiles of 64 keys through four LDS stages,
//   fetched three tiles ahead with buffer -> LDS DMA (buffer_load_dwordx4 ...
//   lds: 1 KB per wave instruction, no registers in between; waves 0..7 each
//   move 8 of the 64 rows).  K' rows land permuted, V rows stay row-major; 16-byte
//   chunks are XOR-swizzled so the operand reads hit every LDS bank.  One
//   barrier per tile (the separate-prep eight-wave forms stagger it between
//   the two waves of a SIMD and fetch two tiles ahead: kStagger);
// * everything is computed transposed so that one lane owns one query column:
//     S^T (keys x queries) = K' Q'^T     with v_mfma_f32_32x32x16_bf16
//                                        (int8: v_mfma_i32_32x32x32_i8)
//     O^T (d x queries)   += V^T P^T     with v_mfma_f32_32x32x16_bf16
//   The row max and row sum of a query are in-lane reductions plus one
//   exchange between lane l and l^32 (v_permlane32_swap), and the rescale of
//   O touches only the lane's own accumulators.  V^T operands are read from
//   the row-major V tile with ds_read_b64_tr_b16, which transposes as it
//   reads;
// * K' rows are placed in LDS so that the 32x32 accumulator layout of S^T
//   (lane half h holds rows 8i+4h+j) directly yields, per lane, 8 consecutive
//   keys for each 16-key step of the P V product: P needs no lane movement;
// * online softmax in base 2: one fp32 FMA per score applies scale*log2(e)
//   (times s_q*s_k in int8 mode) and subtracts the running max m, then exp2
//   (the fused bf16 form carries the scale in Q' and starts each Q'K'^T
//   chain from -m, so its scores go to exp2 as they are).
//   The running max is only raised when it grows by more than 2^8 (exact: the
//   stale max cancels between numerator and denominator, P stays <= 256).  The
//   row sum adds the bf16-rounded P that the P V product uses, two at a time
//   with a bf16 dot product;
// * the blockIdx -> (head, query tile) map keeps the work-groups that one XCD
//   runs at a time on adjacent query tiles of one head, so K'/V tiles are
//   shared through that XCD's L2 (int8 K': plain order, see the kernel).
//
// The int8 instantiations also run as the scores test hook (kScores): the
// same Q'K'^T path, with the exact int32 scores of a window written out.
#include <cfloat>
#include <type_traits>

#include "common.h"
#include "params.h"
#include "rope_norm.h"
#include "h3attn_phase_timing.h"

namespace h3 {

constexpr int kBM = 256;            // query rows per work-group of eight waves
constexpr int kBN = 64;             // keys per tile
constexpr int kXcds = 8;
constexpr float kRescaleLog2 = 8.0f;
// A lane's tile row sum (32 keys) at most this bounds each of its P by it, so
// every logit is at most 7 = log2(128) above the running max: no raise needed.
constexpr float kSumCheck = 128.0f;
// The same for the FP8 P.V form, whose P' carries the factor 2^0.8:
// 200 < 2^(7 + 0.8) = 222.9.
constexpr float kSumCheckFp8 = 200.0f;

// LDS tile sizes in bytes; four stages of each are in flight
constexpr int kStages = 4;          // LDS stages of the K'/V stream

// Tile-local key held by LDS row rho: the 32x32 accumulator row order
// (rows 8i + 4h + j) mapped so that accumulator element 8s+e of lane half h
// is key 16s + 8h + e of its 32-key block.
__device__ __forceinline__ int key_of_row(int rho) {
    const int blk = rho >> 5, r = rho & 31;
    const int i = r >> 3, hh = (r >> 2) & 1, j = r & 3;
    return 32 * blk + 16 * (i >> 1) + 8 * hh + 4 * (i & 1) + j;
}

// The same for the FP8 P V product, whose B operand gives each lane half 32
// consecutive keys: accumulator element e of block kb in lane half h is key
// 32h + 16kb + e, so LDS row 32kb + 8i + 4h + j holds key 32h + 16kb + 4i + j.
__device__ __forceinline__ int key_of_row_f8(int rho) {
    const int kb = rho >> 5, r = rho & 31;
    const int i = r >> 3, hh = (r >> 2) & 1, j = r & 3;
    return 32 * hh + 16 * kb + 4 * i + j;
}

// 16-byte chunk c of K' row rho sits in LDS slot c ^ k_swizzle(rho) of the row.
// An operand read (ds_read_b128) serves 16 lanes at a time, each taking 4 of
// the 64 four-byte banks; its 16 lanes read one chunk of 16 consecutive rows.
// bf16 rows (256 bytes) start on bank 0, so the slots of the 16 rows must
// differ: rho & 15.  Int8 rows (128 bytes) start on bank 0 (even rows) or 32
// (odd rows), so the slots must differ among the 8 rows of each parity:
// (rho >> 1) & 7.  (rho & 7 would leave rows rho and rho + 8 on the same banks.)
template <bool kInt8>
__device__ __forceinline__ int k_swizzle(int rho) {
    return kInt8 ? (rho >> 1) & 7 : rho & 15;
}

// Raw buffer resource for `base` (stride 0, no range limit in practice: every
// offset the kernel forms is inside the tensor).  Word 3 selects the 32-bit
// data format that gfx9 buffer loads need.
__device__ __forceinline__ u32x4 raw_rsrc(const void* base) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    r[2] = 0xFFFFFFFFu;
    r[3] = 0x00020000u;
    return r;
}

// One 16-byte-per-lane buffer -> LDS DMA: lane i's 16 bytes at rsrc + voff land
// at lds_dst + 16 i.  The per-lane offsets stay in registers for the whole
// kernel; only the scalar base moves from tile to tile.  Issued as asm so the
// compiler does not treat it as an LDS write it must wait for before later
// LDS reads: the kernel's own vmcnt + barrier protocol orders every stage's
// fill before its use.  M0 holds the LDS destination, and an LDS DMA reads M0
// one wait state after a scalar write to it (the compiler's own lowering of
// the buffer -> LDS builtin places the same s_nop 0 there): without it the
// load may take the previous M0 and land on the previous destination.
// The M0 clobber is declared so that the compiler keeps nothing of its own in
// M0 across the DMA; clang warns that M0 is a reserved register, which is
// exactly why it must be declared, so that one warning is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// lds_dst is the destination's LDS byte address (an integer, so that no
// generic-to-LDS pointer conversion with its null check is made per copy).
__device__ __forceinline__ void dma16_buf(const u32x4& rsrc, uint32_t voff, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_dst)) : "memory", "m0");
}
// The same with a scalar byte offset added to every lane's offset (both
// non-negative, their sum below 2^32).
__device__ __forceinline__ void dma16_buf_so(const u32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_dst)),
                    "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
#pragma clang diagnostic pop

// ---- S^T = K' Q'^T ---------------------------------------------------------

// S accumulates in arch VGPRs (the softmax reads it with VALU ops) while Q'
// stays in AGPRs: these MFMAs are issued as inline asm to pin the register
// classes.  The first of a chain writes an early-clobber destination (it must
// not overlap the A/B operands); the rest accumulate in place.
// A matrix-core product reads a register two wait states after a VALU write of
// it at the earliest (the compiler pads its own products so on gfx950), but it
// cannot see a product inside asm, and where it places the VALU moves that
// feed one (a start value, a Q' operand copied into an AGPR) depends on its
// register allocation: a build with another scheduler option put such a copy
// right before a product of the fused int8 chain and changed its results.
// Every asm product therefore starts with s_nop 1 (same process and box, all
// forms within +-0.2% except bf16 Q'/K' with E4M3 V, 1.3% faster; outputs
// bit-identical).
__device__ __forceinline__ void mfma_s(f32x16& d, const bf16x8& a, const bf16x8& b, bool first) {
    if (first)
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
    else
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// The chain's first product of the fused-Q form: it adds to c0, which holds
// -m in every element (the running max leaves with the start value).
__device__ __forceinline__ void mfma_s_from(f32x16& d, const bf16x8& a, const bf16x8& b, const f32x16& c0) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c0));
}

// The int8 form of mfma_s: int32 scores in arch VGPRs (the softmax converts
// them there), Q' codes in AGPRs.
// The chain's first product adds to c0 (the int8 forward passes the bits of
// 1.5 * 2^23 in every element; see kI8Bias).
__device__ __forceinline__ void mfma_s_i8(i32x16& d, const i32x4& a, const i32x4& b, bool first,
                                          const i32x16& c0) {
    if (first)
        asm("s_nop 1\n\tv_mfma_i32_32x32x32_i8 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c0));
    else
        asm("s_nop 1\n\tv_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// Tile-local key of accumulator element e of block kb for lane half hh.
__device__ __forceinline__ int key_of_elem(int kb, int e, int hh) {
    return 32 * kb + 16 * (e >> 3) + 8 * hh + (e & 7);
}

template <bool kFp8V>
__device__ __forceinline__ int key_of(int kb, int e, int hh) {
    return kFp8V ? 32 * hh + 16 * kb + e : key_of_elem(kb, e, hh);
}

// acc *= alpha with acc pinned to the accumulation registers (AGPRs): the rare
// rescale of the running output then never forces O into arch VGPRs.
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
    float tmp;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float x = acc[e];
        if (e == 0)      // wait states after the matrix core last wrote acc
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
                         "v_accvgpr_read_b32 %1, %0\n\t"
                         "v_mul_f32 %1, %1, %2\n\t"
                         "v_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(tmp) : "v"(alpha));
        else
            asm volatile("v_accvgpr_read_b32 %1, %0\n\t"
                         "v_mul_f32 %1, %1, %2\n\t"
                         "v_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(tmp) : "v"(alpha));
        acc[e] = x;
    }
}

// max / sum of x over lanes l and l ^ 32, in every lane: v_permlane32_swap
// exchanges the two lane halves on the VALU (no LDS round trip, which would
// queue behind the tile's operand reads)
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// the end of the tile loop: every copy has landed (the comment marks this
// one full wait in the generated code)
__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0) ; all copies landed" ::: "memory"); }

// Race-detection build (compiled with -DH3_DEBUG_SYNC=1 into a separate
// library): every LDS stage of the tile loop -- the buffer -> LDS fill, the
// K' operand reads, the V operand reads -- is closed by a wait for all of the
// wave's memory traffic and a work-group barrier, so no stage can overlap
// another.  Its outputs must equal the release build's bit for bit; a
// difference would expose an ordering the release protocol leaves open.
#ifndef H3_DEBUG_SYNC
#define H3_DEBUG_SYNC 0
#endif
constexpr bool kDebugSync = H3_DEBUG_SYNC != 0;
__device__ __forceinline__ void debug_stage_sync() {
    if constexpr (kDebugSync) {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
    }
}
// Phase-timing build (compiled with -DH3_PHASE_TIMING=1 into a third
// library, a measurement aid): every wave reads the shader clock (s_memtime)
// at the start of each key tile, after its Q'K'^T chain, after its softmax,
// after its last P V issue and after the tile's barrier, and at the ends of
// its prologue, loop and epilogue; lane 0 adds the wave's sums into
// g_phase_cycles (vector atomics) for its group of four waves (one wave per
// SIMD: waves 4g..4g+3).  The stamps' results are consumed after the barrier,
// so the waits they need fall there.  The release build compiles none of it.
#ifndef H3_PHASE_TIMING
#define H3_PHASE_TIMING 0
#endif
constexpr bool kPhaseTiming = H3_PHASE_TIMING != 0;
// per wave group: Q'K'^T, softmax, P V issue, barrier, tiles, prologue, loop,
// epilogue, waves (9 of kPhaseSlots)
constexpr int kPhaseSlots = 10, kPhaseGroups = 3;
#if H3_PHASE_TIMING
__device__ unsigned long long g_phase_cycles[kPhaseSlots * kPhaseGroups];
#endif
__device__ __forceinline__ uint64_t phase_clock() {
    if constexpr (kPhaseTiming) return __builtin_amdgcn_s_memtime();
    return 0;
}

// Wait until at most kOutstanding of this wave's DMA instructions are still in
// flight (vmcnt retires in issue order): with the newest fetches allowed
// outstanding, every older tile has landed.
template <int kOutstanding>
__device__ __forceinline__ void wait_vmem_upto() {
    static_assert(kOutstanding >= 0 && kOutstanding <= 16, "no vmcnt wait for this count");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kOutstanding) : "memory");
}

// ============================================================================
// The forward kernel (see the file comment).
// ============================================================================
template <bool kInt8, bool kFp8V, int kW>
struct DmaOffsets8 {
    static constexpr int kRowB = kInt8 ? 128 : 256;   // K' row bytes
    static constexpr int kDW = 8;                     // waves 0..7 copy (of 8 or 12)
    static constexpr int kRowsPW = 64 / kDW;          // K' rows moved per wave
    static constexpr int kN = kRowsPW * kRowB / 1024; // K' DMA instructions per wave
    static constexpr int kNV = kFp8V ? (128 / kDW) * 64 / 1024 : 2;   // V DMA instructions per wave
    // bf16 V: the second copy's offsets are the first's plus 4 rows (a scalar
    // offset), so only the first is kept
    static constexpr int kNVo = kFp8V ? kNV : 1;
    uint32_t k[kN], v[kNVo];
    __device__ __forceinline__ DmaOffsets8(int wave, int lane, int64_t v_st) {
        // wave w moves K' rows kRowsPW * w ...: 8 (int8) or 4 (bf16) rows per instruction
        constexpr int cpr = kRowB / 16, rpi = 64 / cpr;
#pragma unroll
        for (int r = 0; r < kN; ++r) {
            const int rho = kRowsPW * wave + rpi * r + lane / cpr;
            const int c = (lane % cpr) ^ k_swizzle<kInt8>(rho);
            k[r] = (uint32_t)((kFp8V ? key_of_row_f8(rho) : key_of_row(rho)) * kRowB + c * 16);
        }
        if constexpr (kFp8V) {
            // E4M3 V^T tile [128 d][64 keys]: wave w moves d-rows 16 w ...,
            // 16 per instruction; LDS slot s of row d holds 16-byte chunk s ^ ((d >> 2) & 3)
#pragma unroll
            for (int r = 0; r < kNV; ++r) {
                const int d = (128 / kDW) * wave + 16 * r + (lane >> 2);
                const int c = (lane & 3) ^ ((d >> 2) & 3);
                v[r] = (uint32_t)(d * 64 + c * 16);
            }
        } else {
            // wave w moves V rows 8 w + 4 r + lane / 16, r = 0, 1 (the chunk
            // swizzle is the same for both r)
            const uint32_t rs = (uint32_t)(v_st * 2);
            const int kappa = 8 * wave + (lane >> 4);
            const int c = (lane & 15) ^ (4 * (kappa & 3));
            v[0] = (uint32_t)kappa * rs + c * 16;
        }
    }
};

// Int8 scores: |S| <= 127 * 127 * 128 < 2^22, so an int32 accumulator that
// starts at the bit pattern of 1.5 * 2^23 ends holding the fp32 value
// 1.5 * 2^23 + S exactly (the magic-number conversion), and no per-score
// int -> float conversion is needed.  The bias is taken out of the row max
// exactly (a subtraction of nearby values) and out of each logit together
// with the running max, in the FMA that applies the scale: one constant per
// tile, fl(1.5 * 2^23 * coef + m), whose rounding (at most 0.75 * coef, under
// one unit of S) is common to every score of the row in that tile.
constexpr float kI8Bias = 12582912.0f;             // 1.5 * 2^23
constexpr int32_t kI8BiasBits = 0x4b400000;

// log2 of the factor applied to P before it is rounded to E4M3: the lazily
// rescaled P is at most 2^8, times 2^0.8 stays below 448, E4M3's largest
// finite value, so more of P's range lands on normal E4M3 numbers.  The
// factor multiplies numerator and denominator alike and cancels.
constexpr float kPLog2Fp8 = 0.8f;

// kFuseQ: Q' is not read from memory but computed in the prologue from raw Q
// with the prep kernel's own per-row routine (rope_norm.h).  bf16 format
// (kFuseBf): rounded to bf16 once with the base-2 logit factor folded in; each
// Q'K'^T chain then starts from -m, so the scores leave the matrix core ready
// for exp2.  Int8 format: rounded to bf16 and quantised per 64-row block
// exactly as the prep does (codes and scales identical), then the int8 path.
// kW = 12 (int8 Q'/K', bf16 or E4M3 V, Q' from the prep or fused): twelve
// waves, three per SIMD, own 384 query rows.  The int8 state is small enough (Q' codes in
// 16 registers, K' operands half the bf16 size) for three waves in a SIMD's
// register file, 168 registers each; the K'/V stream then serves 384 queries
// instead of 256 (a third fewer L2 -> LDS bytes per FLOP) and each SIMD has a
// third wave to issue from.  Waves 0..7 issue the copies exactly as in the
// eight-wave form, so the LDS layout is unchanged, and each row's arithmetic
// is unchanged (outputs bit-identical).  The bf16 forms need more than 168
// registers and keep eight waves.
// kScores (int8 only; the test hook h3attn_debug_scores_i32): the kernel runs
// its own Q'K'^T path -- Q' codes in registers, the K' stream with its DMA
// offsets and LDS row permutation, the int8 product chain from the
// magic-number start -- over the key tiles of a window of one head, and
// writes the exact int32 scores of the window in place of the softmax and the
// P V product (no V is fetched).
template <bool kInt8, bool kFp8V, bool kFuseQ = false, int kW = 8, bool kScores = false>
__global__ void __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(kW / 4, kW / 4)))
fwd8_kernel(FwdParams P) {
    static_assert(!(kFuseQ && (kFp8V || kScores)), "the fused Q prologue: bf16 V");
    // fused Q in the bf16 format: Q' carries the logit scale and the chains start
    // from -m (the int8 form quantises Q' as the prep does and runs the int8 path)
    constexpr bool kFuseBf = kFuseQ && !kInt8;
    static_assert(kW == 8 || (kW == 12 && kInt8), "twelve waves: int8 Q'/K' only");
    static_assert(!kScores || kInt8, "the scores hook covers the int8 Q'K'^T path");
    constexpr int kBMw = 32 * kW;                  // query rows per work-group
    using D = DmaOffsets8<kInt8, kFp8V, kW>;
    constexpr int kKTileB = kBN * D::kRowB;        // 16 KB (bf16) or 8 KB (int8)
    constexpr int kVTileB = kBN * (kFp8V ? 128 : 256);   // 8 KB (E4M3) or 16 KB (bf16)
    constexpr int kDma8 = D::kN + (kScores ? 0 : D::kNV);   // DMA instructions per wave per tile
    // Staggered barrier (the eight-wave bf16 Q'/K' forms with Q' from the
    // prep): waves 4..7 take the per-tile barrier between their softmax and
    // their P V product instead of after it, so after each barrier they run
    // P V of tile j while waves 0..3 start Q'K'^T of tile j + 1: the two waves
    // of each SIMD stay half a tile apart.  Each row's arithmetic is unchanged
    // (outputs bit-identical).  A lagging wave still reads V of tile j after
    // the barrier that ends tile j, so the stage of tile j may only be
    // refilled after the next barrier: tiles are fetched two ahead instead of
    // three.  The SIMD's issue arbiter favours the older wave (0..3), which
    // starved the lagging wave's P V behind the other's Q'K'^T chain; with
    // bf16 V the lagging wave runs its P V at raised issue priority.  Same
    // process and box, 129,410 tokens, against the common barrier: bf16 Q'/K'
    // with E4M3 V -2.8% (the raised priority made it +5.5%), bf16 Q'/K' and V
    // -1.5 to -2.2% (+2.9% without the raised priority); the fused-Q form was
    // level with it (+0.4 to -0.5%) and keeps the common barrier, as do the
    // twelve-wave int8 forms.  With the older group lagging instead (its P V
    // then wins the arbitration unaided) every form was 4-8% slower.
    constexpr bool kStagger = kW == 8 && !kInt8 && !kScores && !kFuseQ;
    // tiles fetched ahead of the one being computed
    constexpr int kAhead = kStagger ? 2 : 3;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * (kKTileB + kVTileB)];

    // blockIdx -> (head, query tile).  bf16 K': XCD-aware (work-group b runs on
    // XCD b mod 8, which takes a contiguous range, so the ~32 work-groups of an
    // XCD stream one head's K'/V through its L2).  int8 K': plain order (all
    // XCDs on the same head at once), measured 2% faster there; the int8 tiles
    // are half the size and the XCD-aware order missed L2 unevenly.
    const int vb = kInt8 ? (int)blockIdx.x : (blockIdx.x % kXcds) * P.per_xcd + blockIdx.x / kXcds;
    if (vb >= P.total) return;
    // scores hook: work-group b takes query tile s_qt0 + b of head s_head
    const int head = kScores ? P.s_head : vb / P.qtiles;
    const int qt = kScores ? P.s_qt0 + vb : vb % P.qtiles;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31, hh = lane >> 5;
    const int q0 = qt * kBMw + wave * 32;
    const int n = P.n;
    // phase timing (kPhaseTiming only): kernel start, tile-phase sums, loop bounds
    [[maybe_unused]] const uint64_t ph_k0 = phase_clock();
    [[maybe_unused]] uint64_t ph_sum[4] = {0, 0, 0, 0}, ph_l0 = 0, ph_l1 = 0, ph_tiles = 0;

    const uint8_t* qhead = static_cast<const uint8_t*>(P.q) + (int64_t)head * P.npad * D::kRowB;
    const uint8_t* khead = static_cast<const uint8_t*>(P.k) + (int64_t)head * P.npad * D::kRowB;
    const uint8_t* vhead = kFp8V ? reinterpret_cast<const uint8_t*>(P.v) + (int64_t)head * P.npad * 128
                                 : reinterpret_cast<const uint8_t*>(P.v + (int64_t)head * P.v_sh);
    auto kbuf = [&](int j) { return lds + (j % kStages) * kKTileB; };
    // the same by stage index (a compile-time constant in the unrolled loop)
    auto kbuf_st = [&](int st) { return lds + st * kKTileB; };
    auto vbuf_st = [&](int st) { return lds + kStages * kKTileB + st * kVTileB; };
    auto vbuf = [&](int j) { return lds + kStages * kKTileB + (j % kStages) * kVTileB; };
    // the same stages as LDS byte addresses, for the copies' M0
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    auto kbuf_addr = [&](int j) { return lds_addr + (uint32_t)((j % kStages) * kKTileB); };
    auto vbuf_addr = [&](int j) { return lds_addr + (uint32_t)(kStages * kKTileB + (j % kStages) * kVTileB); };

    // this wave's 32 query rows as MFMA B operands
    using QOp = typename std::conditional<kInt8, i32x4, bf16x8>::type;
    constexpr int kSteps = kInt8 ? 4 : 8;          // d-steps of 32 (int8) or 16 (bf16)
    QOp q[kSteps];
    if constexpr (!kFuseQ) {
#pragma unroll
        for (int t = 0; t < kSteps; ++t)
            // rows past the padded tensor (384-row tiles) load row npad - 1: never stored
            q[t] = __builtin_bit_cast(QOp, ld16(qhead + (int64_t)min(q0 + n32, P.npad - 1) * D::kRowB + 32 * t + 16 * hh));
    }
    // Fused Q: thread (r = tid / 8, slot tid % 8) prepares rows r + kBMw / 4 * ps,
    // ps = 0..3, of the work-group's kBMw; its raw Q chunks, positions, gamma
    // and the slot's RoPE frequencies are loaded here, before the K'/V stream
    // starts (see the wait below).
    constexpr int kPsRows = kBMw / 4;              // rows per ps: 64 or 96
    const Slot fsl = slot_of(tid & 7, P.sec0, P.sec1, P.sec2);
    u32x4 fqa[4], fqb[4], fga, fgb;
    double fpv[4], ffreq[8];
    if constexpr (kFuseQ) {
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
            const int tok = qt * kBMw + kPsRows * ps + (tid >> 3);
            if (tok < n) {
                const uint16_t* qr = P.qraw + (int64_t)tok * P.q_st + (int64_t)head * P.q_sh;
                fqa[ps] = ld16(qr + 8 * fsl.a);
                fqb[ps] = ld16(qr + 8 * fsl.b);
                fpv[ps] = (double)P.pos[(int64_t)tok * 3 + fsl.axis];
            } else {
                fqa[ps] = fqb[ps] = u32x4{0, 0, 0, 0};
                fpv[ps] = 0.0;
            }
        }
        fga = ld16(P.gq + (int64_t)head * P.g_sh + 8 * fsl.a);
        fgb = ld16(P.gq + (int64_t)head * P.g_sh + 8 * fsl.b);
        rope_freqs(fsl, P.rho0, P.rho1, P.rho2, ffreq);
    }
    float qscale = 1.f;
    i32x16 bias16;
#pragma unroll
    for (int e = 0; e < 16; ++e) bias16[e] = kI8BiasBits;
    // A matrix-core product reads its C operand late, while the wave issues
    // on: a write to those registers within a few wait states of the product
    // (up to 15 for a 32x32 product) can reach it first.  The compiler cannot
    // see that for a product in asm; it would rebuild the chain-start values
    // (bias16 here, negm in the fused form) before each chain and hand their
    // registers to other values right after it.  Made opaque (here, or for
    // the fused int8 form after its prologue, which needs the registers) and
    // used again after the tile loop, they stay in registers, untouched by
    // anything but their own updates, for the whole loop.
    if constexpr (!(kFuseQ && kInt8)) asm volatile("" : "+v"(bias16));
    if constexpr (kInt8 && !kScores && !kFuseQ) qscale = q0 < n ? P.qs[(int64_t)head * P.nblk + q0 / kQuantBlock] : 0.f;
    // K block scales through the constant address space: one scalar load per
    // tile, counted by lgkmcnt.  A vector load would be waited for with
    // vmcnt(0), which also drains the buffer -> LDS prefetch.
    typedef const __attribute__((address_space(4))) float* const_f32_ptr;
    const const_f32_ptr kscale = kInt8 ? (const_f32_ptr)(P.ks + (int64_t)head * P.nblk) : nullptr;
    // All loads above complete here, and the compiler knows it.  Otherwise its
    // wait-count bookkeeping carries the Q' loads into the tile loop as possibly
    // outstanding and waits for them with vmcnt(7..0) between the Q K^T
    // products of every tile; vmcnt also counts the buffer -> LDS copies (asm,
    // invisible to it), so vmcnt(0) would wait for the tile fetched three ahead.
    __builtin_amdgcn_s_waitcnt(0);

    f32x16 O[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) O[cc] = f32x16{};
    float m = -INFINITY, l = 0.f;
    // kFuseBf: Q' carries the base-2 logit scale, and every Q'K'^T chain starts
    // from -mch (negm), so the scores come out as logit - mch, ready for exp2.
    // mch is the running max except before the first tile (m = -inf, mch = 0).
    float mch = 0.f;
    f32x16 negm = f32x16{};
    if constexpr (kFuseBf) asm volatile("" : "+v"(negm));     // see bias16

    const int ntiles = (n + kBN - 1) / kBN;
    // key tiles jb..last run (the scores hook: the tiles of its key window)
    const int jb = kScores ? P.kt0 : 0;
    const int last = kScores ? P.kt1 : ntiles - 1;
    const bool ragged = (n % kBN) != 0 && last == ntiles - 1;

    const D dmo(wave & 7, lane, P.v_st);     // waves 8..11 copy nothing
    float ks_cur = kInt8 && !kScores ? kscale[0] : 1.f;
    auto fetch = [&](int t) {
        if constexpr (kW > D::kDW)
            if (wave >= D::kDW) return;
        const int kt = min(t, last);
        const u32x4 kr = raw_rsrc(khead + (int64_t)kt * kKTileB);
#pragma unroll
        for (int r = 0; r < D::kN; ++r)
            dma16_buf(kr, dmo.k[r], kbuf_addr(t) + (D::kRowsPW * wave + (kInt8 ? 8 : 4) * r) * D::kRowB);
        if constexpr (kScores) {
            // scores only: no V
        } else if constexpr (kFp8V) {
            // pad keys of the last tile are zero codes in memory: no clamp
            const u32x4 vr = raw_rsrc(vhead + (int64_t)kt * kVTileB);
#pragma unroll
            for (int r = 0; r < D::kNV; ++r) dma16_buf(vr, dmo.v[r], vbuf_addr(t) + 1024 * (D::kNV * wave + r));
        } else {
            const u32x4 vr = raw_rsrc(vhead + (int64_t)kt * kBN * P.v_st * 2);
            const uint32_t rs = (uint32_t)(P.v_st * 2);
            if (kt == last) {
                // the last tile's V rows past N are clamped to row N - 1 (their P
                // is 0): the offsets are formed here, from an opaque copy of the
                // lane index, rather than kept in registers through the loop
                const int kmax = n - 1 - last * kBN;
                int ln = lane;
                asm volatile("" : "+v"(ln));
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int kappa = 8 * wave + 4 * r + (ln >> 4);
                    const int c = (ln & 15) ^ (4 * (kappa & 3));
                    const uint32_t off = (uint32_t)min(kappa, kmax) * rs + c * 16;
                    dma16_buf(vr, off, vbuf_addr(t) + (8 * wave + 4 * r) * 256);
                }
            } else {
                dma16_buf(vr, dmo.v[0], vbuf_addr(t) + (8 * wave) * 256);
                dma16_buf_so(vr, dmo.v[0], 4 * rs, vbuf_addr(t) + (8 * wave + 4) * 256);
            }
        }
    };

    const int r16 = lane & 15, g16 = lane >> 4;
    const int rk = r16 >> 2;
    const int v_lane_off = kFp8V ? n32 * 64 : (8 * (g16 >> 1) + rk) * 256 + (2 * (g16 & 1) + ((r16 & 3) >> 1)) * 16 + 8 * (r16 & 1);
    const int v_sw = (n32 >> 2) & 3;               // E4M3 V^T chunk swizzle of this lane's rows
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

    // the end of a tile: this wave's copies of tile j + 1 have landed, then
    // the work-group barrier (after it, tile j + 1 is complete in LDS)
    auto tile_sync = [&]() {
        debug_stage_sync();
        wait_vmem_upto<(kAhead - 1) * kDma8>();
        __syncthreads();
    };
    const bool behind = kStagger && wave >= 4;
    // bf16 Q'/K' with E4M3 V issues a tile's copies after its Q'K'^T chain,
    // while the products run (same process and box, both orders: -1.1% and
    // -1.4%); the bf16-V forms were slower so (+0.7 to +1.3%), and the int8
    // forms spill.  Either way the copies refill the stage of tile j - 1
    // (j - 2 when staggered), which every wave has left at the last barrier.
    constexpr bool kLateFetch = kFp8V && !kInt8;
    auto tile = [&](int j, bool masked, int st) {
        [[maybe_unused]] const uint64_t ph0 = phase_clock();
        [[maybe_unused]] uint64_t ph1 = ph0, ph2 = ph0;
        if constexpr (!kLateFetch) fetch(j + kAhead);
        debug_stage_sync();
        // S^T of this wave's 32 queries: S[kb] = LDS rows 32kb..32kb+31
        f32x16 S[2];
        i32x16 Si[2];
        const uint8_t* kb_ = kbuf_st(st);
        if constexpr (kInt8) {
            i32x4 a[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int rho = 32 * kb + n32;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    a[kb][t] = *reinterpret_cast<const i32x4*>(kb_ + rho * 128 + (((2 * t + hh) ^ k_swizzle<true>(rho)) * 16));
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                mfma_s_i8(Si[0], a[0][t], q[t], t == 0, bias16);
                mfma_s_i8(Si[1], a[1][t], q[t], t == 0, bias16);
            }
            // wait states before the VALU reads the matrix core's results: 13, one
            // more than the 12 this compiler pads its own 32x32 products with on
            // gfx950 (s_nop 11 before a dependent VALU read)
            asm volatile("s_nop 7\n\ts_nop 4" : "+v"(Si[0]), "+v"(Si[1]));
            ph1 = phase_clock();
            debug_stage_sync();
            // the fp32 values 1.5 * 2^23 + S (kI8Bias).  Whole-vector bit casts: a
            // bit cast of a single vector element is miscompiled by this compiler
            // (every such read returns element 0).
            S[0] = __builtin_bit_cast(f32x16, Si[0]);
            S[1] = __builtin_bit_cast(f32x16, Si[1]);
        } else {
            bf16x8 a[2][8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int rho = 32 * kb + n32;
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    a[kb][t] = *reinterpret_cast<const bf16x8*>(kb_ + rho * 256 + (((2 * t + hh) ^ k_swizzle<false>(rho)) * 16));
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (kFuseBf && t == 0) {
                    mfma_s_from(S[0], a[0][t], q[t], negm);
                    mfma_s_from(S[1], a[1][t], q[t], negm);
                } else {
                    mfma_s(S[0], a[0][t], q[t], t == 0);
                    mfma_s(S[1], a[1][t], q[t], t == 0);
                }
            }
            if constexpr (kLateFetch) fetch(j + kAhead);
            asm volatile("s_nop 7\n\ts_nop 4" : "+v"(S[0]), "+v"(S[1]));      // as above
            ph1 = phase_clock();
            debug_stage_sync();
        }
        if constexpr (kScores) {
            // the exact int32 scores: the accumulator ends at 0x4b400000 + S
            // (kI8Bias), written for the window's rows and keys
            const int r = q0 + n32 - P.s_row0;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int c = j * kBN + key_of<kFp8V>(kb, e, hh) - P.s_col0;
                    if (r >= 0 && r < P.s_nrows && c >= 0 && c < P.s_ncols)
                        P.s_out[(int64_t)r * P.s_ncols + c] = Si[kb][e] - kI8BiasBits;
                }
        } else {
            // base-2 logit scale of this tile (int8: times the two block scales)
            float coef = P.c;
            if constexpr (kInt8) {
                coef = P.c * qscale * ks_cur;
                ks_cur = kscale[min(j + 1, last)];     // the next tile's scale, loaded a tile early
            }
            if (masked) {
                // keys >= N: the most negative finite score for the max, probability 0 below
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (j * kBN + key_of<kFp8V>(kb, e, hh) >= n) S[kb][e] = -FLT_MAX;
            }
            // P is formed from the running max m as it stands.  The row max of the
            // tile is only needed when m may have to be raised: a lane whose 32
            // probabilities sum to at most kSumCheck has every P <= kSumCheck, i.e.
            // every base-2 logit at most log2(kSumCheck) = 7 above m, one unit short
            // of the rescale threshold.  So the max is computed, and the raise
            // decided exactly as before, only for the (rare) tiles where some lane's
            // sum exceeds that bound, and for the ragged last tile; P is recomputed
            // only if m was raised.  The rescale decisions, hence the results, are
            // those of computing the max for every tile, as long as the logits stay
            // far below 2^20 in base-2 units (there fp32 rounding of m + 8 cannot
            // move a decision across the one-unit margin).
            auto raise_max = [&]() -> bool {
                float mx = S[0][0];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) mx = __builtin_fmaxf(mx, S[kb][e]);
                mx = kInt8 ? (max_halves(mx) - kI8Bias) * coef : kFuseBf ? max_halves(mx) + mch : max_halves(mx) * coef;
                if (__any(mx > m + kRescaleLog2)) {
                    const float mm = fmaxf(m, mx);
                    const float alpha = __builtin_amdgcn_exp2f(m - mm);
                    m = mm;
                    l *= alpha;
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) scale_acc(O[cc], alpha);
                    return true;
                }
                return false;
            };
            if constexpr (kFp8V) {
                // P' = 2^0.8 * P rounded to E4M3, 32 consecutive keys per lane half;
                // the row sum adds the fp32 P' before rounding
                i32x8 Pf;
                float rs[4];
                auto make_p = [&]() {
                    const float mb0 = m - kPLog2Fp8;
                    // int8: the score bias leaves with the max (kI8Bias)
                    const float mb = kInt8 ? __builtin_fmaf(kI8Bias, coef, mb0) : mb0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) rs[u] = 0.f;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int w4 = 0; w4 < 4; ++w4) {
                            float x[4];
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                const int e = 4 * w4 + u;
                                x[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][e], coef, -mb));
                                if (masked && j * kBN + key_of<true>(kb, e, hh) >= n) x[u] = 0.f;
                                rs[u] += x[u];
                            }
                            // the first conversion fills the low half and keeps the high half of
                            // its third operand, which the second overwrites: any live value
                            // serves there (a constant 0 would cost a register move per word)
                            int wd = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], __float_as_int(x[0]), false);
                            wd = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], wd, true);
                            Pf[4 * kb + w4] = wd;
                        }
                };
                make_p();
                float t = (rs[0] + rs[1]) + (rs[2] + rs[3]);
                // P' carries the factor 2^0.8: 2^7.64 = 200 < 2^(7 + 0.8)
                if (masked || __any(!(t <= kSumCheckFp8)))
                    if (raise_max()) {
                        make_p();
                        t = (rs[0] + rs[1]) + (rs[2] + rs[3]);
                    }
                l += t;
                ph2 = phase_clock();
                if (behind) tile_sync();
                // O^T += V^T P'^T: lane (n32, hh) reads d-row 32cc + n32, keys 32hh..32hh+31
                const uint8_t* vb_ = vbuf_st(st) + v_lane_off;
                const int s0 = ((2 * hh) ^ v_sw) * 16, s1 = ((2 * hh + 1) ^ v_sw) * 16;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const i32x4 lo = *reinterpret_cast<const i32x4*>(vb_ + 32 * 64 * cc + s0);
                    const i32x4 hi = *reinterpret_cast<const i32x4*>(vb_ + 32 * 64 * cc + s1);
                    const i32x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    // formats 0/0: E4M3 A and B; unit E8M0 block scales (127 = 2^0)
                    O[cc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, Pf, O[cc], 0, 0, 0, 0x7f7f7f7f, 0,
                                                                            0x7f7f7f7f);
                }
            } else {
                bf16x8 Pb[2][2];
                float rs[2];
                // shifted (kFuseBf, after m was raised): the scores still hold
                // logit - mch, so m - mch more is subtracted
                auto make_p = [&](const bool shifted) {
                    // int8: the score bias leaves with the max (kI8Bias)
                    const float mk = kInt8 ? __builtin_fmaf(kI8Bias, coef, m) : m;
                    const float off = mch - m;
                    rs[0] = rs[1] = 0.f;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int s = 0; s < 2; ++s) {
                            u32x4 w;
#pragma unroll
                            for (int ii = 0; ii < 4; ++ii) {
                                const int e = 8 * s + 2 * ii;
                                float x0, x1;
                                if constexpr (kFuseBf) {
                                    x0 = __builtin_amdgcn_exp2f(shifted ? S[kb][e] + off : S[kb][e]);
                                    x1 = __builtin_amdgcn_exp2f(shifted ? S[kb][e + 1] + off : S[kb][e + 1]);
                                } else {
                                    x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][e], coef, -mk));
                                    x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][e + 1], coef, -mk));
                                }
                                if (masked) {
                                    if (j * kBN + key_of_elem(kb, e, hh) >= n) x0 = 0.f;
                                    if (j * kBN + key_of_elem(kb, e + 1, hh) >= n) x1 = 0.f;
                                }
                                const f32x2 f = {x0, x1};
                                const bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
                                rs[s] = __builtin_amdgcn_fdot2_f32_bf16(b, ones, rs[s], false);
                                w[ii] = __builtin_bit_cast(uint32_t, b);
                            }
                            Pb[kb][s] = __builtin_bit_cast(bf16x8, w);
                        }
                };
                make_p(false);
                float t = rs[0] + rs[1];
                // kFuseBf: the first tile sets the running max (its chain started from 0)
                if (masked || (kFuseBf && j == 0) || __any(!(t <= kSumCheck)))
                    if (raise_max()) {
                        make_p(true);
                        t = rs[0] + rs[1];
                        if constexpr (kFuseBf) {
                            mch = m;
#pragma unroll
                            for (int e = 0; e < 16; ++e) negm[e] = -m;
                            asm volatile("" : "+v"(negm));
                        }
                    }
                l += t;
                ph2 = phase_clock();
                if (behind) {
                    tile_sync();
                    __builtin_amdgcn_s_setprio(2);     // the lagging wave's P V (kStagger)
                }
                // O^T += V^T P^T
                const uint8_t* vb_ = vbuf_st(st);
                typedef short i16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        bf16x8 a[4];
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc) {
                            const int off = v_lane_off + 64 * (cc ^ rk) + (32 * kb + 16 * s) * 256;
                            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (__attribute__((address_space(3))) i16x4*)(vb_ + off));
                            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (__attribute__((address_space(3))) i16x4*)(vb_ + off + 4 * 256));
                            a[cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                        }
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc)
                            O[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cc], Pb[kb][s], O[cc], 0, 0, 0);
                    }
                if (behind) {
                    __builtin_amdgcn_sched_barrier(0);   // every product issued first
                    __builtin_amdgcn_s_setprio(0);
                }
            }
        }
        [[maybe_unused]] const uint64_t ph3 = phase_clock();
        if (!behind) tile_sync();
        if constexpr (kPhaseTiming) {
            const uint64_t ph4 = phase_clock();
            ph_sum[0] += ph1 - ph0;
            ph_sum[1] += ph2 - ph1;
            ph_sum[2] += ph3 - ph2;
            ph_sum[3] += ph4 - ph3;
            ph_tiles += 1;
        }
    };

    // the first tiles stream in while Q' is prepared (the int8 form prepares
    // it first: its prologue needs the registers)
    if constexpr (!(kFuseQ && kInt8)) {
        fetch(jb);
        fetch(jb + 1);
        if constexpr (kAhead == 3) fetch(jb + 2);
    }
    if constexpr (kFuseBf) {
        // Q' of the work-group's 256 rows, computed while tiles 0..2 stream
        // in, in two halves of 128 rows staged through LDS stage 3 (K' part:
        // rows 0..63 of the half, V part: rows 64..127), 16-byte chunks
        // XOR-swizzled by the row; waves 4h..4h+3 take their MFMA operands
        // from half h.
        float ga[8], gb[8];
        unpack8(fga, ga);
        unpack8(fgb, gb);
        const int r = tid >> 3;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ps = 2 * half + s;
                float cs[8], sn[8], xa[8], xb[8], ra[8], rb[8];
                rope_angles(fpv[ps], ffreq, cs, sn);
                unpack8(fqa[ps], xa);
                unpack8(fqb[ps], xb);
                u32x4 oa, ob;
                // Q' is rounded to bf16 once, with the base-2 logit scale folded in
                norm_rotate<true>(xa, xb, ga, gb, cs, sn, P.eps, oa, ob, ra, rb, P.c);
                if (qt * kBMw + kPsRows * ps + r >= n) oa = ob = u32x4{0, 0, 0, 0};
                uint8_t* st = (s == 0 ? kbuf(3) : vbuf(3)) + r * 256;
                *reinterpret_cast<u32x4*>(st + ((fsl.a ^ (r & 15)) * 16)) = oa;
                *reinterpret_cast<u32x4*>(st + ((fsl.b ^ (r & 15)) * 16)) = ob;
            }
            __syncthreads();
            if ((wave >> 2) == half) {
                const int row = (wave & 3) * 32 + n32;            // row of the half
                const uint8_t* src = ((wave & 3) < 2 ? kbuf(3) : vbuf(3)) + (row & 63) * 256;
#pragma unroll
                for (int t = 0; t < kSteps; ++t)
                    q[t] = *reinterpret_cast<const QOp*>(src + (((2 * t + hh) ^ (row & 15)) * 16));
            }
            // the staging reads are complete before stage 3 is written again
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }
    if constexpr (kFuseQ && kInt8) {
        // Int8 Q': the work-group's kBMw rows are 64-row quantisation blocks;
        // thread (r = tid / 8, slot tid % 8) prepares rows r + kPsRows ps.  Per
        // half (ps = 2h, 2h + 1: rows rho = r + kPsRows s of the half, s = 0, 1,
        // two or three blocks): Q' rounded to bf16 exactly as the prep does,
        // the block absmax over the work-group, the prep's scale and codes,
        // staged through stage 3 (half row rho < 64 in the K' part, the rest in
        // the V part; 128-byte rows, 16-byte chunks XOR-swizzled as the K'
        // tiles).  A wave's 8 rows of one ps lie in one block, so per wave and
        // ps one absmax goes to LDS.  Wave w's 32 rows belong to half
        // w / (kW / 2); it takes its operands and its block's scale there.
        constexpr int kHalfRows = kBMw / 2, kBlkPerHalf = kHalfRows / 64, kWPerHalf = kW / 2;
        __shared__ float red[kW][2];                              // [wave][s]
        float ga[8], gb[8];
        unpack8(fga, ga);
        unpack8(fgb, gb);
        const int r = tid >> 3;
        auto stage_row = [&](int rho) {
            return rho < 64 ? kbuf(3) + rho * 128 : vbuf(3) + (rho - 64) * 128;
        };
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float rv[2][16];
            float mx[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ps = 2 * half + s;
                float cs[8], sn[8], xa[8], xb[8];
                rope_angles(fpv[ps], ffreq, cs, sn);
                unpack8(fqa[ps], xa);
                unpack8(fqb[ps], xb);
                u32x4 oa, ob;
                norm_rotate(xa, xb, ga, gb, cs, sn, P.eps, oa, ob, rv[s], rv[s] + 8);
                mx[s] = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (qt * kBMw + kPsRows * ps + r >= n) rv[s][i] = 0.f;
                    mx[s] = fmaxf(mx[s], fabsf(rv[s][i]));
                }
#pragma unroll
                for (int sh = 1; sh < 64; sh <<= 1) mx[s] = fmaxf(mx[s], __shfl_xor(mx[s], sh));
            }
            if (lane == 0) {
                red[wave][0] = mx[0];
                red[wave][1] = mx[1];
            }
            __syncthreads();
            // absmax of each block of the half: the partials of the (wave, s)
            // whose rows 8 wave + kPsRows s .. + 7 fall in it
            float amax[kBlkPerHalf];
#pragma unroll
            for (int b = 0; b < kBlkPerHalf; ++b) {
                amax[b] = 0.f;
#pragma unroll
                for (int w = 0; w < kW; ++w)
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        if (((8 * w + kPsRows * s) >> 6) == b) amax[b] = fmaxf(amax[b], red[w][s]);
            }
            // IEEE fp32 divisions, as in the prep (no fast-math in this library).
            // The scale is uniform over the wave: kept in a scalar register.
            if (wave / kWPerHalf == half)
                qscale = __int_as_float(__builtin_amdgcn_readfirstlane(
                    __float_as_int(amax[(wave % kWPerHalf) >> 1] / 127.0f)));
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int rho = kPsRows * s + r;                   // row of the half
                const float a = amax[(8 * wave + kPsRows * s) >> 6];
                const float inv = a > 0.f ? 127.0f / a : 0.f;
                uint8_t* st = stage_row(rho);
                const int sw = k_swizzle<true>(rho);
                const Slot& sl = fsl;
                *reinterpret_cast<u32x2*>(st + (((sl.a >> 1) ^ sw) * 16) + (sl.a & 1) * 8) =
                    u32x2{quant4(rv[s], inv), quant4(rv[s] + 4, inv)};
                *reinterpret_cast<u32x2*>(st + (((sl.b >> 1) ^ sw) * 16) + (sl.b & 1) * 8) =
                    u32x2{quant4(rv[s] + 8, inv), quant4(rv[s] + 12, inv)};
            }
            __syncthreads();
            if (wave / kWPerHalf == half) {
                const int rho = (wave % kWPerHalf) * 32 + n32;    // row of the half
                const uint8_t* src = stage_row(rho);
#pragma unroll
                for (int t = 0; t < kSteps; ++t)
                    q[t] = *reinterpret_cast<const QOp*>(src + (((2 * t + hh) ^ k_swizzle<true>(rho)) * 16));
            }
            // the staging reads are complete before stage 3 is written again
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }
    if constexpr (kFuseQ && kInt8) {
        asm volatile("" : "+v"(bias16));
        fetch(jb);
        fetch(jb + 1);
        fetch(jb + 2);
    }
    wait_vmem_upto<(kAhead - 1) * kDma8>();
    __syncthreads();
    // The fused-Q forms run the loop unrolled by the four stages, so that each
    // stage's LDS offsets are immediates of the operand reads (fewer address
    // adds per tile): measured -1.8% for bf16 and -0.7% for int8 Q'/K' with
    // bf16 V in the eight-wave form (same process and box, outputs
    // bit-identical); the other eight-wave forms were slower so (bf16 +1.5%,
    // bf16 Q'/K' with E4M3 V +4.6%), and the twelve-wave forms spill unrolled
    // (168 registers), so these keep the rolled loop.
    constexpr bool kUnroll = kFuseQ && kW == 8;
    int j = jb;
    ph_l0 = phase_clock();
    if constexpr (kUnroll) {
        for (; j < last && (j & 3); ++j) tile(j, false, j & 3);
        for (; j + 4 <= last; j += 4) {
            tile(j, false, 0);
            tile(j + 1, false, 1);
            tile(j + 2, false, 2);
            tile(j + 3, false, 3);
        }
    }
    for (; j < last; ++j) tile(j, false, j % kStages);
    tile(last, ragged, last % kStages);
    ph_l1 = phase_clock();
    // the chain-start values stay allocated until every chain has read them
    if constexpr (kInt8) asm volatile("" ::"v"(bias16));
    if constexpr (kFuseBf) asm volatile("" ::"v"(negm));
    wait_vmem_all();
    if constexpr (kScores) return;
    // O is complete here in every lane.  A matrix-core product reads the
    // operands (and the E4M3 path's per-lane scale registers) of all 64 lanes,
    // so none may move into the store branch below, where the lanes of rows
    // >= N are switched off: this empty statement consumes O before it.
    asm volatile("" ::"a"(O[0]), "a"(O[1]), "a"(O[2]), "a"(O[3]));

    const float lt = sum_halves(l);
    const float inv = 1.0f / lt;
    const int qrow = q0 + n32;
    if (qrow < n) {
        uint16_t* orow = P.o + (int64_t)qrow * P.o_st + (int64_t)head * P.o_sh;
        const float* vsh = kFp8V ? P.vs + (int64_t)head * 128 : nullptr;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * cc + 8 * i + 4 * hh;
                float f[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) f[u] = kFp8V ? O[cc][4 * i + u] * (vsh[d0 + u] * inv) : O[cc][4 * i + u] * inv;
                const u32x2 w = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
                st8(orow + d0, w);
            }
    }
#if H3_PHASE_TIMING
    const uint64_t ph_k1 = phase_clock();
    if (lane == 0) {
        unsigned long long* g = g_phase_cycles + kPhaseSlots * (wave / 4);
        const uint64_t v[9] = {ph_sum[0], ph_sum[1], ph_sum[2], ph_sum[3], ph_tiles,
                               ph_l0 - ph_k0, ph_l1 - ph_l0, ph_k1 - ph_l1, 1};
#pragma unroll
        for (int i = 0; i < 9; ++i) atomicAdd(g + i, (unsigned long long)v[i]);
    }
#endif
}

hipError_t launch_forward(const FwdParams& P, bool int8, bool fp8v, hipStream_t stream) {
    (void)hipGetLastError();     // clear an error left by an earlier, unrelated call
    const dim3 grid(kXcds * P.per_xcd), block(512);
    // int8: twelve waves, 384-row tiles (forward_tile_rows), plain block order
    if (int8 && fp8v)
        hipLaunchKernelGGL((fwd8_kernel<true, true, false, 12>), dim3(P.total), dim3(768), 0, stream, P);
    else if (int8)
        hipLaunchKernelGGL((fwd8_kernel<true, false, false, 12>), dim3(P.total), dim3(768), 0, stream, P);
    else if (fp8v)
        hipLaunchKernelGGL((fwd8_kernel<false, true>), grid, block, 0, stream, P);
    else
        hipLaunchKernelGGL((fwd8_kernel<false, false>), grid, block, 0, stream, P);
    return hipGetLastError();
}

hipError_t launch_forward_fused_q(const FwdParams& P, bool int8, hipStream_t stream) {
    (void)hipGetLastError();     // clear an error left by an earlier, unrelated call
    if (int8)      // twelve waves, 384-row tiles (forward_tile_rows), plain block order
        hipLaunchKernelGGL((fwd8_kernel<true, false, true, 12>), dim3(P.total), dim3(768), 0, stream, P);
    else
        hipLaunchKernelGGL((fwd8_kernel<false, false, true>), dim3(kXcds * P.per_xcd), dim3(512), 0, stream, P);
    return hipGetLastError();
}

int forward_tile_rows(bool int8) { return int8 ? 384 : kBM; }

// The int8 forward's own Q'K'^T path over a window (kScores), in the
// twelve-wave form the int8 forwards run: `fp8v_layout` picks the K' row
// order of the E4M3-V forward instead of the bf16-V one.  P.total work-groups
// take query tiles s_qt0.. of head s_head; key tiles kt0..kt1 stream through
// the stages.
hipError_t launch_scores_i8(const FwdParams& P, bool fp8v_layout, hipStream_t stream) {
    (void)hipGetLastError();     // clear an error left by an earlier, unrelated call
    if (fp8v_layout)
        hipLaunchKernelGGL((fwd8_kernel<true, true, false, 12, true>), dim3(P.total), dim3(768), 0, stream, P);
    else
        hipLaunchKernelGGL((fwd8_kernel<true, false, false, 12, true>), dim3(P.total), dim3(768), 0, stream, P);
    return hipGetLastError();
}

}  // namespace h3

// The phase-timing accessors (include/h3attn_phase_timing.h): live in the
// phase-timing build, H3ATTN_E_UNSUPPORTED in the others.
extern "C" int h3attn_phase_timing_read(unsigned long long* out) {
#if H3_PHASE_TIMING
    if (!out) return -1;
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(h3::g_phase_cycles), sizeof(h3::g_phase_cycles)) == hipSuccess ? 0 : -6;
#else
    (void)out;
    return -3;
#endif
}
extern "C" int h3attn_phase_timing_clear(void) {
#if H3_PHASE_TIMING
    static const unsigned long long zero[h3::kPhaseSlots * h3::kPhaseGroups] = {};
    return hipMemcpyToSymbol(HIP_SYMBOL(h3::g_phase_cycles), zero, sizeof(zero)) == hipSuccess ? 0 : -6;
#else
    return -3;
#endif
}
