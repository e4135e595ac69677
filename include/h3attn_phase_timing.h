/*
 * h3attn_phase_timing.h - measurement aid: where the forward's key-tile loop
 * spends its cycles.
 *
 * The library built with -DH3_PHASE_TIMING=1 (libh3attn_timing.so, from the
 * same sources) reads the shader clock (s_memtime) in every wave of the
 * forward kernels at the start of each key tile, after the tile's Q'K'^T
 * product chain, after its softmax, after its last P V product is issued and
 * after the tile's work-group barrier, and at the ends of the wave's prologue,
 * tile loop and epilogue.  Lane 0 of each wave adds the wave's sums into a
 * device array, per group of four waves (waves 4g .. 4g+3, one per SIMD).
 * The stamps add a little time (their results are read after each barrier).
 * The forward's outputs are bit-identical to the release build's.
 *
 * In every other build both calls return H3ATTN_E_UNSUPPORTED (-3).
 * Neither call is ordered with the caller's streams: synchronise first.
 */
#ifndef H3ATTN_PHASE_TIMING_H
#define H3ATTN_PHASE_TIMING_H

#ifdef __cplusplus
extern "C" {
#endif

/* Number of unsigned 64-bit counters h3attn_phase_timing_read writes. */
#define H3ATTN_PHASE_TIMING_COUNTERS 30

/*
 * Copies the counters, accumulated since the last clear over every forward
 * launch, to host memory out[30]: for wave group g = 0, 1, 2 at out[10 g + i],
 *   i = 0  cycles from a tile's start to the end of its Q'K'^T chain
 *          (including the tile's buffer -> LDS copy issue),
 *   i = 1  cycles of the softmax (to the start of the P V product),
 *   i = 2  cycles to the issue of the tile's last P V product (the staggered
 *          forms' lagging waves take their barrier inside this interval),
 *   i = 3  cycles from there to after the tile's barrier,
 *   i = 4  tiles, i = 5 prologue cycles, i = 6 tile-loop cycles,
 *   i = 7  epilogue cycles, i = 8 waves, i = 9 unused (0).
 * Returns 0, H3ATTN_E_NULL (-1) for out == NULL, H3ATTN_E_HIP (-6) if the
 * copy fails, H3ATTN_E_UNSUPPORTED (-3) outside the phase-timing build.
 */
int h3attn_phase_timing_read(unsigned long long* out);

/* Zeroes the counters.  Returns 0, -6 or -3 as above. */
int h3attn_phase_timing_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_PHASE_TIMING_H */
