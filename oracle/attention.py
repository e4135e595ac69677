"""Plain, slow, obviously correct CPU reference of the packed-attention hot path.

TEST INFRASTRUCTURE ONLY: the product path must never import this module.
It shares no code with the HIP library or its binding.

What it computes (the hot path of one H3 denoiser block, as described on the
pages "H3 Runtime Current State" and "H3 Blackwell Runtime Plan"):

1. Q/K RMSNorm per (token, head) over the head dimension
   ("H3 Runtime Current State", Owned Performance Kernels: the entry kernel
   fuses Q/K RMSNorm with split-half RoPE; "H3 Blackwell Runtime Plan",
   2026-08-15 Handoff: fused Q/K RMS + RoPE + HND layout).
2. 3-axis (t, h, w) split-half RoPE ("H3 Blackwell Runtime Plan",
   Architecture: 3-axis RoPE; "H3 Runtime Current State", Owned Performance
   Kernels: split-half RoPE).
3. Non-causal softmax(Q K^T * scale) V over the whole packed sequence, one
   softmax per query row, no padding of semantic tokens ("H3 Blackwell Runtime
   Plan", Architecture and Non-Negotiable Validation).
4. Optional int8 Q/K quantisation with one fp32 absmax scale per 64-token
   block per head, and exact int32 Q K^T accumulation (the int8-QK step of the
   SageAttention2 path: "H3 Runtime Current State", Owned Performance Kernels,
   Q quantization and K quantization).
5. Optional FP8 (OCP E4M3) V with one fp32 scale per channel per head, the
   FP8-PV step of the same path ("H3 Runtime Current State", Owned Performance
   Kernels: V scale/FP8 quantization; the V-preparation study emits E4M3 V plus
   FP32 per-channel scales).  The GPU also rounds P to E4M3 inside its P V
   product; the oracle keeps P exact, as it keeps P exact against bf16.
6. Optional K smoothing before the int8 K quantisation: subtract the per-head,
   per-channel mean of K' over all tokens (the K-mean step of the same path:
   "H3 Runtime Current State", Owned Performance Kernels, K mean).  Every
   score of a query row moves by the same q . mean, so the softmax, and the
   exact attention, do not change; only the quantisation error does.

All floating point is fp64 except where the method fixes fp32 (the int8
quantiser, whose rounding decisions must match bit for bit).

Readings where the pages are silent (each one is listed with its reason in
the design notes of the repository):
* RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma, eps inside the sqrt,
  gamma of shape [d] (shared by heads) or [H, d].
* RoPE sections are contiguous slices [0,32) t, [32,80) h, [80,128) w; inside a
  section of width s the pairs are (j, j + s/2) for j < s/2 and the angle is
  pos_axis * theta^(-2j/s) (the textbook RoFormer frequencies), rotating
  (a, b) -> (a cos - b sin, b cos + a sin).
* Int8: round-half-even, symmetric +-127, blocks of 64 tokens from token 0
  with a partial last block, scale = fl32(absmax/127), codes =
  rint(fl32(x * fl32(127/absmax))), an all-zero block has scale 0 and codes 0.
* K smoothing: the mean is taken of the bf16-rounded prepped K' (the int8
  quantiser's input), in float32 and in a fixed order: a sequential sum over
  each 64-token block in token order, a sequential sum of the block sums in
  block order, then one IEEE division by N.  The quantiser then sees
  fl32(k - mean) in place of k.
* FP8 V: per head and channel over all N tokens, scale = fl32(absmax/448),
  value = clamp(fl32(v * fl32(448/absmax)), -448, 448), rounded to the nearest
  E4M3 value (ties to even mantissa, subnormals kept); an all-zero channel has
  scale 0 and codes 0.  448 is the largest finite E4M3 value.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "f32_to_bf16_bits", "round_to_bf16",
    "rmsnorm", "rope_layout", "rope", "prep", "prep_head",
    "softmax_rows", "attention", "attention_head", "attention_rows_head",
    "quantize_i8", "scores_i32", "attention_i8_rows_head",
    "e4m3_bits", "e4m3_bits_to_f64", "quantize_v_fp8", "dequantize_v_fp8",
    "FP8_P_LOG2_FACTOR", "attention_fp8v_rows",
    "k_mean_blocked", "smooth_k",
]


# ----------------------------------------------------------------------------
# bfloat16 <-> float (own converters; bf16 is the storage type of the
# activations on the pages: "H3 Blackwell Runtime Plan", Next Performance
# Plan keeps RMSNorm, RoPE and softmax in BF16/FP16)
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even; NaN stays NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r[nan] = ((u[nan] >> 16).astype(np.uint16) | np.uint16(0x0040))
    return r


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values directly to the nearest bf16 value (ties to even), as float64.

    bf16 keeps 8 significant bits; below 2^-126 the spacing stays 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(x / quantum) * quantum
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


# ----------------------------------------------------------------------------
# 1. RMSNorm per (token, head)
# ----------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean_d(x^2) + eps) * gamma over the last (head) dimension.

    ``x`` is float64 [..., H, d]; ``gamma`` is [d] or [H, d].
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma


# ----------------------------------------------------------------------------
# 2. 3-axis split-half RoPE
# ----------------------------------------------------------------------------

def rope_layout(sections) -> list:
    """[(axis, offset, width)] of the contiguous t/h/w slices of the head dim."""
    out, off = [], 0
    for axis, s in enumerate(sections):
        if s % 2:
            raise ValueError("each RoPE section must have even width")
        out.append((axis, off, s))
        off += s
    return out


def rope(y: np.ndarray, pos: np.ndarray, sections, theta: float) -> np.ndarray:
    """Rotate each (j, j + s/2) pair of every section by pos[axis] * theta^(-2j/s).

    ``y`` float64 [N, H, d] (or [N, d]); ``pos`` integer [N, 3] in (t, h, w).
    """
    y = np.asarray(y, dtype=np.float64)
    out = y.copy()
    pos = np.asarray(pos, dtype=np.float64)
    for axis, off, s in rope_layout(sections):
        half = s // 2
        j = np.arange(half, dtype=np.float64)
        omega = theta ** (-2.0 * j / s)                       # [half]
        phi = pos[:, axis][:, None] * omega[None, :]          # [N, half]
        if y.ndim == 3:
            phi = phi[:, None, :]
        c, sn = np.cos(phi), np.sin(phi)
        a = y[..., off:off + half]
        b = y[..., off + half:off + s]
        out[..., off:off + half] = a * c - b * sn
        out[..., off + half:off + s] = b * c + a * sn
    return out


def prep(x_bits: np.ndarray, gamma_bits: np.ndarray, pos: np.ndarray, sections,
         theta: float, eps: float) -> np.ndarray:
    """RMSNorm then RoPE of bf16 [N, H, d] input; float64 [N, H, d] result."""
    x = bf16_bits_to_f64(x_bits)
    g = bf16_bits_to_f64(gamma_bits)
    return rope(rmsnorm(x, g, eps), pos, sections, theta)


def prep_head(x_bits_head: np.ndarray, gamma_bits: np.ndarray, head: int, pos: np.ndarray,
              sections, theta: float, eps: float) -> np.ndarray:
    """:func:`prep` of one head, from bf16 [N, d]; gamma [d] or [H, d]."""
    g = bf16_bits_to_f64(gamma_bits)
    if g.ndim == 2:
        g = g[head]
    return rope(rmsnorm(bf16_bits_to_f64(x_bits_head), g, eps), pos, sections, theta)


# ----------------------------------------------------------------------------
# 3. Non-causal softmax attention (exact, two-pass per query block)
# ----------------------------------------------------------------------------

def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax of a score matrix, max-subtracted (the max cancels exactly)."""
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_rows_head(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                        block: int = 256) -> np.ndarray:
    """O = softmax(q_rows K^T * scale) V for one head, all N keys, float64.

    ``q_rows`` [R, d], ``k`` [N, d], ``v`` [N, d]; processed in query blocks of
    ``block`` rows (each block is exact; blocking only bounds memory).
    """
    out = np.empty((q_rows.shape[0], v.shape[1]), dtype=np.float64)
    for r0 in range(0, q_rows.shape[0], block):
        s = (q_rows[r0:r0 + block] @ k.T) * scale
        out[r0:r0 + block] = softmax_rows(s) @ v
    return out


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Full attention of one head: q, k, v float64 [N, d]."""
    return attention_rows_head(q, k, v, scale)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Full attention over [N, H, d] float64 tensors, heads independent."""
    out = np.empty(q.shape[:1] + (q.shape[1], v.shape[2]), dtype=np.float64)
    for h in range(q.shape[1]):
        out[:, h, :] = attention_head(q[:, h, :], k[:, h, :], v[:, h, :], scale)
    return out


# ----------------------------------------------------------------------------
# 4. Int8 per-64-token-block Q/K quantisation and exact int32 scores
# ----------------------------------------------------------------------------

QUANT_BLOCK = 64


def quantize_i8(x: np.ndarray, block: int = QUANT_BLOCK):
    """Quantise one head's [N, d] values to int8 codes with one fp32 scale per block.

    ``x`` must already be float32 (the bf16-rounded prepped values).  Every
    operation is a single IEEE float32 operation rounded to nearest even:
    a = max|x| over the block (exact), s = a / 127, inv = 127 / a,
    code = clamp(rint(x * inv), -127, 127); a == 0 gives s = 0 and zero codes.
    Returns (codes int8 [N, d], scales float32 [ceil(N/block)]).
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("quantize_i8 expects float32 input")
    n = x.shape[0]
    nb = (n + block - 1) // block
    codes = np.zeros(x.shape, dtype=np.int8)
    scales = np.zeros(nb, dtype=np.float32)
    f127 = np.float32(127.0)
    for b in range(nb):
        xb = x[b * block:(b + 1) * block]
        a = np.float32(np.max(np.abs(xb))) if xb.size else np.float32(0)
        if a == 0:
            continue
        scales[b] = a / f127
        inv = f127 / a
        q = np.rint((xb * inv).astype(np.float32))
        codes[b * block:(b + 1) * block] = np.clip(q, -127, 127).astype(np.int8)
    return codes, scales


def scores_i32(codes_q: np.ndarray, codes_k: np.ndarray) -> np.ndarray:
    """Exact integer Q K^T of int8 codes, returned as int64 [R, C].

    Computed as a float64 product of integer-valued matrices: every partial sum
    is an integer of magnitude <= d * 127^2, far below 2^53, so it is exact.
    """
    s = codes_q.astype(np.float64) @ codes_k.astype(np.float64).T
    return s.astype(np.int64)


def attention_i8_rows_head(rows: np.ndarray, codes_q: np.ndarray, scales_q: np.ndarray,
                           codes_k: np.ndarray, scales_k: np.ndarray, v: np.ndarray,
                           scale: float, block: int = QUANT_BLOCK, qblock: int = 256) -> np.ndarray:
    """Attention of query ``rows`` of one head from int8 Q/K codes, float64 output.

    S = S_int * s_q[row block] * s_k[key block] * scale, then an exact fp64
    softmax and P V with V float64 [N, d].
    """
    rows = np.asarray(rows, dtype=np.int64)
    n = codes_k.shape[0]
    sk = scales_k.astype(np.float64)[np.arange(n) // block]             # [N]
    out = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    for r0 in range(0, rows.size, qblock):
        rr = rows[r0:r0 + qblock]
        s_int = scores_i32(codes_q[rr], codes_k).astype(np.float64)
        sq = scales_q.astype(np.float64)[rr // block]
        s = s_int * sq[:, None] * sk[None, :] * scale
        out[r0:r0 + qblock] = softmax_rows(s) @ v
    return out


# ----------------------------------------------------------------------------
# 5. FP8 (OCP E4M3) V with per-channel fp32 scales
# ----------------------------------------------------------------------------
# E4M3 (OCP 8-bit floating point, "fn" variant): 1 sign bit, 4 exponent bits
# with bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN; the largest
# finite value is 1.75 * 2^8 = 448; normals start at 2^-6; subnormals are
# m * 2^-9 for m = 1..7.

E4M3_MAX = 448.0


def e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Encode finite values with |x| <= 448 as E4M3 bytes, nearest value, ties to even.

    Works per element in float64 (every step below is exact in float64 for
    float32 inputs): pick the binade, scale the magnitude to units of the
    binade's spacing, round half to even with numpy's rint, and carry a
    mantissa overflow into the next binade.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_bits expects finite values with |x| <= 448")
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x)
    out = np.zeros(x.shape, dtype=np.uint8)
    # exponent of the binade (values below 2^-6 use the subnormal spacing 2^-9)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    e = np.clip(e, -6, 8)
    # log2 of an exact power of two can be off by one in floating point: fix up
    e = np.where((a > 0) & (a < np.ldexp(1.0, e)) & (e > -6), e - 1, e)
    e = np.where((a >= np.ldexp(1.0, e + 1)) & (e < 8), e + 1, e)
    sub = a < 2.0 ** -6
    # mantissa in units of 2^(e-3) (normal) or 2^-9 (subnormal)
    unit = np.where(sub, 2.0 ** -9, np.ldexp(1.0, e - 3))
    q = np.rint(a / unit)                      # exact division by a power of two
    # normal: q in [8, 16]; 16 carries into the next binade
    carry = (~sub) & (q >= 16)
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    # subnormal rounding up to 8 units is the smallest normal 2^-6 (exponent field 1)
    mant = np.where(sub, np.where(q >= 8, 0, q), q - 8).astype(np.int64)
    expf = np.where(sub, np.where(q >= 8, 1, 0), e + 7).astype(np.int64)
    out = (sign | ((expf << 3) | mant).astype(np.uint8)).astype(np.uint8)
    return out


def e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode E4M3 bytes (finite codes) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    expf = (b >> 3) & 0xF
    mant = b & 0x7
    if np.any((expf == 0xF) & (mant == 0x7)):
        raise ValueError("NaN code")
    val = np.where(expf == 0, mant * 2.0 ** -9, np.ldexp(1.0 + mant / 8.0, expf - 7))
    return sign * val


def quantize_v_fp8(v: np.ndarray):
    """Quantise one head's V (float32 [N, d]) to E4M3 with one fp32 scale per channel.

    Per channel c (a single float32 operation per step, rounded to nearest even):
    a = max_n |v[n, c]| (exact), s = a / 448, inv = 448 / a,
    x = clamp(v * inv, -448, 448), code = E4M3 nearest (ties to even).
    a == 0 gives s = 0 and zero codes.  Returns (codes uint8 [N, d], scales float32 [d]).
    """
    v = np.asarray(v)
    if v.dtype != np.float32:
        raise TypeError("quantize_v_fp8 expects float32 input")
    n, d = v.shape
    codes = np.zeros((n, d), dtype=np.uint8)
    scales = np.zeros(d, dtype=np.float32)
    f448 = np.float32(E4M3_MAX)
    for c in range(d):
        col = v[:, c]
        a = np.float32(np.max(np.abs(col))) if n else np.float32(0)
        if a == 0:
            continue
        scales[c] = a / f448
        inv = f448 / a
        x = np.clip((col * inv).astype(np.float32), -f448, f448)
        codes[:, c] = e4m3_bits(x)
    return codes, scales


def dequantize_v_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The V the FP8 P V product multiplies: code value times channel scale (float64)."""
    return e4m3_bits_to_f64(codes) * scales.astype(np.float64)[None, :]


# log2 of the factor the FP8 P V product applies to each softmax numerator
# before rounding it to E4M3 (reading R20 of the design notes): it cancels
# between numerator and denominator and only moves small numerators away from
# the subnormal range.
FP8_P_LOG2_FACTOR = 0.8


def attention_fp8v_rows(s: np.ndarray, v_hat: np.ndarray, p_log2_factor: float = FP8_P_LOG2_FACTOR):
    """Reference and per-element error bound of the FP8 P V product.

    The FP8-PV step of the SageAttention2 path ("H3 Runtime Current State",
    Owned Performance Kernels: INT8 QK and FP8 PV) multiplies the softmax
    numerators, rounded to E4M3, by the dequantised E4M3 V, and divides by the
    sum of the unrounded numerators (softmax statistics stay in fp32 there).

    ``s``: the scores of some query rows against all N keys, already times the
    softmax scale, float64 [R, N].  ``v_hat``: the dequantised V of the head,
    float64 [N, d] (:func:`dequantize_v_fp8`).

    Returns ``(ref, bound)``, both float64 [R, d]:
    * ref = softmax(s) @ v_hat, the exact attention over the dequantised V (the
      result with P kept exact, as against bf16);
    * bound: the largest change that rounding each numerator to E4M3 can make.
      With r = softmax(s) and Z = sum_m exp(s_m - max s), the numerator of key m
      is a * exp(s_m - m') for a = 2^p_log2_factor and some running max
      m' <= max s, so the denominator is at least a * Z; nearest rounding to
      E4M3 moves a numerator x by at most 2^-4 x when x is normal (3 mantissa
      bits) and by at most 2^-10 (half the subnormal spacing 2^-9) otherwise.
      Summed against |v_hat| this gives
          bound = 2^-4 * r @ |v_hat| + 2^-10 / (a Z) * sum_m |v_hat_m|.
    """
    s = np.asarray(s, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    smax = s.max(axis=1, keepdims=True)
    e = np.exp(s - smax)
    z = e.sum(axis=1, keepdims=True)
    r = e / z
    av = np.abs(v_hat)
    ref = r @ v_hat
    a = 2.0 ** p_log2_factor
    bound = 2.0 ** -4 * (r @ av) + 2.0 ** -10 / (a * z) * av.sum(axis=0)[None, :]
    return ref, bound


# ----------------------------------------------------------------------------
# K smoothing (softmax-invariant mean subtraction before the int8 K quantiser)
# ----------------------------------------------------------------------------

def k_mean_blocked(k: np.ndarray, block: int = QUANT_BLOCK) -> np.ndarray:
    """Per-channel mean of one head's K' (float32 [N, d], bf16-valued), float32.

    Fixed order, one float32 rounding per addition: each block of ``block``
    tokens is summed sequentially in token order (numpy's cumsum is a plain
    running sum), the block sums are summed sequentially in block order, and
    the total is divided by N (IEEE float32 division).
    """
    k = np.asarray(k)
    if k.dtype != np.float32:
        raise TypeError("k_mean_blocked expects float32 input")
    n, d = k.shape
    if n == 0:
        raise ValueError("no tokens")
    sums = [np.cumsum(k[b:b + block], axis=0, dtype=np.float32)[-1] for b in range(0, n, block)]
    total = np.cumsum(np.stack(sums), axis=0, dtype=np.float32)[-1]
    return (total / np.float32(n)).astype(np.float32)


def smooth_k(k: np.ndarray, block: int = QUANT_BLOCK):
    """(mean, k - mean) of one head's K' in float32: the int8 quantiser's input
    after K smoothing (each difference rounded once to float32)."""
    mu = k_mean_blocked(k, block)
    return mu, (np.asarray(k, dtype=np.float32) - mu[None, :]).astype(np.float32)

