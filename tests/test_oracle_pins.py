"""Pins of the CPU oracle against mathematics, library routines and hand-derived values.

Each check is chosen so that a plausible mistake in the oracle (a dropped
term, a wrong sign, section offset, frequency exponent or axis, a transposed
operand) fails at least one of them.  None of them re-types the oracle's own
formula as the expected value.
"""
import math
import struct

import numpy as np
import pytest
import torch

import oracle as O
from audio_video_diffusion_amd import workloads as W

SECTIONS = W.ROPE_SECTIONS
THETA = W.ROPE_THETA
EPS = W.RMS_EPS


# --------------------------------------------------------------------------
# bf16 converters: library routine (torch's RNE cast) and exhaustive neighbours
# --------------------------------------------------------------------------

def test_f32_to_bf16_matches_torch_random_and_specials():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(400_000).astype(np.float32),
        (rng.standard_normal(300_000) * 1e30).astype(np.float32),
        (rng.standard_normal(300_000) * 1e-38).astype(np.float32),   # subnormal range
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                  1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, 1.4e-45, 3.4028235e38],
                 dtype=np.float32),
        np.frombuffer(rng.integers(0, 2 ** 32, 100_000, dtype=np.uint64).astype(np.uint32).tobytes(),
                      dtype=np.float32),
    ])
    finite = np.isfinite(x) | np.isinf(x)
    ours = O.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours[finite], ref[finite])
    nan = ~finite
    assert np.all(np.isnan(O.bf16_bits_to_f64(ours[nan])))


def test_round_to_bf16_is_nearest_even_neighbour():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(50_000), rng.standard_normal(50_000) * 1e-3,
                        rng.standard_normal(2_000) * 1e-39])
    r = O.round_to_bf16(x)
    # r must be a bf16 value: round trip through the fp32 bit converter is exact
    assert np.array_equal(O.bf16_bits_to_f64(O.f32_to_bf16_bits(r.astype(np.float32))), r)
    # neighbours of r on the bf16 grid
    bits = O.f32_to_bf16_bits(r.astype(np.float32)).astype(np.int32)
    sign = np.where(r < 0, -1, 1)
    up = O.bf16_bits_to_f64((bits + 1).astype(np.uint16))
    dn = O.bf16_bits_to_f64(np.where((bits & 0x7FFF) == 0, bits ^ 0x8000, bits - 1).astype(np.uint16))
    del sign
    err = np.abs(x - r)
    assert np.all(err <= np.abs(x - up))
    assert np.all(err <= np.abs(x - dn))
    # hand-made ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert O.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert O.round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert O.round_to_bf16(np.array([-(1 + 2 ** -8)]))[0] == -1.0


# --------------------------------------------------------------------------
# RMSNorm: closed forms and a library routine
# --------------------------------------------------------------------------

def test_rmsnorm_closed_form_mean_square():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 3, 128)) * np.array([1e-4, 1.0, 30.0])[None, :, None]
    y = O.rmsnorm(x, np.ones(128), EPS)
    for n in range(7):
        for h in range(3):
            ms = sum(float(v) * float(v) for v in x[n, h]) / 128.0
            got = sum(float(v) * float(v) for v in y[n, h]) / 128.0
            assert got == pytest.approx(ms / (ms + EPS), rel=1e-12)


def test_rmsnorm_hand_example_and_gamma():
    x = np.zeros((1, 1, 128))
    x[0, 0, 0], x[0, 0, 1] = 3.0, 4.0
    g = np.full(128, 2.0)
    y = O.rmsnorm(x, g, 0.0)
    # mean square = 25/128, so y = x * sqrt(128) / 5 * 2
    assert y[0, 0, 0] == pytest.approx(3 * math.sqrt(128) / 5 * 2, rel=1e-14)
    assert y[0, 0, 1] == pytest.approx(4 * math.sqrt(128) / 5 * 2, rel=1e-14)
    assert np.all(y[0, 0, 2:] == 0)
    # eps enters under the square root: x = 0 except one entry of size sqrt(eps*128)
    x2 = np.zeros((1, 1, 128))
    x2[0, 0, 5] = math.sqrt(EPS * 128)
    y2 = O.rmsnorm(x2, np.ones(128), EPS)
    assert y2[0, 0, 5] == pytest.approx(math.sqrt(128) / math.sqrt(2), rel=1e-12)


def test_rmsnorm_per_head_gamma_and_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, 4, 128))
    g = 1 + 0.1 * rng.standard_normal((4, 128))
    y = O.rmsnorm(x, g, EPS)
    for h in range(4):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x[:, h, :]), (128,),
                                           weight=torch.from_numpy(g[h]), eps=EPS).numpy()
        np.testing.assert_allclose(y[:, h, :], ref, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# RoPE: hand-derived rotations, invariants, complex formulation
# --------------------------------------------------------------------------

def _unit(i, d=128):
    e = np.zeros((1, d))
    e[0, i] = 1.0
    return e


@pytest.mark.parametrize("i,pos,angle,partner", [
    (0, (1, 0, 0), 1.0, 16),                          # t section, j=0: omega = 1
    (5, (3, 0, 0), 3 * 10000 ** (-10 / 32), 21),       # t section, j=5
    (32, (0, 2, 0), 2.0, 56),                          # h section starts at 32, half 24
    (32 + 12, (0, 7, 0), 7 * 10000 ** (-0.5), 56 + 12),
    (80, (0, 0, 4), 4.0, 104),                         # w section starts at 80
    (80 + 23, (0, 0, 11), 11 * 10000 ** (-46 / 48), 104 + 23),
])
def test_rope_unit_vectors(i, pos, angle, partner):
    # textbook rotation: first half (a) -> a cos, its partner b gets + a sin
    y = O.rope(_unit(i), np.array([pos]), SECTIONS, THETA)
    expect = np.zeros(128)
    expect[i], expect[partner] = math.cos(angle), math.sin(angle)
    np.testing.assert_allclose(y[0], expect, atol=1e-15)
    # the partner (second half) rotates to (-sin, cos)
    y2 = O.rope(_unit(partner), np.array([pos]), SECTIONS, THETA)
    expect2 = np.zeros(128)
    expect2[i], expect2[partner] = -math.sin(angle), math.cos(angle)
    np.testing.assert_allclose(y2[0], expect2, atol=1e-15)


def test_rope_axis_isolation():
    # moving along one axis leaves the other two sections untouched
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 128))
    for axis, (lo, hi) in enumerate([(0, 32), (32, 80), (80, 128)]):
        p = np.zeros((1, 3), dtype=np.int64)
        p[0, axis] = 9
        y = O.rope(x, p, SECTIONS, THETA)
        mask = np.ones(128, bool)
        mask[lo:hi] = False
        assert np.array_equal(y[0, mask], x[0, mask])
        assert not np.allclose(y[0, lo:hi], x[0, lo:hi])


def test_rope_identity_at_zero_and_norm_preservation():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 3, 128))
    pos = rng.integers(-300, 300, size=(50, 3))
    assert np.array_equal(O.rope(x, np.zeros((50, 3), int), SECTIONS, THETA), x)
    y = O.rope(x, pos, SECTIONS, THETA)
    for off, s in [(0, 32), (32, 48), (80, 48)]:
        half = s // 2
        for j in range(half):
            nx = x[..., off + j] ** 2 + x[..., off + j + half] ** 2
            ny = y[..., off + j] ** 2 + y[..., off + j + half] ** 2
            np.testing.assert_allclose(ny, nx, rtol=1e-13, atol=1e-13)


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((40, 128))
    k = rng.standard_normal((40, 128))
    pq = rng.integers(0, 100, size=(40, 3))
    pk = rng.integers(0, 100, size=(40, 3))
    base = np.sum(O.rope(q, pq, SECTIONS, THETA) * O.rope(k, pk, SECTIONS, THETA), axis=1)
    for axis in range(3):
        d = np.zeros(3, dtype=np.int64)
        d[axis] = 37
        moved = np.sum(O.rope(q, pq + d, SECTIONS, THETA) * O.rope(k, pk + d, SECTIONS, THETA), axis=1)
        np.testing.assert_allclose(moved, base, rtol=1e-11, atol=1e-11)
    # and it does depend on the difference
    d = np.array([0, 0, 5])
    moved = np.sum(O.rope(q, pq + d, SECTIONS, THETA) * O.rope(k, pk, SECTIONS, THETA), axis=1)
    assert np.max(np.abs(moved - base)) > 1e-3


def test_rope_composition():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((20, 2, 128))
    p1 = rng.integers(0, 60, size=(20, 3))
    p2 = rng.integers(0, 60, size=(20, 3))
    a = O.rope(O.rope(x, p1, SECTIONS, THETA), p2, SECTIONS, THETA)
    b = O.rope(x, p1 + p2, SECTIONS, THETA)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


def test_rope_complex_formulation():
    # (x_j + i x_{j+half}) * exp(i phi), written with Python complex numbers
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 128))
    pos = rng.integers(0, 250, size=(6, 3))
    y = O.rope(x, pos, SECTIONS, THETA)
    for n in range(6):
        off = 0
        for axis, s in enumerate(SECTIONS):
            half = s // 2
            for j in range(half):
                w = 10000.0 ** (-(2.0 * j) / s)
                z = complex(x[n, off + j], x[n, off + j + half]) * complex(
                    math.cos(pos[n, axis] * w), math.sin(pos[n, axis] * w))
                assert y[n, off + j] == pytest.approx(z.real, abs=1e-12)
                assert y[n, off + j + half] == pytest.approx(z.imag, abs=1e-12)
            off += s


# --------------------------------------------------------------------------
# attention: invariants, closed forms, library routine, brute force
# --------------------------------------------------------------------------

def test_softmax_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(10)
    s = rng.standard_normal((30, 500)) * 20
    p = O.softmax_rows(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(p >= 0)
    np.testing.assert_allclose(O.softmax_rows(s + 1234.5), p, rtol=1e-9, atol=1e-300)


def test_attention_closed_forms():
    rng = np.random.default_rng(11)
    n, d = 300, 128
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d)) + rng.uniform(-2, 2, size=(1, d))
    # N = 1 gives O = V
    np.testing.assert_allclose(O.attention_head(k[:1], k[:1], v[:1], 0.1), v[:1], rtol=1e-15)
    # Q = 0 gives the mean of V over all keys
    o = O.attention_head(np.zeros((5, d)), k, v, 1 / math.sqrt(d))
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=1e-12, atol=1e-14)
    # V = 1 gives 1
    q = rng.standard_normal((17, d)) * 3
    o1 = O.attention_head(q, k, np.ones((n, d)), 1 / math.sqrt(d))
    np.testing.assert_allclose(o1, 1.0, rtol=1e-13)
    # one key aligned far above all others picks its value row
    q2 = np.zeros((1, d))
    q2[0, 0] = 1.0
    k2 = np.zeros((n, d))
    k2[n - 1, 0] = 200.0
    o2 = O.attention_head(q2, k2, v, 1.0)
    np.testing.assert_allclose(o2[0], v[n - 1], rtol=1e-12)


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(12)
    n, h, d = 200, 3, 128
    q, k, v = (rng.standard_normal((n, h, d)) for _ in range(3))
    scale = 1 / math.sqrt(d)
    ours = O.attention(q, k, v, scale)
    tq, tk, tv = (torch.from_numpy(a).permute(1, 0, 2) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    np.testing.assert_allclose(ours, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-13)


def test_prep_then_attention_matches_torch_when_rope_is_identity():
    # all positions zero and bf16 inputs: RMSNorm + SDPA from torch in fp64
    wl = W.ragged_workload(70, 2)
    inp = W.make_inputs(0, wl)
    pos0 = np.zeros_like(inp.pos)
    qp = O.prep(inp.q, inp.gamma_q, pos0, SECTIONS, THETA, EPS)
    kp = O.prep(inp.k, inp.gamma_k, pos0, SECTIONS, THETA, EPS)
    v = O.bf16_bits_to_f64(inp.v)
    ours = O.attention(qp, kp, v, 1 / math.sqrt(128))

    def t(bits):
        return torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64)

    tq = torch.nn.functional.rms_norm(t(inp.q), (128,), weight=t(inp.gamma_q), eps=EPS)
    tk = torch.nn.functional.rms_norm(t(inp.k), (128,), weight=t(inp.gamma_k), eps=EPS)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(1, 0, 2), tk.permute(1, 0, 2), t(inp.v).permute(1, 0, 2), scale=1 / math.sqrt(128))
    np.testing.assert_allclose(ours, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-13)


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(13)
    n, h, d = 9, 2, 128
    q, k, v = (rng.standard_normal((n, h, d)) for _ in range(3))
    ours = O.attention(q, k, v, 0.3)
    for hh in range(h):
        for i in range(n):
            logits = [0.3 * sum(q[i, hh, c] * k[j, hh, c] for c in range(d)) for j in range(n)]
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            tot = sum(w)
            for c in range(0, d, 17):
                want = sum(w[j] * v[j, hh, c] for j in range(n)) / tot
                assert ours[i, hh, c] == pytest.approx(want, rel=1e-12, abs=1e-14)


def test_attention_rows_subset_equals_full():
    rng = np.random.default_rng(14)
    n, d = 700, 128
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    full = O.attention_head(q, k, v, 0.09)
    rows = np.array([0, 1, 255, 256, 511, 699])
    np.testing.assert_allclose(O.attention_rows_head(q[rows], k, v, 0.09, block=4), full[rows],
                               rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# int8 quantiser: second scalar route, hand cases, exact integer scores
# --------------------------------------------------------------------------

def _f32(x):
    """Round a Python float to the nearest float32 (via struct, nearest-even)."""
    return struct.unpack("f", struct.pack("f", x))[0]


def _quant_scalar(block_vals):
    """Scalar int8 quantiser using fp64 arithmetic + one fp32 rounding per step.

    Division and multiplication of two float32 values done in float64 and then
    rounded once to float32 equal the correctly rounded float32 results
    (float64 has more than 2*24+2 bits), so this reaches the same values by a
    different route than numpy float32 arithmetic.
    """
    a = max(abs(float(v)) for v in block_vals)
    if a == 0.0:
        return [0] * len(block_vals), 0.0
    s = _f32(a / 127.0)
    inv = _f32(127.0 / a)
    codes = []
    for v in block_vals:
        t = _f32(float(v) * inv)
        r = round(t)                    # Python round(): ties to even
        codes.append(max(-127, min(127, r)))
    return codes, s


def test_quantizer_matches_scalar_route():
    rng = np.random.default_rng(15)
    n, d = 64 * 3 + 17, 8
    x = O.bf16_bits_to_f64(O.f32_to_bf16_bits(
        (rng.standard_normal((n, d)) * rng.uniform(0.01, 30, size=(n, 1))).astype(np.float32))).astype(np.float32)
    x[64:128] = 0.0                                   # an all-zero block
    codes, scales = O.quantize_i8(x)
    assert scales.shape == (4,)
    for b in range(4):
        blk = x[b * 64:(b + 1) * 64]
        c, s = _quant_scalar(blk.ravel())
        assert np.float32(s) == scales[b]
        assert list(codes[b * 64:(b + 1) * 64].ravel()) == c


def test_quantizer_hand_cases():
    # absmax 127 -> scale exactly 1 and codes = rint(x), ties to even
    x = np.zeros((64, 4), dtype=np.float32)
    x[0, :] = [127.0, -127.0, 0.5, 1.5]
    x[1, :] = [2.5, -2.5, -0.5, 3.5]
    codes, scales = O.quantize_i8(x)
    assert scales[0] == np.float32(1.0)
    assert list(codes[0]) == [127, -127, 0, 2]
    assert list(codes[1]) == [2, -2, 0, 4]
    # one-token tail block, and a zero block gives scale 0
    x2 = np.zeros((65, 2), dtype=np.float32)
    x2[64, :] = [-3.0, 1.5]
    c2, s2 = O.quantize_i8(x2)
    assert s2[0] == 0 and np.all(c2[:64] == 0)
    assert s2[1] == np.float32(3.0) / np.float32(127.0)
    assert list(c2[64]) == [-127, 64]       # 1.5 * (127/3) = 63.5 -> fl32 then even -> 64


def test_quantizer_error_bound():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((640, 128)).astype(np.float32)
    codes, scales = O.quantize_i8(x)
    s = np.repeat(scales, 64)[:, None].astype(np.float64)
    err = np.abs(codes.astype(np.float64) * s - x)
    assert np.all(err <= s * 0.5 * (1 + 1e-5) + 1e-12)
    assert np.max(np.abs(codes)) == 127


def test_scores_i32_exact_against_integer_matmul():
    rng = np.random.default_rng(17)
    a = rng.integers(-127, 128, size=(70, 128)).astype(np.int8)
    b = rng.integers(-127, 128, size=(90, 128)).astype(np.int8)
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(O.scores_i32(a, b), ref)
    # extreme magnitude: all 127 / -127 gives +-128*127^2
    full = np.full((1, 128), 127, dtype=np.int8)
    assert O.scores_i32(full, -full)[0, 0] == -128 * 127 * 127


def test_int8_attention_reduces_to_float_when_lossless():
    # integer values with block absmax 127 quantise losslessly (scale exactly 1)
    rng = np.random.default_rng(18)
    n, d = 130, 128
    q = rng.integers(-20, 21, size=(n, d)).astype(np.float32)
    k = rng.integers(-20, 21, size=(n, d)).astype(np.float32)
    q[::64, 0] = 127.0
    k[::64, 1] = -127.0
    v = rng.standard_normal((n, d))
    cq, sq = O.quantize_i8(q)
    ck, sk = O.quantize_i8(k)
    assert np.all(sq == 1) and np.all(sk == 1)
    rows = np.arange(n)
    got = O.attention_i8_rows_head(rows, cq, sq, ck, sk, v, 1e-3)
    want = O.attention_head(q.astype(np.float64), k.astype(np.float64), v, 1e-3)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
    # a per-block scale of 2 on the keys of block 1 doubles those logits
    k2 = k.copy()
    k2[64:128] *= 2
    ck2, sk2 = O.quantize_i8(k2)
    assert sk2[1] == 2 and sk2[0] == 1
    got2 = O.attention_i8_rows_head(rows, cq, sq, ck2, sk2, v, 1e-3)
    want2 = O.attention_head(q.astype(np.float64), k2.astype(np.float64), v, 1e-3)
    np.testing.assert_allclose(got2, want2, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# E4M3 encoder / FP8 V quantiser: OCP format values, exhaustive round trip,
# brute-force nearest value, a library cast, and the format's error bound
# --------------------------------------------------------------------------

def _e4m3_table():
    """Every finite E4M3 value with its code, from the bit fields (sign, 4-bit
    exponent with bias 7, 3-bit mantissa; exponent field 0 is subnormal)."""
    codes, vals = [], []
    for b in range(256):
        e, m = (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            continue                                    # NaN
        mag = m / 8.0 * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        codes.append(b)
        vals.append(-mag if b & 0x80 else mag)
    return np.array(codes, dtype=np.uint8), np.array(vals)


def test_e4m3_format_values():
    cases = [(448.0, 0x7E), (-448.0, 0xFE), (1.0, 0x38), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01),
             (7 * 2.0 ** -9, 0x07), (0.0, 0x00), (-0.0, 0x80), (240.0, 0x77), (1.75, 0x3E), (0.5, 0x30)]
    xs = np.array([c[0] for c in cases])
    got = O.e4m3_bits(xs)
    assert [int(g) for g in got] == [c[1] for c in cases]
    dec = O.e4m3_bits_to_f64(np.array([c[1] for c in cases], dtype=np.uint8))
    assert np.array_equal(dec, xs) and np.array_equal(np.signbit(dec), np.signbit(xs))
    with pytest.raises(ValueError):
        O.e4m3_bits(np.array([449.0]))
    with pytest.raises(ValueError):
        O.e4m3_bits_to_f64(np.array([0x7F], dtype=np.uint8))


def test_e4m3_exhaustive_round_trip_and_sign_symmetry():
    codes, vals = _e4m3_table()
    assert len(codes) == 254
    assert np.array_equal(O.e4m3_bits_to_f64(codes), vals)
    assert np.array_equal(O.e4m3_bits(vals), codes)
    x = np.random.default_rng(40).uniform(0, 448, 20000)
    assert np.array_equal(O.e4m3_bits(-x), O.e4m3_bits(x) | 0x80)


def test_e4m3_ties_go_to_even_mantissa():
    # midpoints between neighbours: the one with an even mantissa field wins
    pairs = [(1.0625, 0x38), (1.1875, 0x3A), (1.5 * 2.0 ** -9, 0x02), (0.5 * 2.0 ** -9, 0x00),
             (7.5 * 2.0 ** -9, 0x08), (432.0, 0x7E), (2.0 ** -6 * (1 + 1 / 16), 0x08)]
    for x, code in pairs:
        assert int(O.e4m3_bits(np.array([x]))[0]) == code, x
    # 0.484375 lies between 0.46875 (0x2F, mantissa 7) and 0.5 (0x30): ties to 0.5
    assert int(O.e4m3_bits(np.array([0.484375]))[0]) == 0x30


def test_e4m3_brute_force_nearest_value():
    """Nearest finite value by exhaustive search; exact ties broken to the even code."""
    codes, vals = _e4m3_table()
    rng = np.random.default_rng(41)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-0.05, 0.05, 3000),
                        np.ldexp(rng.uniform(-1, 1, 2000), rng.integers(-12, 9, 2000))]).astype(np.float32)
    got = O.e4m3_bits(x.astype(np.float64))
    for xi, g in zip(x.astype(np.float64), got):
        d = np.abs(vals - xi)
        best = np.nonzero(d == d.min())[0]
        cand = [c for c in codes[best] if (c & 0x80) == (0x80 if np.signbit(xi) else 0) or xi == 0] or list(codes[best])
        if len(cand) > 1:
            cand = [c for c in cand if (c & 1) == 0]
        assert int(g) in [int(c) for c in cand], (xi, g, cand)


def test_e4m3_matches_torch_float8_cast():
    rng = np.random.default_rng(42)
    x = np.concatenate([rng.uniform(-448, 448, 200000), rng.uniform(-2.0 ** -5, 2.0 ** -5, 100000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_bits(x.astype(np.float64)), ref)


def test_quantize_v_fp8_hand_cases_and_bound():
    v = np.zeros((5, 4), dtype=np.float32)
    v[:, 0] = [1.0, -2.0, 0.5, 0.0, 0.25]          # absmax 2 -> scale 2/448, 1.0 -> 224
    v[:, 1] = [0.0] * 5                            # zero channel: scale 0, codes 0
    v[:, 2] = [-3.0, 1.0, 3.0, 0.0, 0.0]
    v[:, 3] = [1e-3, 0, 0, 0, 0]
    codes, scales = O.quantize_v_fp8(v)
    assert scales[0] == np.float32(2.0) / np.float32(448.0)
    assert scales[1] == 0 and np.all(codes[:, 1] == 0)
    assert int(codes[1, 0]) == 0xFE and int(codes[2, 2]) == 0x7E and int(codes[0, 2]) == 0xFE
    assert int(codes[0, 0]) == 0x76                 # 224 = 1.75 * 2^7: exponent field 14, mantissa 6
    assert int(codes[0, 3]) == 0x7E                 # a lone value is its channel's absmax
    # the format's bound: relative 2^-4 for normal codes, absolute 2^-10 * scale below
    rng = np.random.default_rng(43)
    x = (rng.standard_normal((3000, 128)) * rng.uniform(0.01, 50, size=(1, 128))).astype(np.float32)
    c, s = O.quantize_v_fp8(x)
    deq = O.dequantize_v_fp8(c, s)
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s[None, :].astype(np.float64) * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    assert np.all(np.max(np.abs(deq), axis=0) == 448.0 * s.astype(np.float64))


# --------------------------------------------------------------------------
# FP8 P V reference: its exact part against the (separately pinned) exact
# attention and a closed form, its bound against a simulation of the rounded
# numerators with torch's own E4M3 cast, and the bound's power to reject a
# wrong rounding
# --------------------------------------------------------------------------

def _simulated_fp8_pv(s, v_hat, stale, cast):
    """Numerators a * exp(s - m') with a stale running max m' = max s - stale
    (per row), each rounded by ``cast``; divided by the unrounded sum."""
    a = 2.0 ** O.FP8_P_LOG2_FACTOR
    m = s.max(axis=1, keepdims=True) - stale[:, None]
    x = a * np.exp(s - m)
    assert x.max() < 448.0
    return (cast(x) @ v_hat) / x.sum(axis=1, keepdims=True)


def _torch_e4m3(x):
    return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8v_reference_exact_part():
    rng = np.random.default_rng(60)
    n, d = 300, 128
    q = rng.standard_normal((17, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d)) * rng.uniform(0.1, 3, size=(1, d))
    scale = 1 / math.sqrt(d)
    ref, bound = O.attention_fp8v_rows((q @ k.T) * scale, v)
    assert np.allclose(ref, O.attention_rows_head(q, k, v, scale), rtol=0, atol=1e-13)
    assert np.all(bound > 0)
    # equal scores: the mean of V; bound = 2^-4 mean|V| + 2^-10 / (2^0.8 N) sum|V|
    ref, bound = O.attention_fp8v_rows(np.full((2, n), 0.7), v)
    assert np.allclose(ref, v.mean(axis=0)[None], rtol=0, atol=1e-13)
    expect = 2.0 ** -4 * np.abs(v).mean(axis=0) + 2.0 ** -10 / (2.0 ** 0.8 * n) * np.abs(v).sum(axis=0)
    assert np.allclose(bound, expect[None], rtol=1e-12, atol=0)


def test_fp8v_reference_bound_holds_for_rounded_numerators():
    # diffuse rows, sharp rows (numerators deep in the subnormal range) and a
    # running max up to 8 base-2 units below the true max (numerators up to 2^8 * 2^0.8)
    rng = np.random.default_rng(61)
    n, d = 500, 64
    v_hat = rng.standard_normal((n, d)) * rng.uniform(0.05, 4, size=(1, d))
    worst = 0.0
    for spread in (0.1, 1.0, 2.0, 4.0, 8.0):
        s = rng.standard_normal((40, n)) * spread
        stale = rng.uniform(0, 8 * math.log(2), size=40) * (rng.uniform(size=40) < 0.5)
        ref, bound = O.attention_fp8v_rows(s, v_hat)
        for cast in (_torch_e4m3, lambda x: O.e4m3_bits_to_f64(O.e4m3_bits(x))):
            sim = _simulated_fp8_pv(s, v_hat, stale, cast)
            use = np.abs(sim - ref) / bound
            assert np.all(use <= 1 + 1e-9), (spread, use.max())
            worst = max(worst, float(use.max()))
    assert worst > 0.05       # not a vacuous bound


def test_fp8v_reference_bound_rejects_truncation():
    # rounding toward zero (errors up to one whole spacing) must break the bound:
    # every numerator 1.1249 truncates to 1.0
    n, d = 64, 8
    s = np.full((1, n), math.log(1.1249 / 2.0 ** 0.8))
    v_hat = np.ones((n, d))
    ref, bound = O.attention_fp8v_rows(s, v_hat)

    def trunc(x):
        e = np.floor(np.log2(x))
        return np.floor(x / 2.0 ** (e - 3)) * 2.0 ** (e - 3)
    sim = _simulated_fp8_pv(s, v_hat, np.zeros(1), trunc)
    assert np.all(np.abs(sim - ref) > bound)
    sim_ok = _simulated_fp8_pv(s, v_hat, np.zeros(1), _torch_e4m3)
    assert np.all(np.abs(sim_ok - ref) <= bound)


# --------------------------------------------------------------------------
# K smoothing: the fixed-order mean, a scalar route, exactness bound,
# softmax invariance, and its effect on the int8 quantisation error
# --------------------------------------------------------------------------

def _mean_scalar(col, block=64):
    """Per-channel mean with numpy float32 scalars, one addition at a time."""
    blocks = []
    for b in range(0, len(col), block):
        s = np.float32(0.0)
        for v in col[b:b + block]:
            s = np.float32(s + np.float32(v))
        blocks.append(s)
    t = np.float32(0.0)
    for s in blocks:
        t = np.float32(t + s)
    return np.float32(t / np.float32(len(col)))


def test_k_mean_blocked_matches_scalar_route_and_bound():
    rng = np.random.default_rng(50)
    for n in (1, 63, 64, 65, 200):
        x = O.bf16_bits_to_f64(O.f32_to_bf16_bits(
            (rng.standard_normal((n, 6)) * 3 + rng.uniform(-5, 5, 6)).astype(np.float32))).astype(np.float32)
        mu = O.k_mean_blocked(x)
        for c in range(6):
            assert mu[c] == _mean_scalar(x[:, c]), (n, c)
        exact = x.astype(np.float64).mean(axis=0)
        # a running float32 sum of m terms is within m * 2^-24 * sum|x| of the exact sum
        bound = (n + 1) * 2.0 ** -24 * np.abs(x.astype(np.float64)).sum(axis=0) / n + 2.0 ** -24 * np.abs(exact)
        assert np.all(np.abs(mu - exact) <= bound)
    mu, xs = O.smooth_k(np.array([[1.0, -2.0], [3.0, 4.0]], dtype=np.float32))
    assert list(mu) == [2.0, 1.0] and xs.tolist() == [[-1.0, -3.0], [1.0, 3.0]]


def test_k_smoothing_is_softmax_invariant():
    rng = np.random.default_rng(51)
    n, d = 300, 128
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    k += rng.uniform(-3, 3, d)[None, :]
    mu = k.mean(axis=0)
    a = O.attention_head(q, k, v, 0.09)
    b = O.attention_head(q, k - mu[None, :], v, 0.09)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)


def test_k_smoothing_lowers_int8_error_on_biased_keys():
    # a channel-wise offset much larger than the spread: without smoothing the
    # block absmax is dominated by it; after subtracting the mean the codes
    # resolve the spread, and the int32 scores (offset by a row constant) stay exact
    rng = np.random.default_rng(52)
    n, d = 256, 128
    k = (rng.standard_normal((n, d)) * 0.3 + rng.uniform(2, 6, d)[None, :]).astype(np.float32)
    k = O.bf16_bits_to_f64(O.f32_to_bf16_bits(k)).astype(np.float32)
    c0, s0 = O.quantize_i8(k)
    mu, ks = O.smooth_k(k)
    c1, s1 = O.quantize_i8(ks)
    blk = np.arange(n) // 64
    e0 = np.abs(c0 * s0[blk][:, None].astype(np.float64) - k)
    e1 = np.abs(c1 * s1[blk][:, None].astype(np.float64) + mu[None, :].astype(np.float64) - k)
    assert e1.mean() < 0.2 * e0.mean()
