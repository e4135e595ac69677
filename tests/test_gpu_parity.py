"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Small cases are compared element by element over all outputs; the full-size
workloads on sampled rows and heads, plus closed forms that hold at any size.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from audio_video_diffusion_amd import h3attn as A
from audio_video_diffusion_amd import workloads as W

from gpu_util import (MAX_ABS, MEAN_ABS, REL_L2, REL_L2_I8, SCALE, SECTIONS, THETA, EPS, check,
                      errors, f64, oracle_rows_bf16, oracle_rows_i8, problem_for, run_forward,
                      run_prep, sample_rows)

pytestmark = pytest.mark.gpu

TAIL_SWEEP = [1, 2, 31, 63, 64, 65, 127, 128, 129, 255, 256, 257, 312, 1000, 4099]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def _prep_ref(inp):
    qp = O.prep(inp.q, inp.gamma_q, inp.pos, SECTIONS, THETA, EPS)
    kp = O.prep(inp.k, inp.gamma_k, inp.pos, SECTIONS, THETA, EPS)
    return qp, kp


def _hnd_to_nhd(t, n):
    return f64(t)[:, :n, :].transpose(1, 0, 2)


# ---------------------------------------------------------------------------
# prep
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,n,h,per_head", [(0, None, None, False), (7, 1000, 3, True), (8, 65, 2, False),
                                              (9, 1, 1, False)])
def test_prep_bf16_matches_oracle(cfg, n, h, per_head):
    wl = W.WORKLOADS[0] if n is None else W.ragged_workload(n, h)
    inp = W.make_inputs(cfg, wl, per_head_gamma=per_head)
    p = problem_for(wl)
    print(f"    N={wl.n_tokens} H={wl.heads}", flush=True)
    q_out, k_out, _, _ = run_prep(p, W.device_inputs(inp))
    qp, kp = _prep_ref(inp)
    for got_t, ref in ((q_out, qp), (k_out, kp)):
        got_all = f64(got_t)
        got = got_all[:, :wl.n_tokens, :].transpose(1, 0, 2)
        # bf16 rounding of an fp32 evaluation: half an ulp (<= 2^-8 |y|) plus an fp32
        # evaluation error of at most 2^-14 |y| that may tip a near-midpoint rounding
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * (1 + 2.0 ** -6) * np.abs(ref) + 4e-6
        assert np.all(err <= bound), (np.max(err - bound), np.max(err))
        assert np.all(got_all[:, wl.n_tokens:, :] == 0)           # pad rows zeroed


@pytest.mark.parametrize("cfg", [W.HEADLINE, 4])
def test_prep_full_workload_sampled_rows(cfg):
    # the bf16 prep at full size, every head, on sampled rows (the sequence
    # ends, the modality boundaries, random rows; the largest positions of the
    # grid are at its end), element by element against the oracle; pad rows zero
    wl = W.WORKLOADS[cfg]
    print(f"    {wl.name} N={wl.n_tokens}", flush=True)
    inp = W.make_inputs(cfg)
    q_out, k_out, _, _ = run_prep(problem_for(wl), W.device_inputs(inp))
    rows = sample_rows(wl, n_random=256)
    n = wl.n_tokens
    for got_t, x, g in ((q_out, inp.q, inp.gamma_q), (k_out, inp.k, inp.gamma_k)):
        got = f64(got_t[:, torch.from_numpy(rows).cuda(), :]).transpose(1, 0, 2)
        ref = O.prep(x[rows], g, inp.pos[rows], SECTIONS, THETA, EPS)
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * (1 + 2.0 ** -6) * np.abs(ref) + 4e-6
        assert np.all(err <= bound), (np.max(err - bound), np.max(err))
        assert torch.count_nonzero(got_t[:, n:, :]).item() == 0


def test_prep_and_forward_on_interleaved_qkv_views():
    # Q/K/V as strided views of one interleaved projection output [N, 3, H, d]
    wl = W.ragged_workload(777, 3)
    inp = W.make_inputs(11, wl, per_head_gamma=True)
    n, h = wl.n_tokens, wl.heads
    qkv = torch.empty((n, 3, h, 128), dtype=torch.bfloat16, device="cuda")
    for i, bits in enumerate((inp.q, inp.k, inp.v)):
        qkv[:, i] = W.bits_to_torch(bits)
    dev = W.device_inputs(inp)
    dev["q"], dev["k"], dev["v"] = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    p = problem_for(wl)
    q_out, k_out, _, _ = run_prep(p, dev)
    # output into a strided view too: every other 128-wide slot of [N, H, 2, d]
    obuf = torch.full((n, h, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    run_forward(p, q_out, k_out, dev["v"], o=obuf[:, :, 0])
    assert torch.all(obuf[:, :, 1] == 7.0)
    qp, kp = _prep_ref(inp)
    ref = O.attention(qp, kp, O.bf16_bits_to_f64(inp.v), SCALE)
    check(f64(obuf[:, :, 0]), ref, what="strided e2e")


# ---------------------------------------------------------------------------
# forward, bf16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [None] + TAIL_SWEEP)
def test_forward_bf16_matches_oracle(n):
    wl = W.WORKLOADS[0] if n is None else W.ragged_workload(n, 2)
    inp = W.make_inputs(0 if n is None else 100 + n, wl)
    p = problem_for(wl)
    print(f"    N={wl.n_tokens} H={wl.heads}", flush=True)
    dev = W.device_inputs(inp)
    q_out, k_out, _, _ = run_prep(p, dev)
    o = run_forward(p, q_out, k_out, dev["v"])
    got = f64(o)
    v = O.bf16_bits_to_f64(inp.v)
    # attention stage alone: oracle attention on the GPU's own prepped Q'/K'
    ref_stage = O.attention(_hnd_to_nhd(q_out, wl.n_tokens), _hnd_to_nhd(k_out, wl.n_tokens), v, SCALE)
    check(got, ref_stage, max_abs=1e-2, mean_abs=MEAN_ABS, rel_l2=6e-3, what="stage")
    # whole path against the fp64 oracle
    qp, kp = _prep_ref(inp)
    check(got, O.attention(qp, kp, v, SCALE), what="e2e")


def test_forward_sharp_softmax_rescaling():
    # gamma x 4 makes logits ~16x sharper, so the running max moves by more than
    # the lazy-rescale threshold while streaming the keys
    wl = W.ragged_workload(3000, 2)
    inp = W.make_inputs(21, wl)
    four = O.f32_to_bf16_bits((O.bf16_bits_to_f64(inp.gamma_q) * 4).astype(np.float32))
    inp.gamma_q = four
    inp.gamma_k = four
    p = problem_for(wl)
    dev = W.device_inputs(inp)
    q_out, k_out, _, _ = run_prep(p, dev)
    o = run_forward(p, q_out, k_out, dev["v"])
    v = O.bf16_bits_to_f64(inp.v)
    ref = O.attention(_hnd_to_nhd(q_out, wl.n_tokens), _hnd_to_nhd(k_out, wl.n_tokens), v, SCALE)
    check(f64(o), ref, max_abs=2e-2, mean_abs=2e-3, rel_l2=1e-2, what="sharp stage")


def test_forward_is_deterministic():
    wl = W.ragged_workload(5000, 3)
    inp = W.make_inputs(22, wl)
    p = problem_for(wl)
    dev = W.device_inputs(inp)
    q_out, k_out, _, _ = run_prep(p, dev)
    a = run_forward(p, q_out, k_out, dev["v"])
    b = run_forward(p, q_out, k_out, dev["v"])
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    q2, k2, _, _ = run_prep(p, dev)
    assert torch.equal(q2.view(torch.int16), q_out.view(torch.int16))


# ---------------------------------------------------------------------------
# closed forms at the full 129,410-token size (forward on crafted Q'/K')
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def full_shape():
    wl = W.WORKLOADS[W.HEADLINE]
    p = problem_for(wl)
    npad = A.padded_tokens(p)
    return wl, p, npad


def test_closed_form_q_zero_v_one_is_exactly_one(full_shape):
    wl, p, npad = full_shape
    n, h = wl.n_tokens, wl.heads
    qz = torch.zeros((h, npad, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(5)
    k = torch.randn((h, npad, 128), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.ones((n, h, 128), dtype=torch.bfloat16, device="cuda")
    o = run_forward(p, qz, k, v)
    # exp(0) = 1 for every key: l = N exactly; any padded or dropped key breaks 1.0
    assert torch.all(o == 1.0)


def test_closed_form_q_zero_gives_mean_of_v(full_shape):
    wl, p, npad = full_shape
    n, h = wl.n_tokens, wl.heads
    qz = torch.zeros((h, npad, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(6)
    k = torch.randn((h, npad, 128), generator=g, device="cuda").to(torch.bfloat16)
    mu = (torch.rand((1, h, 128), generator=g, device="cuda") * 4 - 2)
    v = (torch.randn((n, h, 128), generator=g, device="cuda") + mu).to(torch.bfloat16)
    o = run_forward(p, qz, k, v).double().cpu().numpy()
    mean = v.double().mean(dim=0).cpu().numpy()
    err = np.abs(o - mean[None])
    assert np.all(err <= 2.0 ** -8 * np.abs(mean)[None] + 1e-5), err.max()


def test_closed_form_last_key_spike(full_shape):
    wl, p, npad = full_shape
    n, h = wl.n_tokens, wl.heads
    # only key N-1 is nonzero and aligned with every query: logit 20, all others 0
    q = torch.zeros((h, npad, 128), dtype=torch.bfloat16, device="cuda")
    q[:, :n, 0] = 1.0
    k = torch.zeros((h, npad, 128), dtype=torch.bfloat16, device="cuda")
    k[:, n - 1, 0] = 20.0 / SCALE
    g = torch.Generator(device="cuda").manual_seed(7)
    v = torch.randn((n, h, 128), generator=g, device="cuda").to(torch.bfloat16)
    o = run_forward(p, q, k, v).double()
    kf = k[:, n - 1, 0].double().cpu().numpy()[0] * SCALE          # bf16-rounded logit
    w_last = np.exp(kf) / (np.exp(kf) + (n - 1))
    vd = v.double()
    expect = w_last * vd[n - 1][None] + (1 - w_last) * (vd.sum(0) - vd[n - 1]) / (n - 1)
    rows = torch.tensor([0, 1, n // 2, n - 2, n - 1], device="cuda")
    d = (o[rows] - expect[None]).abs().max().item()
    assert d <= 2e-2, d
    assert w_last > 0.8


# ---------------------------------------------------------------------------
# full workloads on sampled rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_full_workload_sampled_rows_bf16(cfg):
    wl = W.WORKLOADS[cfg]
    print(f"    {wl.name} N={wl.n_tokens}", flush=True)
    inp = W.make_inputs(cfg)
    p = problem_for(wl)
    dev = W.device_inputs(inp)
    q_out, k_out, _, _ = run_prep(p, dev)
    o = run_forward(p, q_out, k_out, dev["v"])
    rows = sample_rows(wl)
    rows_t = torch.from_numpy(rows).cuda()
    got_rows = f64(o[rows_t])
    all_got, all_ref = [], []
    for h in (0, wl.heads // 2, wl.heads - 1):
        ref = oracle_rows_bf16(inp, h, rows)
        all_got.append(got_rows[:, h, :])
        all_ref.append(ref)
    check(np.stack(all_got), np.stack(all_ref), what=f"{wl.name} sampled")
    assert torch.isfinite(o.float()).all()


def test_block24_shape_sampled_rows_bf16():
    # the pages' own block-24 attention shape: 37,810 tokens, 56 heads
    wl = W.BLOCK24
    print(f"    {wl.name} N={wl.n_tokens} H={wl.heads}", flush=True)
    inp = W.make_inputs(100, wl)
    p = problem_for(wl)
    dev = W.device_inputs(inp)
    q_out, k_out, _, _ = run_prep(p, dev)
    o = run_forward(p, q_out, k_out, dev["v"])
    rows = sample_rows(wl, n_random=64)
    got_rows = f64(o[torch.from_numpy(rows).cuda()])
    heads = (0, 27, 55)
    ref = np.stack([oracle_rows_bf16(inp, h, rows) for h in heads])
    check(np.stack([got_rows[:, h, :] for h in heads]), ref, what=f"{wl.name} sampled")
    assert torch.isfinite(o.float()).all()


def test_head_shard_matches_full_heads():
    # one GPU's share of the heads (strided views of the full tensors) gives
    # bit-identical rows to the same heads of the full problem
    wl = W.ragged_workload(3000, 8)
    inp = W.make_inputs(61, wl)
    dev = W.device_inputs(inp)
    full = run_forward(problem_for(wl), *run_prep(problem_for(wl), dev)[:2], dev["v"])
    part = dataclasses.replace(wl, heads=3)
    view = {**dev, "q": dev["q"][:, :3], "k": dev["k"][:, :3], "v": dev["v"][:, :3]}
    ps = problem_for(part)
    q_out, k_out, _, _ = run_prep(ps, view)
    o = run_forward(ps, q_out, k_out, view["v"])
    assert torch.equal(o, full[:, :3])


# ---------------------------------------------------------------------------
# int8 Q/K path
# ---------------------------------------------------------------------------

def _prep_both(wl, inp):
    dev = W.device_inputs(inp)
    p16 = problem_for(wl)
    p8 = problem_for(wl, int8=True)
    q16, k16, _, _ = run_prep(p16, dev)
    q8, k8, qs, ks = run_prep(p8, dev)
    return dev, p16, p8, q16, k16, q8, k8, qs, ks


@pytest.mark.parametrize("cfg,n,h", [(0, None, None), (31, 1000, 3), (32, 63, 2), (33, 129, 2)])
def test_int8_codes_and_scales_bit_exact(cfg, n, h):
    wl = W.WORKLOADS[0] if n is None else W.ragged_workload(n, h)
    inp = W.make_inputs(cfg, wl)
    _, _, _, q16, k16, q8, k8, qs, ks = _prep_both(wl, inp)
    for b16, codes, scales in ((q16, q8, qs), (k16, k8, ks)):
        vals = f64(b16)
        codes_h = codes.cpu().numpy()
        scales_h = scales.cpu().numpy()
        for hh in range(wl.heads):
            c_ref, s_ref = O.quantize_i8(vals[hh, :wl.n_tokens].astype(np.float32))
            assert np.array_equal(scales_h[hh], s_ref)
            assert np.array_equal(codes_h[hh, :wl.n_tokens], c_ref)
            assert np.all(codes_h[hh, wl.n_tokens:] == 0)


def _scores_windows(n):
    """(row0, nrows, col0, ncols) windows: the sequence start, the end (the
    ragged last query tile and key block), single elements, a window that
    crosses several query tiles and key tiles, and one across the first
    384-row query tile edge."""
    w = [(0, min(n, 300), 0, min(n, 200)), (max(0, n - 70), min(70, n), max(0, n - 130), min(130, n)),
         (n // 3, 1, n // 2, 1), (5, min(n - 5, 250), 3, min(n - 3, 333)),
         (360, min(60, n - 360), 0, min(n, 100))]
    return [x for x in w if x[1] >= 1 and x[3] >= 1]


def _check_scores(p8, q8, k8, heads, windows, layouts=(0, 1)):
    for hh in heads:
        qc = q8[hh].cpu().numpy()
        kc = k8[hh].cpu().numpy()
        for (r0, nr, c0, nc) in windows:
            ref = O.scores_i32(qc[r0:r0 + nr], kc[c0:c0 + nc])
            for lay in layouts:
                out = torch.full((nr, nc), -1, dtype=torch.int32, device="cuda")
                A.debug_scores_i32(p8, q8, k8, hh, r0, nr, c0, nc, out, fp8v_layout=lay)
                assert np.array_equal(out.cpu().numpy().astype(np.int64), ref), (hh, r0, nr, c0, nc, lay)


@pytest.mark.parametrize("cfg,n,h", [(0, None, None), (41, 4099, 2), (42, 129, 1), (43, 1, 1), (44, 385, 2)])
def test_int8_scores_i32_bit_exact(cfg, n, h):
    # the int8 forward kernels' own Q'K'^T path (the bf16-V and the E4M3-V
    # forms' K' row orders) against exact integer products
    wl = W.WORKLOADS[0] if n is None else W.ragged_workload(n, h)
    inp = W.make_inputs(cfg, wl)
    _, _, p8, _, _, q8, k8, _, _ = _prep_both(wl, inp)
    _check_scores(p8, q8, k8, range(wl.heads), _scores_windows(wl.n_tokens))


# 383, 385, 769: either side of the int8 forward's 384-row query tiles (1000 and
# 65 also take rows past N_pad in the last tile)
@pytest.mark.parametrize("cfg,n,h", [(0, None, None), (51, 1000, 2), (52, 65, 2), (53, 4099, 2),
                                     (54, 383, 2), (55, 385, 2), (56, 769, 1)])
def test_int8_forward_matches_oracle(cfg, n, h):
    wl = W.WORKLOADS[0] if n is None else W.ragged_workload(n, h)
    inp = W.make_inputs(cfg, wl)
    dev, _, p8, q16, k16, q8, k8, qs, ks = _prep_both(wl, inp)
    o = run_forward(p8, q8, k8, dev["v"], qs, ks)
    got = f64(o)
    rows = np.arange(wl.n_tokens)
    qv, kv = f64(q16), f64(k16)
    ref_stage = np.stack([oracle_rows_i8(inp, hh, rows, q_bf16=qv[hh, :wl.n_tokens], k_bf16=kv[hh, :wl.n_tokens])
                          for hh in range(wl.heads)], axis=1)
    check(got, ref_stage, max_abs=1e-2, mean_abs=MEAN_ABS, rel_l2=6e-3, what="int8 stage")
    qp, kp = _prep_ref(inp)
    ref = O.attention(qp, kp, O.bf16_bits_to_f64(inp.v), SCALE)
    if n is None:       # the tiny workload itself: the absolute bounds of the workload definition
        check(got, ref, rel_l2=REL_L2_I8, what="int8 vs fp64")
    else:               # few keys -> O(1) outputs: the int8 step error is gated relatively
        check(got, ref, max_abs=2 * MAX_ABS, mean_abs=2 * MEAN_ABS, rel_l2=REL_L2_I8, what="int8 vs fp64")


def test_int8_full_workload_sampled_rows():
    cfg = 4
    wl = W.WORKLOADS[cfg]
    print(f"    {wl.name} N={wl.n_tokens}", flush=True)
    inp = W.make_inputs(cfg)
    dev = W.device_inputs(inp)
    p8 = problem_for(wl, int8=True)
    q8, k8, qs, ks = run_prep(p8, dev)
    o = run_forward(p8, q8, k8, dev["v"], qs, ks)
    rows = sample_rows(wl, n_random=64)
    got_rows = f64(o[torch.from_numpy(rows).cuda()])
    g, r = [], []
    for h in (0, wl.heads - 1):
        r.append(oracle_rows_i8(inp, h, rows))
        g.append(got_rows[:, h, :])
    check(np.stack(g), np.stack(r), rel_l2=REL_L2_I8, what="int8 full sampled")
    # the int32 scores of the forward kernels' own products are exact, on windows
    # at the start, across query-tile and key-tile edges in the middle, and at the
    # end, where the last key block holds 62 tokens
    n = wl.n_tokens
    assert n % 64 == 62
    windows = [(0, 40, 0, 70), (n // 2 - 20, 300, n // 2 - 100, 200), (n - 300, 300, n - 190, 190),
               (n - 1, 1, 0, 64), (7, 3, n - 62, 62)]
    _check_scores(p8, q8, k8, (5, wl.heads - 1), windows)


def test_int8_full_workload_codes_bit_exact():
    # the 243-frame workload's int8 codes and scales of two heads, bit-exact
    # against the oracle's quantiser applied to the GPU's own bf16 prep output
    cfg = 4
    wl = W.WORKLOADS[cfg]
    inp = W.make_inputs(cfg)
    dev = W.device_inputs(inp)
    n = wl.n_tokens
    q16, k16, _, _ = run_prep(problem_for(wl), dev)
    q8, k8, qs, ks = run_prep(problem_for(wl, int8=True), dev)
    for hh in (0, wl.heads - 1):
        for b16, codes, scales in ((q16, q8, qs), (k16, k8, ks)):
            vals = f64(b16[hh])
            c_ref, s_ref = O.quantize_i8(vals[:n].astype(np.float32))
            assert np.array_equal(scales[hh].cpu().numpy(), s_ref), hh
            ch = codes[hh].cpu().numpy()
            assert np.array_equal(ch[:n], c_ref), hh
            assert np.all(ch[n:] == 0), hh


def test_int8_forward_is_deterministic():
    wl = W.ragged_workload(3001, 2)
    inp = W.make_inputs(61, wl)
    dev, _, p8, _, _, q8, k8, qs, ks = _prep_both(wl, inp)
    a = run_forward(p8, q8, k8, dev["v"], qs, ks)
    b = run_forward(p8, q8, k8, dev["v"], qs, ks)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
