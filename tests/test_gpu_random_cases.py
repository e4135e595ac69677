"""Seeded random cases across the boundary's parameters, each against the oracle.

Every case draws a token count (1 .. 5000), a head count, RoPE
section widths (even, summing to 128; some multiples of 16, some not), the
RoPE base, the RMSNorm epsilon, shared or per-head gamma, and one of the
forms: prep + forward in bf16 or int8, or the fused-Q forward in bf16 or int8
(these only with widths that are multiples of 16).  The outputs of sampled
rows (all rows for small N) are compared with the oracle:

* bf16 forms: the oracle's prep and exact attention, at the workload bounds;
* int8 forms: the oracle's attention on the int8 codes of the GPU's own bf16
  prep (the int8 stage, at the stage bounds), as in the fixed-size tests.

A second list of cases runs the E4M3 P·V forward (bf16 or int8 Q'/K' from the
prep, V staged by ``h3attn_prep_v_fp8``) against the oracle's exact softmax
over the dequantised V with its P-rounding bound (``attention_fp8v_rows``), on
the scores of the GPU's own prep output, as in ``test_gpu_fp8v.py``.

The list of cases is drawn once from a fixed seed, so the test is
deterministic; it spreads coverage over combinations the fixed tests leave
out (odd tile tails with generic sections, per-head gamma with int8, ...).
"""
import numpy as np
import pytest
import torch

import oracle as O
from audio_video_diffusion_amd import h3attn as A
from audio_video_diffusion_amd import workloads as W

from gpu_util import MEAN_ABS, SCALE, check, f64, run_forward
from test_gpu_fp8v import check_fp8, v_hat_of

pytestmark = pytest.mark.gpu


def _draw_cases(n_cases=32, seed=0x5EC7):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        # half log-uniform over 1 .. 5000 (short tails), half uniform over 600 .. 5000
        if rng.random() < 0.5:
            n = int(round(np.exp(rng.uniform(0.0, np.log(5000.0)))))
        else:
            n = int(rng.integers(600, 5001))
        h = int(rng.integers(1, 4))
        if rng.random() < 0.5:       # whole 16-element multiples
            cut = np.sort(rng.choice(np.arange(0, 129, 16), size=2))
        else:                        # any even widths
            cut = np.sort(rng.choice(np.arange(0, 129, 2), size=2))
        sections = (int(cut[0]), int(cut[1] - cut[0]), int(128 - cut[1]))
        chunks = all(s % 16 == 0 for s in sections)
        forms = ["bf16", "int8"] + (["fused", "fused_i8"] if chunks else [])
        form = forms[int(rng.integers(0, len(forms)))]
        theta = float(rng.choice([10000.0, 500.0, 1e6]))
        eps = float(rng.choice([1e-6, 1e-5, 0.0]))
        per_head = bool(rng.random() < 0.5)
        cases.append((i, n, h, sections, theta, eps, per_head, form))
    return cases


CASES = _draw_cases()


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def _rows(n, seed):
    if n <= 600:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    rows = set(range(32)) | set(range(n - 64, n)) | set(rng.integers(0, n, size=32).tolist())
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("case", CASES, ids=[f"c{c[0]}-n{c[1]}-h{c[2]}-{c[7]}" for c in CASES])
def test_random_case_matches_oracle(case):
    i, n, h, sections, theta, eps, per_head, form = case
    print(f"    N={n} H={h} sections={sections} theta={theta} eps={eps} per_head={per_head} form={form}",
          flush=True)
    wl = W.ragged_workload(n, h)
    inp = W.make_inputs(600 + i, wl, per_head_gamma=per_head)
    dev = W.device_inputs(inp)
    int8 = form in ("int8", "fused_i8")
    fmt = A.QK_I8_BLK64 if int8 else A.QK_BF16
    p = A.problem(n, h, fmt, sections=sections, theta=theta, eps=eps)
    o = torch.empty_like(dev["v"])
    q_out, k_out, qs, ks = A.alloc_prepped(p)
    if form == "fused":
        A.prep_k(p, dev["k"], dev["gamma_k"], dev["pos"], k_out)
        A.forward_fused_q(p, dev["q"], dev["gamma_q"], dev["pos"], k_out, dev["v"], o, SCALE)
    elif form == "fused_i8":
        A.prep_k_i8(p, dev["k"], dev["gamma_k"], dev["pos"], k_out, ks)
        A.forward_fused_q_i8(p, dev["q"], dev["gamma_q"], dev["pos"], k_out, ks, dev["v"], o, SCALE)
    else:
        A.prep(p, dev["q"], dev["k"], dev["gamma_q"], dev["gamma_k"], dev["pos"], q_out, k_out, qs, ks)
        run_forward(p, q_out, k_out, dev["v"], qs, ks, o=o)
    rows = _rows(n, i)
    got = f64(o)[rows]
    v = O.bf16_bits_to_f64(inp.v)
    if not int8:
        ref = np.stack([
            O.attention_rows_head(
                O.prep_head(inp.q[rows, hh, :], inp.gamma_q, hh, inp.pos[rows], sections, theta, eps),
                O.prep_head(inp.k[:, hh, :], inp.gamma_k, hh, inp.pos, sections, theta, eps),
                v[:, hh, :], SCALE)
            for hh in range(h)], axis=1)
        check(got, ref, what=f"case {i} {form}")
        return
    # int8: the oracle's attention on the codes of the GPU's own bf16 prep
    p16 = A.problem(n, h, A.QK_BF16, sections=sections, theta=theta, eps=eps)
    q16, k16, _, _ = A.alloc_prepped(p16)
    A.prep(p16, dev["q"], dev["k"], dev["gamma_q"], dev["gamma_k"], dev["pos"], q16, k16, None, None)
    qv, kv = f64(q16), f64(k16)
    ref = []
    for hh in range(h):
        cq, sq = O.quantize_i8(qv[hh, :n].astype(np.float32))
        ck, sk = O.quantize_i8(kv[hh, :n].astype(np.float32))
        ref.append(O.attention_i8_rows_head(rows, cq, sq, ck, sk, v[:, hh, :], SCALE))
    check(got, np.stack(ref, axis=1), max_abs=1e-2, mean_abs=MEAN_ABS, rel_l2=6e-3, what=f"case {i} {form} stage")


def _draw_fp8_cases(n_cases=12, seed=0xF8F8):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        n = int(round(np.exp(rng.uniform(0.0, np.log(5000.0))))) if rng.random() < 0.5 else int(rng.integers(600, 5001))
        h = int(rng.integers(1, 4))
        cut = np.sort(rng.choice(np.arange(0, 129, 2), size=2))
        sections = (int(cut[0]), int(cut[1] - cut[0]), int(128 - cut[1]))
        theta = float(rng.choice([10000.0, 500.0, 1e6]))
        eps = float(rng.choice([1e-6, 1e-5, 0.0]))
        cases.append((i, n, h, sections, theta, eps, bool(rng.random() < 0.5), bool(rng.random() < 0.5)))
    return cases


FP8_CASES = _draw_fp8_cases()


@pytest.mark.parametrize("case", FP8_CASES,
                         ids=[f"f{c[0]}-n{c[1]}-h{c[2]}-{'int8' if c[7] else 'bf16'}" for c in FP8_CASES])
def test_random_case_fp8v_matches_oracle(case):
    i, n, h, sections, theta, eps, per_head, int8 = case
    print(f"    N={n} H={h} sections={sections} theta={theta} eps={eps} per_head={per_head} int8={int8}",
          flush=True)
    wl = W.ragged_workload(n, h)
    inp = W.make_inputs(700 + i, wl, per_head_gamma=per_head)
    dev = W.device_inputs(inp)
    p = A.problem(n, h, A.QK_I8_BLK64 if int8 else A.QK_BF16, sections=sections, theta=theta, eps=eps)
    q_out, k_out, qs, ks = A.alloc_prepped(p)
    A.prep(p, dev["q"], dev["k"], dev["gamma_q"], dev["gamma_k"], dev["pos"], q_out, k_out, qs, ks)
    codes, vsc = A.alloc_v_fp8(p)
    A.prep_v_fp8(p, dev["v"], codes, vsc)
    o = torch.empty_like(dev["v"])
    A.forward_fp8v(p, q_out, k_out, codes, vsc, o, SCALE, qs, ks)
    rows = _rows(n, 50 + i)
    got = f64(o)[rows]
    refs, bounds = [], []
    for hh in range(h):
        if int8:
            cq, cs = q_out[hh, :n].cpu().numpy(), qs[hh].cpu().numpy().astype(np.float64)
            ck, ksc = k_out[hh, :n].cpu().numpy(), ks[hh].cpu().numpy().astype(np.float64)
            s = O.scores_i32(cq[rows], ck).astype(np.float64) * cs[rows // 64][:, None] \
                * ksc[np.arange(n) // 64][None, :] * SCALE
        else:
            s = (f64(q_out)[hh, rows] @ f64(k_out)[hh, :n].T) * SCALE
        ref, bound = O.attention_fp8v_rows(s, v_hat_of(inp.v[:, hh, :]))
        refs.append(ref)
        bounds.append(bound)
    check_fp8(got.transpose(1, 0, 2), np.stack(refs), np.stack(bounds), what=f"case {i} fp8v int8={int8}")
