"""GPU tests of the Q-prep fusion: h3attn_prep_k + h3attn_forward_fused_q.

The fused forward computes Q' in its prologue with the prep kernel's own
per-row routine, so its output must equal h3attn_prep + h3attn_forward bit for
bit, and the K-only prep must equal the K' of the full prep bit for bit (pad
rows included).  The plain path is checked against the oracle in the parity
tests; the tiny workload and the 129,410-token workload are also checked
against the oracle here.
"""
import numpy as np
import pytest
import torch

import oracle as O
from audio_video_diffusion_amd import h3attn as A
from audio_video_diffusion_amd import workloads as W

from gpu_util import SCALE, check, f64, oracle_rows_bf16, problem_for, run_forward, run_prep, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def run_prep_k(p, dev):
    _, k_out, _, _ = A.alloc_prepped(p)
    k_out.view(torch.int16).fill_(0x7fc1)           # NaN sentinel: every row must be written
    A.prep_k(p, dev["k"], dev["gamma_k"], dev["pos"], k_out)
    return k_out


def run_fused(p, dev, k_out, o=None):
    if o is None:
        o = torch.full(dev["v"].shape, 5.0, dtype=torch.bfloat16, device="cuda")
    A.forward_fused_q(p, dev["q"], dev["gamma_q"], dev["pos"], k_out, dev["v"], o, SCALE)
    return o


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("n,h,per_head,seed", [
    (1, 1, False, 401), (2, 2, True, 402), (63, 1, False, 403), (64, 2, False, 404), (255, 1, True, 405),
    (256, 3, False, 406), (257, 2, True, 407), (511, 1, False, 408), (1000, 3, True, 409), (4099, 2, False, 410),
])
def test_fused_matches_prep_then_forward_bitwise(n, h, per_head, seed):
    wl = W.ragged_workload(n, h)
    print(f"    N={n} H={h} per_head_gamma={per_head}", flush=True)
    dev = W.device_inputs(W.make_inputs(seed, wl, per_head_gamma=per_head))
    p = problem_for(wl)
    q_out, k_full, _, _ = run_prep(p, dev)
    k_only = run_prep_k(p, dev)
    assert same_bits(k_only, k_full)
    plain = run_forward(p, q_out, k_full, dev["v"])
    fused = run_fused(p, dev, k_only)
    assert same_bits(fused, plain)


@pytest.mark.parametrize("sections,theta,eps", [((64, 32, 32), 500.0, 1e-5), ((16, 16, 96), 1e6, 0.0)])
def test_fused_other_rope_sections_and_constants(sections, theta, eps):
    wl = W.ragged_workload(1500, 2)
    dev = W.device_inputs(W.make_inputs(411, wl, per_head_gamma=True))
    p = A.problem(wl.n_tokens, wl.heads, sections=sections, theta=theta, eps=eps)
    q_out, k_full, _, _ = run_prep(p, dev)
    k_only = run_prep_k(p, dev)
    assert same_bits(k_only, k_full)
    assert same_bits(run_fused(p, dev, k_only), run_forward(p, q_out, k_full, dev["v"]))


def test_fused_tiny_workload_against_oracle():
    wl = W.WORKLOADS[0]
    inp = W.make_inputs(0)
    dev = W.device_inputs(inp)
    p = problem_for(wl)
    o = run_fused(p, dev, run_prep_k(p, dev))
    qp = O.prep(inp.q, inp.gamma_q, inp.pos, W.ROPE_SECTIONS, W.ROPE_THETA, W.RMS_EPS)
    kp = O.prep(inp.k, inp.gamma_k, inp.pos, W.ROPE_SECTIONS, W.ROPE_THETA, W.RMS_EPS)
    check(f64(o), O.attention(qp, kp, O.bf16_bits_to_f64(inp.v), SCALE), what="fused tiny")


def test_fused_on_interleaved_views_and_strided_output():
    # raw Q, K, V as views of one interleaved projection output [N, 3, H, d];
    # O into every other 128-wide slot of [N, H, 2, d]
    wl = W.ragged_workload(777, 3)
    inp = W.make_inputs(412, wl, per_head_gamma=True)
    n, h = wl.n_tokens, wl.heads
    qkv = torch.empty((n, 3, h, 128), dtype=torch.bfloat16, device="cuda")
    for i, bits in enumerate((inp.q, inp.k, inp.v)):
        qkv[:, i] = W.bits_to_torch(bits)
    dev = W.device_inputs(inp)
    dev["q"], dev["k"], dev["v"] = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    p = problem_for(wl)
    q_out, k_full, _, _ = run_prep(p, dev)
    plain = run_forward(p, q_out, k_full, dev["v"])
    obuf = torch.full((n, h, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    run_fused(p, dev, run_prep_k(p, dev), o=obuf[:, :, 0])
    assert torch.all(obuf[:, :, 1] == 7.0)
    assert same_bits(obuf[:, :, 0].contiguous(), plain)


def test_fused_repeated_calls_are_deterministic():
    wl = W.ragged_workload(3001, 2)
    dev = W.device_inputs(W.make_inputs(413, wl))
    p = problem_for(wl)
    k_only = run_prep_k(p, dev)
    first = run_fused(p, dev, k_only)
    for _ in range(3):
        assert same_bits(run_fused(p, dev, k_only), first)


def test_fused_full_workload_bitwise_and_sampled_rows():
    cfg = W.HEADLINE
    wl = W.WORKLOADS[cfg]
    print(f"    {wl.name} N={wl.n_tokens} H={wl.heads}", flush=True)
    inp = W.make_inputs(cfg)
    dev = W.device_inputs(inp)
    p = problem_for(wl)
    q_out, k_full, _, _ = run_prep(p, dev)
    plain = run_forward(p, q_out, k_full, dev["v"])
    del q_out
    k_only = run_prep_k(p, dev)
    assert same_bits(k_only, k_full)
    del k_full
    fused = run_fused(p, dev, k_only)
    assert same_bits(fused, plain)
    rows = sample_rows(wl, n_random=32)
    got = f64(fused[torch.from_numpy(rows).cuda()])
    for hh in (0, wl.heads - 1):
        check(got[:, hh, :], oracle_rows_bf16(inp, hh, rows), what=f"fused {wl.name} head {hh}")
    assert np.isfinite(got).all()


def test_fused_output_into_head_major_view():
    wl = W.ragged_workload(1500, 3)
    dev = W.device_inputs(W.make_inputs(414, wl))
    n, h = wl.n_tokens, wl.heads
    p = problem_for(wl)
    q_out, k_full, _, _ = run_prep(p, dev)
    plain = run_forward(p, q_out, k_full, dev["v"])
    hnd = torch.full((h, n, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    run_fused(p, dev, run_prep_k(p, dev), o=hnd.permute(1, 0, 2))
    assert same_bits(hnd.permute(1, 0, 2).contiguous(), plain)


def test_fused_block24_shape_bitwise():
    # the pages' block-24 attention shape: 37,810 tokens, 56 heads
    wl = W.BLOCK24
    print(f"    {wl.name} N={wl.n_tokens} H={wl.heads}", flush=True)
    dev = W.device_inputs(W.make_inputs(100, wl))
    p = problem_for(wl)
    q_out, k_full, _, _ = run_prep(p, dev)
    plain = run_forward(p, q_out, k_full, dev["v"])
    del q_out
    k_only = run_prep_k(p, dev)
    assert same_bits(k_only, k_full)
    assert same_bits(run_fused(p, dev, k_only), plain)
