"""GPU tests of the Q-prep fusion in the int8 format: h3attn_prep_k_i8 +
h3attn_forward_fused_q_i8.

The int8 fused forward prepares Q' in its prologue with the prep's per-row
routine, rounds it to bf16 and quantises each 64-row block with the prep's
absmax, scale and rounding, so its codes and scales are those h3attn_prep
writes and its output must equal h3attn_prep + h3attn_forward bit for bit:
on ragged sizes (a partial last key tile, partial last quantisation block and
query tile), with per-head gamma, strided input views and a head-major output,
and on the whole 246,462-token workload.  The K-only int8 prep must write the
codes and scales of the full prep bit for bit, pad rows included.  Against the
oracle it is checked as the int8 forward is (the oracle's int8 attention over
the quantisation of the GPU's own bf16 Q'/K').
"""
import numpy as np
import pytest
import torch

from audio_video_diffusion_amd import h3attn as A
from audio_video_diffusion_amd import workloads as W

from gpu_util import MEAN_ABS, SCALE, check, f64, oracle_rows_i8, problem_for, run_forward, run_prep

pytestmark = pytest.mark.gpu

# 384, 385, 769: at and past the edges of the int8 forward's 384-row query tiles
SIZES = [(1, 1, False), (2, 2, True), (63, 1, False), (65, 2, False), (255, 1, True), (257, 3, False),
         (384, 1, False), (385, 2, True), (769, 2, False), (1000, 2, True), (4099, 2, False), (20011, 2, True)]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


def run_prep_k_i8(p, dev):
    _, k_out, _, ks = A.alloc_prepped(p)
    k_out.fill_(0x55)                                # every byte must be written
    ks.fill_(float("nan"))
    A.prep_k_i8(p, dev["k"], dev["gamma_k"], dev["pos"], k_out, ks)
    return k_out, ks


def run_fused_i8(p, dev, k_out, ks, o=None):
    if o is None:
        o = torch.full(dev["v"].shape, 5.0, dtype=torch.bfloat16, device="cuda")
    A.forward_fused_q_i8(p, dev["q"], dev["gamma_q"], dev["pos"], k_out, ks, dev["v"], o, SCALE)
    return o


@pytest.mark.parametrize("n,h,per_head", SIZES)
def test_fused_i8_bit_identical_to_prep_then_forward(n, h, per_head):
    wl = W.ragged_workload(n, h)
    print(f"    N={n} H={h} per_head_gamma={per_head}", flush=True)
    inp = W.make_inputs(700 + n, wl, per_head_gamma=per_head)
    dev = W.device_inputs(inp)
    p8 = problem_for(wl, int8=True)
    q8, k8, qs, ks = run_prep(p8, dev)
    k_only, ks_only = run_prep_k_i8(p8, dev)
    assert torch.equal(k_only, k8)
    nb = (n + 63) // 64
    assert torch.equal(ks_only[:, :nb].view(torch.int32), ks[:, :nb].view(torch.int32))
    ref = run_forward(p8, q8, k8, dev["v"], qs, ks)
    got = run_fused_i8(p8, dev, k_only, ks_only)
    torch.cuda.synchronize()
    assert same_bits(got, ref)


def test_fused_i8_views_and_head_major_output():
    n, h = 3001, 3
    wl = W.ragged_workload(n, h)
    inp = W.make_inputs(771, wl, per_head_gamma=True)
    dev = W.device_inputs(inp)
    # Q, K, V as views into one interleaved [N, 3, H, d] buffer
    qkv = torch.empty((n, 3, h, 128), dtype=torch.bfloat16, device="cuda")
    qkv[:, 0], qkv[:, 1], qkv[:, 2] = dev["q"], dev["k"], dev["v"]
    strided = dict(dev, q=qkv[:, 0], k=qkv[:, 1], v=qkv[:, 2])
    p8 = problem_for(wl, int8=True)
    q8, k8, qs, ks = run_prep(p8, dev)
    ref = run_forward(p8, q8, k8, dev["v"], qs, ks)
    k_only, ks_only = run_prep_k_i8(p8, strided)
    assert torch.equal(k_only, k8)
    obuf = torch.full((h, n, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    got = run_fused_i8(p8, strided, k_only, ks_only, o=obuf.transpose(0, 1))
    torch.cuda.synchronize()
    assert same_bits(got, ref)


def test_fused_i8_matches_oracle():
    n, h = 4099, 2
    wl = W.ragged_workload(n, h)
    inp = W.make_inputs(781, wl)
    dev = W.device_inputs(inp)
    p16, p8 = problem_for(wl), problem_for(wl, int8=True)
    q16, k16, _, _ = run_prep(p16, dev)
    k_only, ks_only = run_prep_k_i8(p8, dev)
    got = f64(run_fused_i8(p8, dev, k_only, ks_only))
    rows = np.arange(n)
    qv, kv = f64(q16), f64(k16)
    ref = np.stack([oracle_rows_i8(inp, hh, rows, q_bf16=qv[hh, :n], k_bf16=kv[hh, :n]) for hh in range(h)], axis=1)
    check(got, ref, max_abs=1e-2, mean_abs=MEAN_ABS, rel_l2=6e-3, what="int8 fused stage")


def test_fused_i8_full_workload_bit_identical():
    cfg = 4
    wl = W.WORKLOADS[cfg]
    print(f"    {wl.name} N={wl.n_tokens} H={wl.heads}", flush=True)
    dev = W.device_inputs(W.make_inputs(cfg, wl, threads=16))
    p8 = problem_for(wl, int8=True)
    q8, k8, qs, ks = run_prep(p8, dev)
    ref = run_forward(p8, q8, k8, dev["v"], qs, ks)
    del q8, qs
    k_only, ks_only = run_prep_k_i8(p8, dev)
    assert torch.equal(k_only, k8)
    got = run_fused_i8(p8, dev, k_only, ks_only)
    torch.cuda.synchronize()
    assert same_bits(got, ref)
