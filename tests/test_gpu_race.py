"""Race detection for the forward's hand-managed LDS protocol.

ROCm has no LDS race checker, so the library is also built with a wait for
all memory traffic and a work-group barrier after every LDS stage of the
forward's tile loop (the K'/V buffer -> LDS fill, the K' operand reads, the V
operand reads): ``libh3attn_sync.so``.  No stage can overlap another there.
Its outputs must equal the release build's bit for bit, for every forward
form (the fused-Q forms included) and the int32 scores hook, on ragged sizes whose last key tile is
partial, and on a size large enough that every LDS stage is reused many times.
"""
import numpy as np
import pytest
import torch

from audio_video_diffusion_amd import h3attn as A
from audio_video_diffusion_amd import workloads as W

from gpu_util import SCALE, problem_for, run_prep

pytestmark = pytest.mark.gpu

SIZES = [(1, 1), (65, 2), (257, 3), (1000, 2), (4099, 2), (20011, 2)]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def dbg():
    return A.variant(A.SYNC_LIB_PATH)


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


def _inputs(n, h, seed):
    wl = W.ragged_workload(n, h)
    inp = W.make_inputs(seed, wl)
    return wl, W.device_inputs(inp)


@pytest.mark.parametrize("n,h", SIZES)
def test_sync_build_bit_identical_bf16_and_fused(dbg, n, h):
    wl, dev = _inputs(n, h, 900 + n)
    print(f"    N={n} H={h}", flush=True)
    p = problem_for(wl)
    q16, k16, _, _ = run_prep(p, dev)
    for lib in (A, dbg):
        o = torch.empty_like(dev["v"])
        lib.forward(p, q16, k16, dev["v"], o, SCALE)
        of = torch.empty_like(dev["v"])
        lib.forward_fused_q(p, dev["q"], dev["gamma_q"], dev["pos"], k16, dev["v"], of, SCALE)
        if lib is A:
            ref, ref_f = o, of
    torch.cuda.synchronize()
    assert same_bits(o, ref)
    assert same_bits(of, ref_f)


@pytest.mark.parametrize("n,h", SIZES)
def test_sync_build_bit_identical_int8_and_fp8v(dbg, n, h):
    wl, dev = _inputs(n, h, 950 + n)
    print(f"    N={n} H={h}", flush=True)
    p16 = problem_for(wl)
    p8 = problem_for(wl, int8=True)
    q16, k16, _, _ = run_prep(p16, dev)
    q8, k8, qs, ks = run_prep(p8, dev)
    codes, vsc = A.alloc_v_fp8(p16)
    A.prep_v_fp8(p16, dev["v"], codes, vsc)
    outs = []
    for lib in (A, dbg):
        o8 = torch.empty_like(dev["v"])
        lib.forward(p8, q8, k8, dev["v"], o8, SCALE, qs, ks)
        o16v = torch.empty_like(dev["v"])
        lib.forward_fp8v(p16, q16, k16, codes, vsc, o16v, SCALE)
        o8v = torch.empty_like(dev["v"])
        lib.forward_fp8v(p8, q8, k8, codes, vsc, o8v, SCALE, qs, ks)
        outs.append((o8, o16v, o8v))
    torch.cuda.synchronize()
    for a, b, what in zip(outs[0], outs[1], ("int8 Q/K", "bf16 Q/K + E4M3 V", "int8 Q/K + E4M3 V")):
        assert same_bits(a, b), what


@pytest.mark.parametrize("n,h", SIZES)
def test_sync_build_bit_identical_int8_fused_q(dbg, n, h):
    wl, dev = _inputs(n, h, 970 + n)
    print(f"    N={n} H={h}", flush=True)
    p8 = problem_for(wl, int8=True)
    _, k8, _, ks = A.alloc_prepped(p8)
    A.prep_k_i8(p8, dev["k"], dev["gamma_k"], dev["pos"], k8, ks)
    outs = []
    for lib in (A, dbg):
        o = torch.empty_like(dev["v"])
        lib.forward_fused_q_i8(p8, dev["q"], dev["gamma_q"], dev["pos"], k8, ks, dev["v"], o, SCALE)
        outs.append(o)
    torch.cuda.synchronize()
    assert same_bits(outs[0], outs[1])


@pytest.mark.parametrize("n,h", [(4099, 2), (20011, 1)])
def test_sync_build_bit_identical_scores_hook(dbg, n, h):
    wl, dev = _inputs(n, h, 990 + n)
    p8 = problem_for(wl, int8=True)
    q8, k8, _, _ = run_prep(p8, dev)
    for lay in (0, 1):
        r0, nr, c0, nc = n // 4, 700, n // 3, 1500
        a = torch.empty((nr, nc), dtype=torch.int32, device="cuda")
        b = torch.empty_like(a)
        A.debug_scores_i32(p8, q8, k8, h - 1, r0, nr, c0, nc, a, fp8v_layout=lay)
        dbg.debug_scores_i32(p8, q8, k8, h - 1, r0, nr, c0, nc, b, fp8v_layout=lay)
        torch.cuda.synchronize()
        assert np.array_equal(a.cpu().numpy(), b.cpu().numpy()), lay
