"""The phase-timing build (``libh3attn_timing.so``, include/h3attn_phase_timing.h).

It reads the shader clock at the phase boundaries of every key tile of the
forward; the measurement must not change what is computed.  For every forward
form on ragged sizes: its outputs equal the release build's bit for bit, and
its counters are consistent with the launch (one entry per wave of each
four-wave group, one tile count per key tile of each wave, the four tile
phases adding up to at most the loop time and to most of it).
"""
import math

import pytest
import torch

from audio_video_diffusion_amd import h3attn as A
from audio_video_diffusion_amd import workloads as W

from gpu_util import SCALE, problem_for, run_prep

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def tim():
    return A.variant(A.TIMING_LIB_PATH)


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


def check_counters(c, n, h, rows_per_wg, waves_per_wg):
    wgs = h * math.ceil(n / rows_per_wg)
    ntiles = math.ceil(n / 64)
    groups = waves_per_wg // 4
    for g in range(3):
        v = c[10 * g:10 * g + 10]
        if g >= groups:
            assert v == [0] * 10, g
            continue
        assert v[8] == 4 * wgs, (g, v[8])                  # waves of the group
        assert v[4] == 4 * wgs * ntiles, (g, v[4])         # key tiles they ran
        phases, loop = sum(v[0:4]), v[6]
        assert all(x > 0 for x in v[0:4]) or ntiles == 1, v[0:4]
        assert 0.5 * loop <= phases <= loop, (phases, loop)
        assert v[5] > 0 and v[7] > 0 and v[9] == 0


@pytest.mark.parametrize("n,h", [(65, 2), (1000, 2), (4099, 2)])
def test_timing_build_bit_identical_and_counts(tim, n, h):
    wl = W.ragged_workload(n, h)
    dev = W.device_inputs(W.make_inputs(1300 + n, wl))
    print(f"    N={n} H={h}", flush=True)
    p16, p8 = problem_for(wl), problem_for(wl, int8=True)
    q16, k16, _, _ = run_prep(p16, dev)
    q8, k8, qs, ks = run_prep(p8, dev)
    codes, vsc = A.alloc_v_fp8(p16)
    A.prep_v_fp8(p16, dev["v"], codes, vsc)
    forms = [
        ("bf16", 256, 8, lambda L, o: L.forward(p16, q16, k16, dev["v"], o, SCALE)),
        ("fused", 256, 8, lambda L, o: L.forward_fused_q(p16, dev["q"], dev["gamma_q"], dev["pos"], k16, dev["v"], o, SCALE)),
        ("int8", 384, 12, lambda L, o: L.forward(p8, q8, k8, dev["v"], o, SCALE, qs, ks)),
        ("fused int8", 384, 12, lambda L, o: L.forward_fused_q_i8(p8, dev["q"], dev["gamma_q"], dev["pos"], k8, ks,
                                                                 dev["v"], o, SCALE)),
        ("bf16 + E4M3 V", 256, 8, lambda L, o: L.forward_fp8v(p16, q16, k16, codes, vsc, o, SCALE)),
        ("int8 + E4M3 V", 384, 12, lambda L, o: L.forward_fp8v(p8, q8, k8, codes, vsc, o, SCALE, qs, ks)),
    ]
    for name, rows, waves, call in forms:
        ref = torch.empty_like(dev["v"])
        call(A, ref)
        torch.cuda.synchronize()
        tim.phase_timing_clear()
        got = torch.empty_like(dev["v"])
        call(tim, got)
        torch.cuda.synchronize()
        assert same_bits(got, ref), name
        check_counters(tim.phase_timing_read(), n, h, rows, waves)
