"""GPU tests of the calling conventions: output views, streams, concurrency,
and the calibration entry point.  Results are compared bit for bit with the
same calls made the plain way (the plain way is checked against the oracle in
the parity tests); the HND-output case is also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from audio_video_diffusion_amd import h3attn as A
from audio_video_diffusion_amd import workloads as W

from gpu_util import SCALE, check, f64, problem_for, run_forward, run_prep

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def _case(n=1500, h=3, seed=301):
    wl = W.ragged_workload(n, h)
    inp = W.make_inputs(seed, wl)
    dev = W.device_inputs(inp)
    p = problem_for(wl)
    q_out, k_out, _, _ = run_prep(p, dev)
    return wl, inp, dev, p, q_out, k_out


def test_output_into_head_major_view():
    wl, inp, dev, p, q_out, k_out = _case()
    n, h = wl.n_tokens, wl.heads
    plain = run_forward(p, q_out, k_out, dev["v"])
    hnd = torch.full((h, n, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    A.forward(p, q_out, k_out, dev["v"], hnd.permute(1, 0, 2), SCALE)
    assert torch.equal(hnd.permute(1, 0, 2).view(torch.int16), plain.view(torch.int16))
    qp = O.prep(inp.q, inp.gamma_q, inp.pos, W.ROPE_SECTIONS, W.ROPE_THETA, W.RMS_EPS)
    kp = O.prep(inp.k, inp.gamma_k, inp.pos, W.ROPE_SECTIONS, W.ROPE_THETA, W.RMS_EPS)
    check(f64(hnd.permute(1, 0, 2)), O.attention(qp, kp, O.bf16_bits_to_f64(inp.v), SCALE), what="HND output")


def test_calls_on_a_side_stream_match_the_default_stream():
    wl, inp, dev, p, q_out, k_out = _case(seed=302)
    plain = run_forward(p, q_out, k_out, dev["v"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q2, k2, _, _ = A.alloc_prepped(p)
        A.prep(p, dev["q"], dev["k"], dev["gamma_q"], dev["gamma_k"], dev["pos"], q2, k2, stream=side)
        o2 = torch.empty_like(dev["v"])
        A.forward(p, q2, k2, dev["v"], o2, SCALE, stream=side)
    side.synchronize()
    assert torch.equal(q2.view(torch.int16), q_out.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), plain.view(torch.int16))


def test_concurrent_forwards_on_two_streams():
    # two independent problems at once; each must equal its own sequential result
    cases = [_case(n=3001, h=2, seed=303), _case(n=777, h=4, seed=304)]
    seq = [run_forward(c[3], c[4], c[5], c[2]["v"]) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for (wl, inp, dev, p, q_out, k_out), s in zip(cases, streams):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            o = torch.empty_like(dev["v"])
            for _ in range(3):
                A.forward(p, q_out, k_out, dev["v"], o, SCALE, stream=s)
            outs.append(o)
    for s in streams:
        s.synchronize()
    for a, b in zip(outs, seq):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_calibration_kernel_runs_and_is_deterministic():
    out = torch.full((64 * 512,), float("nan"), dtype=torch.float32, device="cuda")
    flops = A.calibrate_mfma_bf16(64, 10, out)
    assert flops == 64 * 8 * 10 * 16 * 32768.0
    first = out.clone()
    A.calibrate_mfma_bf16(64, 10, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.equal(first, out)
    with pytest.raises(ValueError):
        A.calibrate_mfma_bf16(65, 10, out)            # out too small for 65 * 512 floats
