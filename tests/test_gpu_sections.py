"""GPU parity of the prep with RoPE section widths that are even but not
multiples of 16 (the prep form that pairs elements through LDS).

Split-half RoPE pairs element j of a section's first half with element j of
its second half, for any even width ("H3 Blackwell Runtime Plan",
Architecture: 3-axis RoPE).  With widths that are multiples of 16 each lane's
8-element chunk pairs with one whole chunk; otherwise the prep gathers each
lane's first-half elements and partners from the row through LDS.  Checked
here, on ragged sizes with per-head gamma:

* the bf16 Q'/K' against the oracle's RMSNorm + RoPE with the same sections,
  element by element, within bf16 rounding of an fp32 evaluation, pad rows 0;
* the K-only prep writes the same K' bits as the prep;
* the int8 codes and scales, and with K smoothing the means, codes and scales,
  bit for bit against the oracle's quantiser (and smoothing) applied to the
  GPU's own bf16 prep output, as for the chunk form;
* prep + forward end to end against the oracle's attention.
"""
import numpy as np
import pytest
import torch

import oracle as O
from audio_video_diffusion_amd import h3attn as A
from audio_video_diffusion_amd import workloads as W

from gpu_util import SCALE, check, f64, run_forward

pytestmark = pytest.mark.gpu

# (sections, theta, eps): halves that end inside a chunk (20, 17, 23, 1, 31 ...),
# an empty section, and one whose first half is a single element
CASES = [((40, 40, 48), 10000.0, 1e-6), ((34, 46, 48), 10000.0, 1e-6), ((2, 62, 64), 500.0, 1e-5),
         ((0, 62, 66), 1e6, 0.0), ((46, 36, 46), 10000.0, 1e-6)]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def _problem(wl, sections, theta, eps, int8=False):
    return A.problem(wl.n_tokens, wl.heads, A.QK_I8_BLK64 if int8 else A.QK_BF16, sections=sections,
                     theta=theta, eps=eps)


def _prep(p, dev):
    q_out, k_out, qs, ks = A.alloc_prepped(p)
    A.prep(p, dev["q"], dev["k"], dev["gamma_q"], dev["gamma_k"], dev["pos"], q_out, k_out, qs, ks)
    return q_out, k_out, qs, ks


@pytest.mark.parametrize("sections,theta,eps", CASES)
@pytest.mark.parametrize("n,h", [(1000, 3), (65, 2)])
def test_prep_bf16_generic_sections_match_oracle(sections, theta, eps, n, h):
    wl = W.ragged_workload(n, h)
    inp = W.make_inputs(300 + n + sections[0], wl, per_head_gamma=True)
    p = _problem(wl, sections, theta, eps)
    print(f"    N={n} H={h} sections={sections}", flush=True)
    dev = W.device_inputs(inp)
    q_out, k_out, _, _ = _prep(p, dev)
    for got_t, x, g in ((q_out, inp.q, inp.gamma_q), (k_out, inp.k, inp.gamma_k)):
        ref = O.prep(x, g, inp.pos, sections, theta, eps)
        got_all = f64(got_t)
        got = got_all[:, :n, :].transpose(1, 0, 2)
        # bf16 rounding of an fp32 evaluation (as for the chunk form)
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * (1 + 2.0 ** -6) * np.abs(ref) + 4e-6
        assert np.all(err <= bound), (np.max(err - bound), np.max(err))
        assert np.all(got_all[:, n:, :] == 0)
    # the K-only prep: the same K' bits
    k_only = torch.empty_like(k_out)
    A.prep_k(p, dev["k"], dev["gamma_k"], dev["pos"], k_only)
    assert torch.equal(k_only, k_out)


@pytest.mark.parametrize("sections,theta,eps", CASES[:3])
def test_int8_and_ksmooth_generic_sections_bit_exact(sections, theta, eps):
    n, h = 1000, 3
    wl = W.ragged_workload(n, h)
    inp = W.make_inputs(400 + sections[0], wl, per_head_gamma=True)
    dev = W.device_inputs(inp)
    q16, k16, _, _ = _prep(_problem(wl, sections, theta, eps), dev)
    p8 = _problem(wl, sections, theta, eps, int8=True)
    q8, k8, qs, ks = _prep(p8, dev)
    qv, kv = f64(q16), f64(k16)
    codes = {"q": q8.cpu().numpy(), "k": k8.cpu().numpy()}
    scales = {"q": qs.cpu().numpy(), "k": ks.cpu().numpy()}
    for hh in range(h):
        for name, vals in (("q", qv), ("k", kv)):
            c_ref, s_ref = O.quantize_i8(vals[hh, :n].astype(np.float32))
            assert np.array_equal(scales[name][hh], s_ref), (name, hh)
            assert np.array_equal(codes[name][hh, :n], c_ref), (name, hh)
            assert np.all(codes[name][hh, n:] == 0)
    # K smoothing: means, codes and scales of the smoothed K'; Q' as the plain prep
    qk, kk, qsk, ksk = A.alloc_prepped(p8)
    mean = torch.empty((h, 128), dtype=torch.float32, device="cuda")
    A.prep_ksmooth(p8, dev["q"], dev["k"], dev["gamma_q"], dev["gamma_k"], dev["pos"], qk, kk, qsk, ksk, mean)
    assert torch.equal(qk, q8) and torch.equal(qsk, qs)
    kc, kscl, mu_g = kk.cpu().numpy(), ksk.cpu().numpy(), mean.cpu().numpy()
    for hh in range(h):
        mu, xs = O.smooth_k(kv[hh, :n].astype(np.float32))
        c_ref, s_ref = O.quantize_i8(xs)
        assert np.array_equal(mu_g[hh], mu), hh
        assert np.array_equal(kscl[hh], s_ref), hh
        assert np.array_equal(kc[hh, :n], c_ref), hh


@pytest.mark.parametrize("sections,theta,eps", CASES[:2])
def test_forward_generic_sections_end_to_end(sections, theta, eps):
    n, h = 1000, 3
    wl = W.ragged_workload(n, h)
    inp = W.make_inputs(500 + sections[0], wl, per_head_gamma=True)
    dev = W.device_inputs(inp)
    p = _problem(wl, sections, theta, eps)
    q_out, k_out, _, _ = _prep(p, dev)
    got = f64(run_forward(p, q_out, k_out, dev["v"]))
    qp = O.prep(inp.q, inp.gamma_q, inp.pos, sections, theta, eps)
    kp = O.prep(inp.k, inp.gamma_k, inp.pos, sections, theta, eps)
    check(got, O.attention(qp, kp, O.bf16_bits_to_f64(inp.v), SCALE), what=f"e2e sections={sections}")
