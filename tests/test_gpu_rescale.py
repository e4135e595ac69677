"""GPU tests of the running-max logic on crafted logits (every forward form).

All Q', K' values are exactly +-1: raw Q and K are +-1 vectors, gamma = 1,
eps = 0 and every position 0, so RMSNorm and RoPE return them unchanged, and
the int8 quantiser maps them to +-127 with scale 1/127 exactly.  With
softmax_scale = 2^-3 / log2(e) a key with p entries equal to its query's has the
base-2 logit (2p - 128) / 8: any multiple of 1/4 in [-16, 16], exactly.  The
key tiles (64 keys each) are laid out so that the forward passes through
every branch of its per-tile decision:
  tile 0        mixed 0 and -1.5 (sets the running max m = 0)
  tile 1        all +3: row sums above the bound, no raise (P kept)
  tile 2        half +5, half -10: row sums above the bound, no raise
  tile 3        one key +9, the rest 0: raise by 9
  tile 4        all +12: above the bound, no raise (3 above m)
  tile 5        all +16: above the bound, 7 above m: no raise
  tile 6        all -16: tiny P
  tiles 7..     seeded random logits in [-16, 16]; the last tile ragged
Half of the query rows are the negated pattern, which reverses the staircase
(their raises fall on tile 6 and the random tiles).  The oracle result is the
exact attention of the same inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from audio_video_diffusion_amd import h3attn as A
from audio_video_diffusion_amd import workloads as W

from gpu_util import MAX_ABS, MEAN_ABS, REL_L2, REL_L2_I8, errors, f64

pytestmark = pytest.mark.gpu

SCALE_EXACT = 0.125 / math.log2(math.e)
N, H = 1000, 2
SECTIONS = (32, 48, 48)


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def key_logits(rng):
    """Base-2 logit of each key for a query of all ones (multiples of 1/4)."""
    lg = np.empty(N)
    t = lambda i: slice(64 * i, 64 * i + 64)
    lg[t(0)] = np.where(np.arange(64) % 3 == 0, -1.5, 0.0)
    lg[t(1)] = 3.0
    lg[t(2)] = np.where(np.arange(64) % 2 == 0, 5.0, -10.0)
    lg[t(3)] = 0.0
    lg[64 * 3 + 37] = 9.0
    lg[t(4)] = 12.0
    lg[t(5)] = 16.0
    lg[t(6)] = -16.0
    lg[64 * 7:] = rng.integers(0, 129, size=N - 64 * 7) / 4.0 - 16.0
    return lg


def make_case(seed):
    """bf16 bit patterns of raw Q, K, V [N, H, 128], gamma = 1, positions 0."""
    rng = np.random.default_rng(seed)
    q = np.ones((N, H, 128), dtype=np.float32)
    q[1::2] = -1.0                                  # odd rows: the negated query
    k = np.empty((N, H, 128), dtype=np.float32)
    for h in range(H):
        lg = key_logits(rng)
        for n in range(N):
            p = int(round(lg[n] * 4 + 64))          # entries equal to the all-ones query
            row = -np.ones(128, dtype=np.float32)
            row[rng.permutation(128)[:p]] = 1.0
            k[n, h] = row
    v = rng.standard_normal((N, H, 128)).astype(np.float32)
    inp = W.Inputs(q=O.f32_to_bf16_bits(q), k=O.f32_to_bf16_bits(k), v=O.f32_to_bf16_bits(v),
                   gamma_q=O.f32_to_bf16_bits(np.ones(128, np.float32)),
                   gamma_k=O.f32_to_bf16_bits(np.ones(128, np.float32)),
                   pos=np.zeros((N, 3), dtype=np.int32))
    return inp


def oracle(inp):
    qp = O.prep(inp.q, inp.gamma_q, inp.pos, SECTIONS, 1e4, 0.0)
    kp = O.prep(inp.k, inp.gamma_k, inp.pos, SECTIONS, 1e4, 0.0)
    # the crafted values pass RMSNorm and RoPE unchanged
    assert np.array_equal(np.abs(qp), np.ones_like(qp)) and np.array_equal(np.abs(kp), np.ones_like(kp))
    return O.attention(qp, kp, O.bf16_bits_to_f64(inp.v), SCALE_EXACT)


def test_crafted_logits_are_what_the_staircase_says():
    inp = make_case(501)
    qp = O.bf16_bits_to_f64(inp.q)
    kp = O.bf16_bits_to_f64(inp.k)
    lg = np.einsum("nd,nd->n", np.broadcast_to(qp[0, 0], kp[:, 0].shape), kp[:, 0]) / 8.0
    assert lg[64] == 3.0 and lg[64 * 3 + 37] == 9.0 and lg[64 * 5] == 16.0 and lg[64 * 6] == -16.0
    assert np.all(lg * 4 == np.round(lg * 4)) and lg.min() >= -16 and lg.max() <= 16


@pytest.mark.parametrize("form", ["bf16", "fused_q", "fp8v", "int8", "int8_ksmooth_fp8v"])
def test_running_max_branches_against_oracle(form):
    inp = make_case(500)
    dev = W.device_inputs(inp)
    int8 = form.startswith("int8")
    p = A.problem(N, H, A.QK_I8_BLK64 if int8 else A.QK_BF16, sections=SECTIONS, eps=0.0)
    q_out, k_out, qs, ks = A.alloc_prepped(p)
    o = torch.full((N, H, 128), 9.0, dtype=torch.bfloat16, device="cuda")
    if form == "fused_q":
        A.prep_k(p, dev["k"], dev["gamma_k"], dev["pos"], k_out)
        A.forward_fused_q(p, dev["q"], dev["gamma_q"], dev["pos"], k_out, dev["v"], o, SCALE_EXACT)
    elif form == "int8_ksmooth_fp8v":
        km = torch.empty((H, 128), dtype=torch.float32, device="cuda")
        A.prep_ksmooth(p, dev["q"], dev["k"], dev["gamma_q"], dev["gamma_k"], dev["pos"], q_out, k_out, qs, ks, km)
    else:
        A.prep(p, dev["q"], dev["k"], dev["gamma_q"], dev["gamma_k"], dev["pos"], q_out, k_out, qs, ks)
    if form in ("fp8v", "int8_ksmooth_fp8v"):
        codes, vsc = A.alloc_v_fp8(p)
        A.prep_v_fp8(p, dev["v"], codes, vsc)
        A.forward_fp8v(p, q_out, k_out, codes, vsc, o, SCALE_EXACT, qs, ks)
    elif form in ("bf16", "int8"):
        A.forward(p, q_out, k_out, dev["v"], o, SCALE_EXACT, qs, ks)
    torch.cuda.synchronize()
    got = f64(o)
    mx, mn, rel = errors(got, oracle(inp))
    print(f"    {form}: max_abs={mx:.3e} mean_abs={mn:.3e} rel_l2={rel:.3e}", flush=True)
    assert np.isfinite(got).all()
    if "fp8v" in form:
        # E4M3 P and V: about 3% rms relative error against exact attention
        assert rel <= 8e-2, rel
    else:
        # P rounded to bf16 is the only rounding left (int8: the +-1 codes are exact)
        assert mx <= MAX_ABS and mn <= MEAN_ABS and rel <= (REL_L2_I8 if int8 else REL_L2), (mx, mn, rel)
