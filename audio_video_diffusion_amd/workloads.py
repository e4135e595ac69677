"""Seeded synthetic workloads for packed joint video+audio+text attention.

This module only *generates inputs*: token counts, integer RoPE positions and
seeded random bf16 tensors.  It holds none of the arithmetic of the method
(no normalisation, rotation, softmax or quantisation), so the CPU oracle's
tests and the GPU path's tests can both draw from it without sharing method
code.

Workload shapes follow the packed-sequence description of the H3 denoiser
("H3 Blackwell Runtime Plan", section Architecture: one packed DiT sequence,
3-axis RoPE) at the resolutions the pages run (864x480/141 frames,
960x544/124 frames, 1344x768/124 and /243 frames: "H3 Runtime Current State",
Implemented And Validated).  The pages do not print token breakdowns; the
video latent grids, audio and text counts below are the stated workload
definitions.

Token order (a reading; the pages are silent): video tokens in (t, h, w)
raster order with w fastest, then audio tokens, then text tokens.
Positions: video token (t, h, w) -> (t, h, w); audio token j -> (j, 0, 0)
(time axis only); text token -> (0, 0, 0).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HEAD_DIM = 128
ROPE_SECTIONS = (32, 48, 48)      # t / h / w widths along the head dimension
ROPE_THETA = 10000.0
RMS_EPS = 1e-6
SEED_ROOT = 0x4833                # first word of every SeedSequence

# tensor ids inside the seed sequence
T_Q, T_K, T_V, T_GAMMA_Q, T_GAMMA_K = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    grid: tuple            # (t, h, w) video latent grid
    audio: int
    text: int
    heads: int
    qk_int8: bool = False
    head_dim: int = HEAD_DIM

    @property
    def video(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def n_tokens(self) -> int:
        return self.video + self.audio + self.text

    @property
    def flops(self) -> float:
        """Dense non-causal attention work, 4 * N^2 * d * H."""
        n = self.n_tokens
        return 4.0 * n * n * self.head_dim * self.heads


WORKLOADS = (
    Workload("tiny_312", (4, 8, 8), 32, 24, 4),
    Workload("864x480_141f", (36, 30, 54), 148, 256, 24),
    Workload("960x544_124f", (32, 34, 60), 130, 256, 24),
    Workload("1344x768_124f", (32, 48, 84), 130, 256, 24),
    Workload("1344x768_243f_int8qk", (61, 48, 84), 254, 256, 24, qk_int8=True),
)
HEADLINE = 3     # index of the 129,410-token 1344x768/124-frame workload

# The pages' own block-24 attention shape: 37,810 packed tokens, 56 heads of
# 128 ("H3 Runtime Current State", Owned Performance Kernels).  The pages give
# only the total; the split below (a 32x24x48 video grid, 690 audio and 256 text
# tokens) is a reading that reproduces it.  Attention cost depends on N and H
# alone; the split only sets the RoPE positions.
BLOCK24 = Workload("block24_37810_h56", (32, 24, 48), 690, 256, 56)

# One GPU's share of the headline workload when its 24 heads are split over
# P = 2, 4, 6, 8 GPUs (heads are independent): same tokens, H / P heads.
SHARDS = tuple(dataclasses.replace(WORKLOADS[HEADLINE], name=f"1344x768_124f_h{24 // p}", heads=24 // p)
               for p in (2, 4, 6, 8))


def positions(grid, audio: int, text: int) -> np.ndarray:
    """Integer (t, h, w) positions, int32 [N, 3], in packed token order."""
    t, h, w = grid
    tt, hh, ww = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
    vid = np.stack([tt.ravel(), hh.ravel(), ww.ravel()], axis=1)
    aud = np.zeros((audio, 3), dtype=np.int64)
    aud[:, 0] = np.arange(audio)
    txt = np.zeros((text, 3), dtype=np.int64)
    return np.ascontiguousarray(np.concatenate([vid, aud, txt]).astype(np.int32))


def _rng(cfg_id: int, tensor_id: int, head: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, cfg_id, tensor_id, head]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even) and return the uint16 bit patterns.

    Uses torch's CPU conversion; it is input generation, not method arithmetic.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_nhd_bits(cfg_id: int, tensor_id: int, n: int, heads: int, d: int = HEAD_DIM,
                    threads: int = 8) -> np.ndarray:
    """Seeded N(0,1) values rounded to bf16, uint16 [N, H, d] (token-major NHD).

    Each head is drawn from its own seed stream, so the value at (n, h, :) does
    not depend on the other heads and can be regenerated alone.
    """
    out = np.empty((n, heads, d), dtype=np.uint16)

    def one(h):
        x = _rng(cfg_id, tensor_id, h).standard_normal((n, d), dtype=np.float32)
        out[:, h, :] = f32_to_bf16_bits(x)

    with ThreadPoolExecutor(max(1, min(threads, heads))) as ex:
        list(ex.map(one, range(heads)))
    return out


def normal_head_bits(cfg_id: int, tensor_id: int, head: int, n: int, d: int = HEAD_DIM) -> np.ndarray:
    """One head of :func:`normal_nhd_bits`, uint16 [N, d]."""
    x = _rng(cfg_id, tensor_id, head).standard_normal((n, d), dtype=np.float32)
    return f32_to_bf16_bits(x)


def gamma_bits(cfg_id: int, tensor_id: int, d: int = HEAD_DIM, heads: int = 0) -> np.ndarray:
    """RMSNorm weight ~ N(1, 0.1) rounded to bf16: uint16 [d], or [H, d] if heads > 0."""
    shape = (heads, d) if heads else (d,)
    x = 1.0 + 0.1 * _rng(cfg_id, tensor_id, 0).standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x.astype(np.float32))


@dataclasses.dataclass
class Inputs:
    """Host-side inputs of one packed-attention problem (bf16 as uint16 bits)."""
    q: np.ndarray            # uint16 [N, H, d]
    k: np.ndarray
    v: np.ndarray
    gamma_q: np.ndarray      # uint16 [d] or [H, d]
    gamma_k: np.ndarray
    pos: np.ndarray          # int32 [N, 3]


def make_inputs(cfg_id: int, wl: Workload | None = None, per_head_gamma: bool = False,
                threads: int = 8) -> Inputs:
    """All inputs of workload ``cfg_id`` (or of a custom ``wl`` seeded as ``cfg_id``)."""
    wl = wl if wl is not None else WORKLOADS[cfg_id]
    n, h, d = wl.n_tokens, wl.heads, wl.head_dim
    gh = h if per_head_gamma else 0
    return Inputs(
        q=normal_nhd_bits(cfg_id, T_Q, n, h, d, threads),
        k=normal_nhd_bits(cfg_id, T_K, n, h, d, threads),
        v=normal_nhd_bits(cfg_id, T_V, n, h, d, threads),
        gamma_q=gamma_bits(cfg_id, T_GAMMA_Q, d, gh),
        gamma_k=gamma_bits(cfg_id, T_GAMMA_K, d, gh),
        pos=positions(wl.grid, wl.audio, wl.text),
    )


def ragged_workload(n: int, heads: int) -> Workload:
    """A custom packed problem of ``n`` tokens: a 1-frame video strip plus audio/text tails.

    Used for tail-length sweeps (n need not be a multiple of any tile size).
    """
    text = min(n, 3)
    audio = min(n - text, 5)
    video = n - text - audio
    return Workload(f"ragged_{n}", (1, 1, video), audio, text, heads)


def bits_to_torch(bits: np.ndarray, device="cuda"):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on ``device`` (same shape)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def torch_to_bits(t) -> np.ndarray:
    """torch.bfloat16 tensor (any device) -> uint16 bit patterns on the host."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def device_inputs(inp: Inputs, device="cuda") -> dict:
    """Upload an :class:`Inputs` to ``device`` as torch tensors."""
    import torch
    return {
        "q": bits_to_torch(inp.q, device), "k": bits_to_torch(inp.k, device),
        "v": bits_to_torch(inp.v, device),
        "gamma_q": bits_to_torch(inp.gamma_q, device), "gamma_k": bits_to_torch(inp.gamma_k, device),
        "pos": torch.from_numpy(inp.pos).to(device),
    }
