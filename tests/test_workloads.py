"""Workload definitions and the seeded input generator (no method arithmetic)."""
import os

import numpy as np

from audio_video_diffusion_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workload_sizes.txt")


def _golden():
    rows, extra = [], {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("@"):
            name, *kv = line[1:].split()
            extra[name] = {k: int(v) for k, v in (x.split("=") for x in kv)}
            continue
        name, t, h, w, a, tx, hd, n = line.split()
        rows.append((name, (int(t), int(h), int(w)), int(a), int(tx), int(hd), int(n)))
    return rows, extra


def test_workloads_match_golden_sizes():
    rows, extra = _golden()
    assert len(rows) == len(W.WORKLOADS)
    for wl, (name, grid, a, tx, hd, n) in zip(W.WORKLOADS, rows):
        assert (wl.name, wl.grid, wl.audio, wl.text, wl.heads, wl.n_tokens) == (name, grid, a, tx, hd, n)
    assert W.WORKLOADS[W.HEADLINE].n_tokens == 129410
    assert W.WORKLOADS[4].qk_int8 and not any(w.qk_int8 for w in W.WORKLOADS[:4])
    v = extra["v_bf16_mib"]
    mib = v["tokens"] * v["heads"] * W.HEAD_DIM * 2 / 2 ** 20
    assert abs(mib - v["approx_mib"]) < 1.0


def test_positions_layout():
    pos = W.positions((2, 3, 4), 5, 6)
    assert pos.shape == (24 + 5 + 6, 3) and pos.dtype == np.int32
    # video raster order with w fastest
    assert pos[0].tolist() == [0, 0, 0] and pos[1].tolist() == [0, 0, 1]
    assert pos[4].tolist() == [0, 1, 0] and pos[12].tolist() == [1, 0, 0]
    assert pos[23].tolist() == [1, 2, 3]
    # audio on the time axis only, text at the origin
    assert pos[24:29].tolist() == [[j, 0, 0] for j in range(5)]
    assert np.all(pos[29:] == 0)


def test_generator_is_seeded_per_head():
    a = W.normal_nhd_bits(0, W.T_Q, 100, 3)
    b = W.normal_nhd_bits(0, W.T_Q, 100, 3, threads=1)
    assert np.array_equal(a, b)
    assert np.array_equal(a[:, 1, :], W.normal_head_bits(0, W.T_Q, 1, 100))
    assert not np.array_equal(a, W.normal_nhd_bits(0, W.T_K, 100, 3))
    x = a.astype(np.uint32) << 16
    f = x.view(np.float32)
    assert abs(float(f.mean())) < 0.05 and abs(float(f.std()) - 1) < 0.05
    g = W.gamma_bits(0, W.T_GAMMA_Q)
    gf = (g.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(gf.mean()) - 1) < 0.05 and 0.05 < float(gf.std()) < 0.15
    assert W.gamma_bits(0, W.T_GAMMA_Q, heads=4).shape == (4, 128)


def test_ragged_workload_counts():
    for n in (1, 2, 7, 8, 63, 64, 65, 257, 4099):
        wl = W.ragged_workload(n, 2)
        assert wl.n_tokens == n
        assert W.positions(wl.grid, wl.audio, wl.text).shape == (n, 3)


def test_block24_and_shard_shapes():
    # the block-24 shape is the pages' canonical 37,810-token, 56-head block
    # (the same figures that fix the 517 MiB V tensor above)
    v = _golden()[1]["v_bf16_mib"]
    assert (W.BLOCK24.n_tokens, W.BLOCK24.heads) == (v["tokens"], v["heads"])
    # head shards keep every token and divide the 24 heads evenly
    head = W.WORKLOADS[W.HEADLINE]
    assert [s.heads for s in W.SHARDS] == [12, 6, 4, 3]
    assert all(s.n_tokens == head.n_tokens and s.grid == head.grid for s in W.SHARDS)
