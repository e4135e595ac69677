"""CPU tests of the C ABI: the library loads, exports what the header declares,
and rejects bad arguments on the host before anything reaches the GPU.

Pointers passed here are fake addresses: every call below is rejected by the
host-side checks, so nothing is dereferenced and no HIP call is made.
"""
import ctypes
import os
import re
import subprocess

import pytest

from audio_video_diffusion_amd import h3attn as A

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
HEADER = os.path.join(INCLUDE, "h3attn.h")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))

F = 0x7f0000000000          # fake, 16-byte aligned "device" addresses, far apart
G = 0x7f1000000000
H = 0x7f2000000000
I = 0x7f3000000000
J = 0x7f4000000000
K = 0x7f5000000000


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(h3attn_\w+)\s*\(", text))
    return sorted(names)


@pytest.mark.parametrize("path", [A.LIB_PATH, A.SYNC_LIB_PATH, A.TIMING_LIB_PATH],
                         ids=["release", "race-detection", "phase-timing"])
def test_library_exports_every_declared_symbol(path):
    names = declared_functions()
    assert {"h3attn_prep", "h3attn_forward", "h3attn_debug_scores_i32", "h3attn_phase_timing_read"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (h3attn_\w+)", out))
    lib = A.lib if path == A.LIB_PATH else A.variant(path).lib
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert lib.h3attn_abi_version() == A.ABI_VERSION


def test_abi_version_and_status_strings():
    assert A.lib.h3attn_abi_version() == A.ABI_VERSION == 8
    for s in (0, -1, -2, -3, -4, -5, -6, 7):
        assert A.lib.h3attn_status_string(s)


def test_sizes():
    p = A.problem(129410, 24)
    assert A.padded_tokens(p) == 129536
    assert A.prepped_qk_bytes(p) == 24 * 129536 * 128 * 2
    assert A.scales_bytes(p) == 0
    p8 = A.problem(246462, 24, A.QK_I8_BLK64)
    assert A.prepped_qk_bytes(p8) == 24 * 246528 * 128
    assert A.scales_bytes(p8) == 24 * 3851 * 4
    assert A.padded_tokens(A.problem(1, 1)) == 256
    assert A.padded_tokens(A.problem(0, 1)) == 0
    assert A.prepped_qk_bytes(A.problem(10, 1, head_dim=64)) == 0
    assert A.prepped_v_bytes(p) == 24 * 129536 * 128
    assert A.v_scales_bytes(p) == 24 * 128 * 4
    assert A.prepped_v_bytes(p8) == 24 * 246528 * 128
    assert A.prepped_v_bytes(A.problem(10, 1, head_dim=64)) == 0


def prep(p, q=F, qst=384, qsh=128, k=G, kst=384, ksh=128, gq=H, gk=H + 256, gsh=0, pos=I,
         qo=J, ko=J + (1 << 32), qs=None, ks=None):
    return A.lib.h3attn_prep(ctypes.byref(p), q, qst, qsh, k, kst, ksh, gq, gk, gsh, pos,
                             qo, ko, qs, ks, None)


def fwd(p, q=F, k=G, qs=None, ks=None, v=H, vst=384, vsh=128, o=I, ost=384, osh=128, scale=0.088):
    return A.lib.h3attn_forward(ctypes.byref(p), q, k, qs, ks, v, vst, vsh, o, ost, osh, scale, None)


@pytest.mark.parametrize("kw,field,val,code", [
    ({}, "head_dim", 64, -3),
    ({}, "qk_format", 5, -3),
    ({}, "n_tokens", 0, -2),
    ({}, "n_heads", 0, -2),
])
def test_problem_validation(kw, field, val, code):
    p = A.problem(1000, 3)
    setattr(p, field, val)
    assert prep(p) == code
    assert fwd(p) == code


def test_size_limits():
    # the largest accepted shapes keep every 32-bit index in range; one past is rejected
    assert A.padded_tokens(A.problem(1 << 30, 1)) == 1 << 30
    assert fwd(A.problem((1 << 30) + 1, 1)) == -2
    assert prep(A.problem((1 << 30) + 1, 1)) == -2
    assert A.prepped_qk_bytes(A.problem(1 << 30, 1 << 10)) == (1 << 30) * (1 << 10) * 128 * 2
    assert fwd(A.problem(1 << 30, (1 << 10) + 1)) == -2      # H * N_pad above 2^40
    # the largest accepted V token stride passes its check and fails only at the later
    # scale check (so nothing is ever launched on these fake pointers)
    assert fwd(A.problem(1000, 3), vst=(1 << 24), scale=0.0) == -2


def test_section_validation():
    p = A.problem(1000, 3, sections=(32, 48, 32))
    assert prep(p) == -2                       # does not sum to 128
    # any even widths pass the descriptor check (the null Q pointer is what fails)
    for sec in ((40, 40, 48), (34, 46, 48), (2, 62, 64), (0, 64, 64), (128, 0, 0)):
        assert prep(A.problem(1000, 3, sections=sec), q=None) == -1, sec
        assert fwd(A.problem(1000, 3, sections=sec), q=None) == -1, sec
    p = A.problem(1000, 3, sections=(33, 47, 48))
    assert prep(p) == -2                       # odd widths
    p = A.problem(1000, 3, sections=(-16, 96, 48))
    assert prep(p) == -2
    # the fused-Q forwards build only whole-chunk pairs
    assert fwd_fq(A.problem(1000, 3, sections=(40, 40, 48))) == -3
    assert fwd_fq8(A.problem(1000, 3, A.QK_I8_BLK64, sections=(40, 40, 48)), ks=None) == -3
    assert prep(A.problem(1000, 3, theta=0.0)) == -2
    assert prep(A.problem(1000, 3, eps=-1.0)) == -2
    assert prep(A.problem(1000, 3, eps=float("nan"))) == -2


def test_prep_pointer_and_alignment_checks():
    p = A.problem(1000, 3)
    assert prep(p, q=None) == -1
    assert prep(p, k=None) == -1
    assert prep(p, gq=None) == -1
    assert prep(p, pos=None) == -1
    assert prep(p, qo=None) == -1
    assert prep(p, q=F + 2) == -4             # not 16-byte aligned
    assert prep(p, qst=383) == -4             # stride not a multiple of 8
    assert prep(p, qsh=-128) == -2
    assert prep(p, gsh=4) == -4
    assert prep(p, qs=K) == -2                # scales given in bf16 format
    p8 = A.problem(1000, 3, A.QK_I8_BLK64)
    assert prep(p8) == -1                     # scales missing in int8 format
    assert prep(p8, qs=K, ks=K + 4096, qo=J + 3) == -4


def prep_ks(p, q=F, qst=384, qsh=128, k=G, kst=384, ksh=128, gq=H, gk=H + 256, gsh=0, pos=I,
            qo=J, ko=J + (1 << 32), qs=K, ks=K + 4096, km=K + 8192):
    return A.lib.h3attn_prep_ksmooth(ctypes.byref(p), q, qst, qsh, k, kst, ksh, gq, gk, gsh, pos,
                                     qo, ko, qs, ks, km, None)


def test_prep_ksmooth_checks():
    p8 = A.problem(1000, 3, A.QK_I8_BLK64)
    assert prep_ks(A.problem(1000, 3)) == -3             # bf16 format: nothing to smooth
    assert prep_ks(p8, km=None) == -1
    assert prep_ks(p8, km=K + 8194) == -4
    assert prep_ks(p8, km=K + 16) == -5                  # mean over the q scales
    assert prep_ks(p8, km=J + 64) == -5                  # mean inside q_out
    assert prep_ks(p8, qs=None) == -1
    assert prep_ks(p8, q=None) == -1


def test_prep_alias_checks():
    p = A.problem(1000, 3)
    assert prep(p, qo=F) == -5                          # output on top of q
    assert prep(p, ko=J + 1000 * 128) == -5             # k_out overlaps q_out
    assert prep(p, qo=I - 64) == -5                     # overlaps positions
    p8 = A.problem(1000, 3, A.QK_I8_BLK64)
    assert prep(p8, qs=J + 16, ks=K) == -5              # scales inside q_out


def test_forward_checks():
    p = A.problem(1000, 3)
    assert fwd(p, q=None) == -1
    assert fwd(p, v=None) == -1
    assert fwd(p, o=None) == -1
    assert fwd(p, scale=0.0) == -2
    assert fwd(p, scale=float("inf")) == -2
    assert fwd(p, scale=-0.1) == -2
    assert fwd(p, o=I + 8) == -4
    assert fwd(p, ost=100) == -4
    assert fwd(p, ost=128, osh=128) == -2                # output rows overlap each other
    assert fwd(p, ost=384, osh=64) == -2
    assert fwd(p, qs=K) == -2                            # scales in bf16 format
    assert fwd(p, vst=(1 << 24) + 8) == -3               # V token stride beyond 32-bit tile offsets
    assert fwd(p, o=F + 4096) == -5                      # output inside q'
    assert fwd(p, o=H + 384 * 10) == -5                  # output inside v
    p8 = A.problem(1000, 3, A.QK_I8_BLK64)
    assert fwd(p8) == -1
    assert fwd(p8, qs=K, ks=K + 4096, o=K + 16) == -5


def prep_v(p, v=F, vst=384, vsh=128, codes=G, scales=H):
    return A.lib.h3attn_prep_v_fp8(ctypes.byref(p), v, vst, vsh, codes, scales, None)


def fwd8v(p, q=F, k=G, qs=None, ks=None, codes=H, vs=J, o=I, ost=384, osh=128, scale=0.088):
    return A.lib.h3attn_forward_fp8v(ctypes.byref(p), q, k, qs, ks, codes, vs, o, ost, osh, scale, None)


def test_prep_v_fp8_checks():
    p = A.problem(1000, 3)
    assert prep_v(A.problem(1000, 3, head_dim=64)) == -3
    assert prep_v(p, v=None) == -1
    assert prep_v(p, codes=None) == -1
    assert prep_v(p, scales=None) == -1
    assert prep_v(p, v=F + 2) == -4
    assert prep_v(p, codes=G + 8) == -4
    assert prep_v(p, scales=H + 2) == -4
    assert prep_v(p, vst=100) == -4
    assert prep_v(p, codes=F + 384 * 10) == -5                 # codes on top of v
    assert prep_v(p, scales=F + 64) == -5                      # scales inside v
    assert prep_v(p, scales=G + A.prepped_v_bytes(p) - 4) == -5   # scales overlap the codes' end


def test_forward_fp8v_checks():
    p = A.problem(1000, 3)
    assert fwd8v(p, codes=None) == -1
    assert fwd8v(p, vs=None) == -1
    assert fwd8v(p, q=None) == -1
    assert fwd8v(p, codes=H + 8) == -4
    assert fwd8v(p, vs=J + 2) == -4
    assert fwd8v(p, scale=0.0) == -2
    assert fwd8v(p, qs=K) == -2                                # scales in bf16 format
    assert fwd8v(p, o=H + 4096) == -5                          # output inside the codes
    assert fwd8v(p, o=J - 64) == -5                            # output over the V scales
    p8 = A.problem(1000, 3, A.QK_I8_BLK64)
    assert fwd8v(p8) == -1


def test_calibration_checks():
    call = A.lib.h3attn_calibrate_mfma_bf16
    assert call(8, 10, None, None) == -1
    assert call(8, 10, K + 2, None) == -4
    assert call(0, 10, K, None) == -2
    assert call(8, 0, K, None) == -2
    assert call((1 << 20) + 1, 10, K, None) == -2


def test_debug_scores_checks():
    p8 = A.problem(300, 2, A.QK_I8_BLK64)
    call = lambda p=p8, head=0, r0=0, nr=10, c0=0, nc=10, lay=0, out=K: A.lib.h3attn_debug_scores_i32(
        ctypes.byref(p), F, G, head, r0, nr, c0, nc, lay, out, None)
    assert call(p=A.problem(300, 2)) == -3
    assert call(head=2) == -2
    assert call(head=-1) == -2
    assert call(nr=0) == -2
    assert call(r0=295, nr=6) == -2
    assert call(c0=300) == -2
    assert call(lay=2) == -2
    assert call(lay=-1) == -2
    assert call(out=None) == -1
    assert call(out=F + 64) == -5


def test_binding_rejects_non_nhd_views():
    torch = pytest.importorskip("torch")
    p = A.problem(4, 1)
    x = torch.zeros(4, 1, 128, dtype=torch.bfloat16).transpose(1, 2)
    with pytest.raises(ValueError):
        A.forward(p, x, x, x, x, 0.1)


def prep_k(p, k=G, kst=384, ksh=128, gk=H, gsh=0, pos=I, ko=J):
    return A.lib.h3attn_prep_k(ctypes.byref(p), k, kst, ksh, gk, gsh, pos, ko, None)


def fwd_fq(p, q=F, qst=384, qsh=128, gq=H, gsh=0, pos=I, k=G, v=K, vst=384, vsh=128, o=J, ost=384, osh=128,
           scale=0.088):
    return A.lib.h3attn_forward_fused_q(ctypes.byref(p), q, qst, qsh, gq, gsh, pos, k, v, vst, vsh, o, ost, osh,
                                        scale, None)


def test_prep_k_checks():
    p = A.problem(1000, 3)
    assert prep_k(A.problem(1000, 3, A.QK_I8_BLK64)) == -3   # K' alone only in bf16
    assert prep_k(A.problem(1000, 3, head_dim=64)) == -3
    assert prep_k(p, k=None) == -1
    assert prep_k(p, gk=None) == -1
    assert prep_k(p, pos=None) == -1
    assert prep_k(p, ko=None) == -1
    assert prep_k(p, k=G + 2) == -4
    assert prep_k(p, kst=383) == -4
    assert prep_k(p, gsh=4) == -4
    assert prep_k(p, ko=J + 8) == -4
    assert prep_k(p, ko=G + 384 * 10) == -5                 # output on top of k
    assert prep_k(p, ko=I - 64) == -5                       # overlaps positions
    assert prep_k(p, ko=H - 64) == -5                       # overlaps gamma


def prep_k_i8(p, k=G, kst=384, ksh=128, gk=H, gsh=0, pos=I, ko=J, ks=K):
    return A.lib.h3attn_prep_k_i8(ctypes.byref(p), k, kst, ksh, gk, gsh, pos, ko, ks, None)


def fwd_fq8(p, q=F, qst=384, qsh=128, gq=H, gsh=0, pos=I, k=G, ks=G + (1 << 32), v=K, vst=384, vsh=128, o=J,
            ost=384, osh=128, scale=0.088):
    return A.lib.h3attn_forward_fused_q_i8(ctypes.byref(p), q, qst, qsh, gq, gsh, pos, k, ks, v, vst, vsh, o, ost,
                                           osh, scale, None)


def test_prep_k_i8_checks():
    p = A.problem(1000, 3, A.QK_I8_BLK64)
    assert prep_k_i8(A.problem(1000, 3)) == -3                # int8 codes only
    assert prep_k_i8(A.problem(1000, 3, A.QK_I8_BLK64, head_dim=64)) == -3
    for kw in ("k", "gk", "pos", "ko", "ks"):
        assert prep_k_i8(p, **{kw: None}) == -1, kw
    assert prep_k_i8(p, k=G + 2) == -4
    assert prep_k_i8(p, ko=J + 8) == -4
    assert prep_k_i8(p, ks=K + 2) == -4
    assert prep_k_i8(p, ko=G + 384 * 10) == -5                # codes on top of k
    assert prep_k_i8(p, ks=H - 64) == -5                      # scales over gamma
    assert prep_k_i8(p, ks=J + 4096) == -5                    # scales inside the codes
    assert prep_k_i8(p, ko=K - 64) == -5                      # codes over the scales


def test_forward_fused_q_i8_checks():
    p = A.problem(1000, 3, A.QK_I8_BLK64)
    assert fwd_fq8(A.problem(1000, 3)) == -3                  # int8 only
    for kw in ("q", "gq", "pos", "k", "ks", "v", "o"):
        assert fwd_fq8(p, **{kw: None}) == -1, kw
    assert fwd_fq8(p, q=F + 2) == -4
    assert fwd_fq8(p, ks=G + (1 << 32) + 2) == -4
    assert fwd_fq8(p, scale=0.0) == -2
    assert fwd_fq8(p, o=F + 384 * 10) == -5                   # output over raw q
    assert fwd_fq8(p, o=G + (1 << 32)) == -5                  # output over the K scales
    assert fwd_fq8(p, o=K + 384 * 10) == -5                   # output inside v


def test_forward_fused_q_checks():
    p = A.problem(1000, 3)
    assert fwd_fq(A.problem(1000, 3, A.QK_I8_BLK64)) == -3  # bf16 only
    for kw in ("q", "gq", "pos", "k", "v", "o"):
        assert fwd_fq(p, **{kw: None}) == -1, kw
    assert fwd_fq(p, q=F + 2) == -4
    assert fwd_fq(p, qst=100) == -4
    assert fwd_fq(p, gsh=4) == -4
    assert fwd_fq(p, pos=I + 2) == -4
    assert fwd_fq(p, k=G + 8) == -4
    assert fwd_fq(p, scale=0.0) == -2
    assert fwd_fq(p, ost=128, osh=128) == -2                 # output rows overlap each other
    assert fwd_fq(p, o=F + 384 * 10) == -5                   # output over raw q
    assert fwd_fq(p, o=H - 64) == -5                         # output over gamma_q
    assert fwd_fq(p, o=I + 64) == -5                         # output over the positions
    assert fwd_fq(p, o=G + 4096) == -5                       # output inside k'
    assert fwd_fq(p, o=K + 384 * 10) == -5                   # output inside v


def test_phase_timing_calls_outside_the_timing_build():
    # release and race-detection builds: unsupported, without touching the GPU
    for lib in (A.lib, A.variant(A.SYNC_LIB_PATH).lib):
        buf = (ctypes.c_ulonglong * A.PHASE_TIMING_COUNTERS)()
        assert lib.h3attn_phase_timing_read(buf) == -3
        assert lib.h3attn_phase_timing_clear() == -3
    # the phase-timing build checks its pointer first
    assert A.variant(A.TIMING_LIB_PATH).lib.h3attn_phase_timing_read(None) == -1
