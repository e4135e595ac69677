"""Thin Python binding of ``libh3attn.so`` (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module only
turns torch tensors into pointers, strides and a stream handle.  There is no
fallback: if the library is not built, importing the binding raises.

The calls mirror ``include/h3attn.h``:

* :func:`prep`      - Q/K RMSNorm + 3-axis split-half RoPE -> head-major Q'/K'
* :func:`prep_ksmooth` - :func:`prep` in the int8 format with K smoothing
* :func:`forward`   - softmax(Q' K'^T * scale) V over the packed sequence
* :func:`prep_v_fp8` - V -> E4M3 codes (d-major 64-key tiles) + fp32 channel scales
* :func:`forward_fp8v` - :func:`forward` with the P V product on FP8 matrix cores
* :func:`debug_scores_i32` - exact int32 Q'K'^T window of the int8 format
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# another build of the library can be bound by loading this module's source
# under a new name with _LIB_PATH set first (see :func:`variant`)
LIB_PATH = globals().get("_LIB_PATH", os.path.join(PKG, "libh3attn.so"))
# the race-detection build: a barrier after every LDS stage of the forward
SYNC_LIB_PATH = os.path.join(PKG, "libh3attn_sync.so")
# the phase-timing build: shader-clock stamps in the forward's tile loop
TIMING_LIB_PATH = os.path.join(PKG, "libh3attn_timing.so")
PHASE_TIMING_COUNTERS = 30

QK_BF16 = 0
QK_I8_BLK64 = 1
ABI_VERSION = 8

STATUS = {0: "OK", -1: "E_NULL", -2: "E_SHAPE", -3: "E_UNSUPPORTED", -4: "E_ALIGN",
          -5: "E_ALIAS", -6: "E_HIP"}


class H3AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {STATUS.get(status, status)} ({_lib.h3attn_status_string(status).decode()})")


class Problem(ctypes.Structure):
    """``h3attn_problem`` (host memory)."""
    _fields_ = [
        ("n_tokens", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rope_sections", ctypes.c_int32 * 3),
        ("rope_theta", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
        ("qk_format", ctypes.c_int32),
    ]


# a binding bound to another build (:func:`variant`) shares this class, so the
# same descriptor objects are accepted by both
Problem = globals().get("_PROBLEM_CLASS", Problem)


def problem(n_tokens: int, n_heads: int, qk_format: int = QK_BF16, head_dim: int = 128,
            sections=(32, 48, 48), theta: float = 10000.0, eps: float = 1e-6) -> Problem:
    p = Problem()
    p.n_tokens, p.n_heads, p.head_dim = n_tokens, n_heads, head_dim
    p.rope_sections[:] = list(sections)
    p.rope_theta, p.rms_eps, p.qk_format = theta, eps, qk_format
    return p


def _hip_runtimes():
    """Distinct HIP runtime files mapped into this process."""
    try:
        maps = open("/proc/self/maps").read().splitlines()
    except OSError:
        return set()
    return {ln.split()[-1] for ln in maps if "libamdhip64" in ln}


def _load():
    # torch brings its own HIP runtime; it must be the only one in the process,
    # so it is loaded first and the library's libamdhip64.so.7 dependency
    # resolves to it (same soname).  Streams and device memory come from torch.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m audio_video_diffusion_amd.build` "
                          "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    pp = ctypes.POINTER(Problem)
    sig = {
        "h3attn_abi_version": (ctypes.c_int, []),
        "h3attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "h3attn_padded_tokens": (i64, [pp]),
        "h3attn_prepped_qk_bytes": (ctypes.c_size_t, [pp]),
        "h3attn_scales_bytes": (ctypes.c_size_t, [pp]),
        "h3attn_prepped_v_bytes": (ctypes.c_size_t, [pp]),
        "h3attn_v_scales_bytes": (ctypes.c_size_t, [pp]),
        "h3attn_prep": (ctypes.c_int, [pp, vp, i64, i64, vp, i64, i64, vp, vp, i64, vp,
                                       vp, vp, vp, vp, vp]),
        "h3attn_forward": (ctypes.c_int, [pp, vp, vp, vp, vp, vp, i64, i64, vp, i64, i64, f32, vp]),
        "h3attn_prep_ksmooth": (ctypes.c_int, [pp, vp, i64, i64, vp, i64, i64, vp, vp, i64, vp,
                                               vp, vp, vp, vp, vp, vp]),
        "h3attn_prep_v_fp8": (ctypes.c_int, [pp, vp, i64, i64, vp, vp, vp]),
        "h3attn_forward_fp8v": (ctypes.c_int, [pp, vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, vp]),
        "h3attn_debug_scores_i32": (ctypes.c_int, [pp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]),
        "h3attn_calibrate_mfma_bf16": (ctypes.c_int, [i32, i32, vp, vp]),
        "h3attn_prep_k": (ctypes.c_int, [pp, vp, i64, i64, vp, i64, vp, vp, vp]),
        "h3attn_forward_fused_q": (ctypes.c_int, [pp, vp, i64, i64, vp, i64, vp, vp, vp, i64, i64, vp, i64, i64,
                                                  f32, vp]),
        "h3attn_prep_k_i8": (ctypes.c_int, [pp, vp, i64, i64, vp, i64, vp, vp, vp, vp]),
        "h3attn_forward_fused_q_i8": (ctypes.c_int, [pp, vp, i64, i64, vp, i64, vp, vp, vp, vp, i64, i64, vp, i64,
                                                     i64, f32, vp]),
        "h3attn_phase_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_ulonglong)]),
        "h3attn_phase_timing_clear": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    if lib.h3attn_abi_version() != ABI_VERSION:
        raise ImportError("libh3attn.so ABI version mismatch: rebuild it")
    if len(_hip_runtimes()) > 1:
        raise ImportError(f"more than one HIP runtime is loaded: {sorted(_hip_runtimes())}")
    return lib


_lib = _load()
lib = _lib


def variant(path: str):
    """This binding, bound to another build of the library (e.g. :data:`SYNC_LIB_PATH`).

    Returns a separate module object whose functions call the library at
    ``path``; this module keeps its own library."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(f"{__name__}_variant_{abs(hash(path))}", __file__)
    mod = importlib.util.module_from_spec(spec)
    mod._LIB_PATH = path
    mod._PROBLEM_CLASS = Problem
    spec.loader.exec_module(mod)
    return mod


def padded_tokens(p: Problem) -> int:
    return _lib.h3attn_padded_tokens(ctypes.byref(p))


def prepped_qk_bytes(p: Problem) -> int:
    return _lib.h3attn_prepped_qk_bytes(ctypes.byref(p))


def scales_bytes(p: Problem) -> int:
    return _lib.h3attn_scales_bytes(ctypes.byref(p))


def prepped_v_bytes(p: Problem) -> int:
    return _lib.h3attn_prepped_v_bytes(ctypes.byref(p))


def v_scales_bytes(p: Problem) -> int:
    return _lib.h3attn_v_scales_bytes(ctypes.byref(p))


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def _nhd(t, name):
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be an [N, H, d] view with a contiguous last axis")
    return t.data_ptr(), t.stride(0), t.stride(1)


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def alloc_prepped(p: Problem, device="cuda"):
    """Caller-side buffers for :func:`prep`: (q_out, k_out, q_scales, k_scales)."""
    import torch
    npad = padded_tokens(p)
    dt = torch.bfloat16 if p.qk_format == QK_BF16 else torch.int8
    q_out = torch.empty((p.n_heads, npad, p.head_dim), dtype=dt, device=device)
    k_out = torch.empty_like(q_out)
    if p.qk_format == QK_BF16:
        return q_out, k_out, None, None
    nblk = (p.n_tokens + 63) // 64
    q_s = torch.empty((p.n_heads, nblk), dtype=torch.float32, device=device)
    return q_out, k_out, q_s, torch.empty_like(q_s)


def prep(p: Problem, q, k, gamma_q, gamma_k, pos, q_out, k_out, q_scales=None, k_scales=None,
         stream=None):
    """``h3attn_prep`` on torch tensors (bf16 q/k views [N,H,d], gamma [d] or [H,d], pos int32 [N,3])."""
    qp, qst, qsh = _nhd(q, "q")
    kp, kst, ksh = _nhd(k, "k")
    if gamma_q.shape != gamma_k.shape or gamma_q.stride() != gamma_k.stride():
        raise ValueError("gamma_q and gamma_k must have the same shape and strides")
    gsh = gamma_q.stride(0) if gamma_q.dim() == 2 else 0
    rc = _lib.h3attn_prep(ctypes.byref(p), qp, qst, qsh, kp, kst, ksh, _ptr(gamma_q), _ptr(gamma_k),
                          gsh, _ptr(pos), _ptr(q_out), _ptr(k_out), _ptr(q_scales), _ptr(k_scales),
                          _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_prep")


def prep_ksmooth(p: Problem, q, k, gamma_q, gamma_k, pos, q_out, k_out, q_scales, k_scales, k_mean,
                 stream=None):
    """``h3attn_prep_ksmooth``: int8 prep with K smoothing; ``k_mean`` fp32 [H, 128] receives the means."""
    qp, qst, qsh = _nhd(q, "q")
    kp, kst, ksh = _nhd(k, "k")
    if gamma_q.shape != gamma_k.shape or gamma_q.stride() != gamma_k.stride():
        raise ValueError("gamma_q and gamma_k must have the same shape and strides")
    gsh = gamma_q.stride(0) if gamma_q.dim() == 2 else 0
    rc = _lib.h3attn_prep_ksmooth(ctypes.byref(p), qp, qst, qsh, kp, kst, ksh, _ptr(gamma_q), _ptr(gamma_k),
                                  gsh, _ptr(pos), _ptr(q_out), _ptr(k_out), _ptr(q_scales), _ptr(k_scales),
                                  _ptr(k_mean), _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_prep_ksmooth")


def forward(p: Problem, q_prep, k_prep, v, o, softmax_scale: float, q_scales=None, k_scales=None,
            stream=None):
    """``h3attn_forward`` on torch tensors (v and o bf16 [N,H,d] views)."""
    vp, vst, vsh = _nhd(v, "v")
    op, ost, osh = _nhd(o, "o")
    rc = _lib.h3attn_forward(ctypes.byref(p), _ptr(q_prep), _ptr(k_prep), _ptr(q_scales),
                             _ptr(k_scales), vp, vst, vsh, op, ost, osh, float(softmax_scale),
                             _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_forward")


def _gamma_stride(g):
    return g.stride(0) if g.dim() == 2 else 0


def prep_k(p: Problem, k, gamma_k, pos, k_out, stream=None):
    """``h3attn_prep_k``: bf16 K' alone (k bf16 [N,H,d] view, gamma [d] or [H,d], pos int32 [N,3])."""
    kp, kst, ksh = _nhd(k, "k")
    rc = _lib.h3attn_prep_k(ctypes.byref(p), kp, kst, ksh, _ptr(gamma_k), _gamma_stride(gamma_k), _ptr(pos),
                            _ptr(k_out), _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_prep_k")


def prep_k_i8(p: Problem, k, gamma_k, pos, k_out, k_scales, stream=None):
    """``h3attn_prep_k_i8``: int8 K' codes and block scales alone (int8 problem)."""
    kp, kst, ksh = _nhd(k, "k")
    rc = _lib.h3attn_prep_k_i8(ctypes.byref(p), kp, kst, ksh, _ptr(gamma_k), _gamma_stride(gamma_k), _ptr(pos),
                               _ptr(k_out), _ptr(k_scales), _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_prep_k_i8")


def forward_fused_q_i8(p: Problem, q, gamma_q, pos, k_codes, k_scales, v, o, softmax_scale: float, stream=None):
    """``h3attn_forward_fused_q_i8``: the int8 forward from raw Q (q, v, o bf16 [N,H,d] views)."""
    qp, qst, qsh = _nhd(q, "q")
    vp, vst, vsh = _nhd(v, "v")
    op, ost, osh = _nhd(o, "o")
    rc = _lib.h3attn_forward_fused_q_i8(ctypes.byref(p), qp, qst, qsh, _ptr(gamma_q), _gamma_stride(gamma_q),
                                        _ptr(pos), _ptr(k_codes), _ptr(k_scales), vp, vst, vsh, op, ost, osh,
                                        float(softmax_scale), _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_forward_fused_q_i8")


def forward_fused_q(p: Problem, q, gamma_q, pos, k_prep, v, o, softmax_scale: float, stream=None):
    """``h3attn_forward_fused_q``: the bf16 forward from raw Q (q, v, o bf16 [N,H,d] views)."""
    qp, qst, qsh = _nhd(q, "q")
    vp, vst, vsh = _nhd(v, "v")
    op, ost, osh = _nhd(o, "o")
    rc = _lib.h3attn_forward_fused_q(ctypes.byref(p), qp, qst, qsh, _ptr(gamma_q), _gamma_stride(gamma_q),
                                     _ptr(pos), _ptr(k_prep), vp, vst, vsh, op, ost, osh, float(softmax_scale),
                                     _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_forward_fused_q")


def alloc_v_fp8(p: Problem, device="cuda"):
    """Caller-side buffers for :func:`prep_v_fp8`: (codes uint8 [H, N_pad/64, 128, 64], scales fp32 [H, 128])."""
    import torch
    npad = padded_tokens(p)
    codes = torch.empty((p.n_heads, npad // 64, p.head_dim, 64), dtype=torch.uint8, device=device)
    return codes, torch.empty((p.n_heads, p.head_dim), dtype=torch.float32, device=device)


def prep_v_fp8(p: Problem, v, v_codes, v_scales, stream=None):
    """``h3attn_prep_v_fp8`` on torch tensors (v bf16 [N,H,d] view)."""
    vp, vst, vsh = _nhd(v, "v")
    rc = _lib.h3attn_prep_v_fp8(ctypes.byref(p), vp, vst, vsh, _ptr(v_codes), _ptr(v_scales), _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_prep_v_fp8")


def forward_fp8v(p: Problem, q_prep, k_prep, v_codes, v_scales, o, softmax_scale: float, q_scales=None,
                 k_scales=None, stream=None):
    """``h3attn_forward_fp8v`` on torch tensors (o bf16 [N,H,d] view)."""
    op, ost, osh = _nhd(o, "o")
    rc = _lib.h3attn_forward_fp8v(ctypes.byref(p), _ptr(q_prep), _ptr(k_prep), _ptr(q_scales),
                                  _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), op, ost, osh,
                                  float(softmax_scale), _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_forward_fp8v")


def debug_scores_i32(p: Problem, q_codes, k_codes, head: int, row0: int, nrows: int, col0: int,
                     ncols: int, out, stream=None, fp8v_layout: int = 0):
    """``h3attn_debug_scores_i32`` into ``out`` (int32 [nrows, ncols], contiguous).

    ``fp8v_layout`` 1 runs the kernel of the int8 + E4M3-V forward (its K' row order)."""
    rc = _lib.h3attn_debug_scores_i32(ctypes.byref(p), _ptr(q_codes), _ptr(k_codes), head, row0,
                                      nrows, col0, ncols, fp8v_layout, _ptr(out), _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_debug_scores_i32")


def calibrate_mfma_bf16(blocks: int, iters: int, out, stream=None):
    """``h3attn_calibrate_mfma_bf16`` into ``out`` (fp32, >= blocks * 512 elements); returns its FLOP count."""
    if out.numel() < blocks * 512:
        raise ValueError("out holds fewer than blocks * 512 floats")
    rc = _lib.h3attn_calibrate_mfma_bf16(blocks, iters, _ptr(out), _stream(stream))
    if rc:
        raise H3AttnError(rc, "h3attn_calibrate_mfma_bf16")
    return blocks * 8 * iters * 16 * 32768.0


def phase_timing_clear():
    """``h3attn_phase_timing_clear``: zero the counters (phase-timing build only)."""
    rc = _lib.h3attn_phase_timing_clear()
    if rc:
        raise H3AttnError(rc, "h3attn_phase_timing_clear")


def phase_timing_read():
    """``h3attn_phase_timing_read``: the 30 counters as a list of ints (phase-timing build only)."""
    buf = (ctypes.c_ulonglong * PHASE_TIMING_COUNTERS)()
    rc = _lib.h3attn_phase_timing_read(buf)
    if rc:
        raise H3AttnError(rc, "h3attn_phase_timing_read")
    return [int(x) for x in buf]
