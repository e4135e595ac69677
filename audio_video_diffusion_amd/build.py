"""Build ``libh3attn.so`` (gfx950 kernels + C ABI) in-tree with hipcc.

    python -m audio_video_diffusion_amd.build          # compile
    python -m audio_video_diffusion_amd.build --asm     # also keep the gfx950 assembly
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libh3attn.so")
# race-detection build of the same sources (tests only)
SYNC_LIB = os.path.join(PKG, "libh3attn_sync.so")
# phase-timing build of the same sources (a measurement aid: include/h3attn_phase_timing.h)
TIMING_LIB = os.path.join(PKG, "libh3attn_timing.so")
SOURCES = ("api.hip", "prep.hip", "prep_v.hip", "forward.hip", "calib.hip")
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code.  No fast-math: the
# int8 quantiser relies on correctly rounded fp32 division.
FLAGS = [
    f"--offload-arch={ARCH}", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libh3attn.so")


def _compile(out: str, defines=(), verbose: bool = False, asm: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if asm:
        os.makedirs(os.path.join(ROOT, "_build"), exist_ok=True)
        cmd[1:1] = ["-save-temps=cwd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    cwd = os.path.join(ROOT, "_build") if asm else CSRC
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, asm: bool = False) -> str:
    """Compile every HIP source into the in-tree shared library, and the same
    sources again into the race-detection build (a barrier after every LDS
    stage of the forward, used by the tests only) and the phase-timing build
    (shader-clock stamps in the forward's tile loop); returns the library path."""
    _compile(LIB, verbose=verbose, asm=asm)
    _compile(SYNC_LIB, defines=("H3_DEBUG_SYNC=1",), verbose=verbose)
    _compile(TIMING_LIB, defines=("H3_PHASE_TIMING=1",), verbose=verbose)
    return LIB


def device_asm(source: str, defines=()) -> str:
    """gfx950 assembly of one HIP source under the library's flags (device pass only)."""
    src = os.path.join(CSRC, source)
    flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [hipcc(), *flags, "--offload-device-only", "-S", *[f"-D{d}" for d in defines],
           "-I", os.path.join(ROOT, "include"), src, "-o", "-"]
    res = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr)
    return res.stdout


if __name__ == "__main__":
    print(build(verbose=True, asm="--asm" in sys.argv))
