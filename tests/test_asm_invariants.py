"""CPU tests of the gfx950 assembly that the forward kernels compile to.

The forward kernel relies on hand-written protocols the compiler cannot see:
buffer -> LDS copies issued from inline asm (M0 holds the LDS destination),
a per-tile vmcnt wait that counts those copies, and matrix-core products
issued from inline asm whose results the VALU reads after explicit wait
states.  These tests build forward.hip to assembly here (hipcc cross-compiles
gfx950 without a GPU) and check, kernel by kernel, the invariants those
protocols need:

* no scratch memory (no spills, no private segment);
* M0 is touched only by the copy helper, and every copy is at least one wait
  state after the scalar write of M0 it reads;
* inside each key-tile loop the only vmcnt waits are the kernel's own, none
  of them vmcnt(0) (which would drain the prefetch);
* every VALU read of a result of an inline-asm matrix-core product comes at
  least 13 wait states after that product (this compiler pads its own 32x32
  bf16 and int8 products on gfx950 with 12 before a dependent VALU read:
  s_nop 11; one to spare);
* every matrix-core product comes at least 2 wait states after the last VALU
  write of any of its source registers (A, B or C; the gfx950 VALU-write ->
  XDL-read spacing, which the compiler enforces only for writes it can see,
  not for the products or the accumulator writes the kernel issues in asm);
* nothing writes the C-operand registers of an inline-asm product whose C is
  not its own destination (a chain's first product) within 18 wait states of
  it: a product reads C late, and a 32x32 product needs at most 15 (the
  compiler, blind to the asm product, once handed those registers to a VALU
  result 0-3 wait states later in a stage-unrolled build of the loop, which
  then computed wrong rows);
"""
import re
import shutil

import pytest

from audio_video_diffusion_amd.build import device_asm

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists(
    "/opt/rocm/bin/hipcc"), reason="hipcc is needed to build the assembly")

KERNELS = {
    # mangled template arguments of fwd8_kernel -> the form it builds
    "ILb0ELb0ELb0ELi8ELb0E": "bf16 Q'/K', bf16 V",
    "ILb0ELb0ELb1ELi8ELb0E": "fused Q prep",
    "ILb1ELb0ELb0ELi12ELb0E": "int8 Q'/K', bf16 V (twelve waves)",
    "ILb1ELb0ELb1ELi12ELb0E": "int8 Q'/K', bf16 V, fused Q prep (twelve waves)",
    "ILb0ELb1ELb0ELi8ELb0E": "bf16 Q'/K', E4M3 V",
    "ILb1ELb1ELb0ELi12ELb0E": "int8 Q'/K', E4M3 V (twelve waves)",
    "ILb1ELb0ELb0ELi12ELb1E": "int32 scores hook, bf16-V K' order",
    "ILb1ELb1ELb0ELi12ELb1E": "int32 scores hook, E4M3-V K' order",
}
MFMA_VALU_WAIT_STATES = 13
VALU_MFMA_WAIT_STATES = 2
SRCC_WAR_WAIT_STATES = 18


@pytest.fixture(scope="module")
def kernels():
    text = device_asm("forward.hip")
    lines = text.split("\n")
    out = {}
    for i, ln in enumerate(lines):
        m = re.match(r"^(_Z\w+fwd8_kernel\w+):", ln)
        if not m:
            continue
        # the kernel descriptor (.amdhsa_kernel ... .end_amdhsa_kernel) closes the function
        meta0 = next(j for j in range(i, len(lines)) if ".amdhsa_kernel " + m.group(1) in lines[j])
        meta1 = next(j for j in range(meta0, len(lines)) if ".end_amdhsa_kernel" in lines[j])
        end = meta0
        key = next((k for k in KERNELS if k in m.group(1)), None)
        assert key is not None, f"unexpected kernel {m.group(1)}"
        out[key] = (lines[i:end], lines[meta0:meta1])
    return out


def instructions(body):
    """(index, text, in_asm) for every instruction line of a function body."""
    res, in_asm = [], False
    for ln in body:
        s = ln.split(";")[0].strip()
        if ";;#ASMSTART" in ln:
            in_asm = True
            continue
        if ";;#ASMEND" in ln:
            in_asm = False
            continue
        if not s or s.endswith(":") or s.startswith("."):
            continue
        res.append((len(res), s, in_asm))
    return res


def regs(operand):
    """Register names (e.g. 'v12', 'a3') an operand covers."""
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", operand)
    if m:
        return {f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", operand)
    return {operand} if m else set()


def operands(ins):
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o.strip() for o in parts[1].split(",")]


def wait_states(ins):
    op, ops = operands(ins)
    if op == "s_nop":
        return int(ops[0], 0) + 1
    return 1


def test_all_forms_present(kernels):
    assert set(kernels) == set(KERNELS)


# Twelve-wave forms (168 registers per wave) that keep a few values in
# scratch outside the tile loop (lane-derived values that only the ragged last
# tile and the epilogue use, prologue state); nothing inside a loop touches it.
SCRATCH_OUTSIDE_LOOPS = {"ILb1ELb1ELb0ELi12ELb0E", "ILb1ELb0ELb1ELi12ELb0E"}


def loop_lines(body):
    """Indices of the lines in loop blocks: the compiler marks each basic block
    of a loop on its label line ("Loop Header" or "in Loop:")."""
    res, inside = set(), False
    for i, ln in enumerate(body):
        if re.match(r"^(\.LBB\w+:|\s*; %bb\.\d+:)", ln):
            inside = "Loop Header" in ln or "in Loop:" in ln
        if inside:
            res.add(i)
    return res


@pytest.mark.parametrize("key", sorted(KERNELS))
def test_no_scratch(kernels, key):
    body, meta = kernels[key]
    scratch = [i for i, ln in enumerate(body) if re.search(r"\bscratch_(load|store)", ln)]
    if key in SCRATCH_OUTSIDE_LOOPS:
        size = next(int(m.group(1)) for ln in meta
                    for m in [re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", ln)] if m)
        assert size <= 64, (KERNELS[key], size)
        loops = loop_lines(body)
        assert loops, KERNELS[key]
        assert not loops.intersection(scratch), KERNELS[key]
    else:
        assert any(re.search(r"\.amdhsa_private_segment_fixed_size 0\b", ln) for ln in meta), KERNELS[key]
        assert not scratch, KERNELS[key]
    assert not any(re.search(r"buffer_store\w* .*s\[0:3\]", ln) for ln in body), KERNELS[key]


@pytest.mark.parametrize("key", sorted(KERNELS))
def test_m0_protocol(kernels, key):
    ins = instructions(kernels[key][0])
    dmas = 0
    for i, s, in_asm in ins:
        if re.search(r"\bm0\b", s):
            # only the copy helper's asm touches M0
            assert in_asm, (KERNELS[key], s)
        if s.endswith(" lds") or " lds " in s:
            dmas += 1
            # walk back to the scalar write of M0 this copy reads: at least one
            # wait state must separate them
            ws = 0
            j = i - 1
            while j >= 0 and not re.match(r"s_\w+ m0,", ins[j][1]):
                ws += wait_states(ins[j][1])
                j -= 1
            assert j >= 0, (KERNELS[key], "copy without an M0 write before it")
            assert ws >= 1, (KERNELS[key], i, s)
    assert dmas > 0


@pytest.mark.parametrize("key", sorted(KERNELS))
def test_tile_loop_waits(kernels, key):
    body = kernels[key][0]
    # map labels and backward branches on the raw lines
    labels = {}
    for i, ln in enumerate(body):
        m = re.match(r"^(\.LBB\w+):", ln)
        if m:
            labels[m.group(1)] = i
    spans = []
    for i, ln in enumerate(body):
        m = re.match(r"\s+s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", ln)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            spans.append((labels[m.group(1)], i))
    tile_loops = [(a, b) for a, b in spans if any(" lds" in body[k] for k in range(a, b + 1))]
    assert tile_loops, KERNELS[key]
    own = 0
    for lo, hi in tile_loops:
        in_asm = False
        for k in range(lo, hi + 1):
            ln = body[k]
            if ";;#ASMSTART" in ln:
                in_asm = True
            elif ";;#ASMEND" in ln:
                in_asm = False
            elif "vmcnt" in ln and ln.strip().startswith("s_waitcnt"):
                if "vmcnt(63)" in ln:
                    continue            # the counter's maximum: no wait on vector memory
                assert in_asm, (KERNELS[key], "compiler vmcnt wait in the tile loop", ln.strip())
                if "all copies landed" in ln:
                    continue            # the drain after the last tile (the compiler may lay
                                        # rare blocks of the loop out after it)
                assert "vmcnt(0)" not in ln, (KERNELS[key], ln.strip())
                own += 1
    assert own >= 1, KERNELS[key]


@pytest.mark.parametrize("key", sorted(KERNELS))
def test_mfma_results_read_after_wait_states(kernels, key):
    ins = instructions(kernels[key][0])
    checked = 0
    for i, s, in_asm in ins:
        if not (in_asm and s.startswith("v_mfma")):
            continue
        op, ops = operands(s)
        dst = regs(ops[0])
        if not dst or not next(iter(dst)).startswith("v"):
            continue
        ws = 0
        for j in range(i + 1, min(len(ins), i + 200)):
            t = ins[j][1]
            top, tops = operands(t)
            if top.startswith("s_cbranch") or top.startswith("s_branch") or top == "s_endpgm":
                break
            used = set().union(*[regs(o) for o in tops]) if tops else set()
            if used & dst:
                if top.startswith("v_mfma") and regs(tops[0]) == dst and regs(tops[-1]) == dst:
                    break           # the chain accumulates in place: checked at its end
                assert ws >= MFMA_VALU_WAIT_STATES, (KERNELS[key], s, t, ws)
                checked += 1
                break
            ws += wait_states(t)
    if "scores" not in KERNELS[key]:
        assert checked > 0, KERNELS[key]


@pytest.mark.parametrize("key", sorted(KERNELS))
def test_mfma_sources_written_before_wait_states(kernels, key):
    ins = instructions(kernels[key][0])
    products = 0
    for i, s, in_asm in ins:
        if not s.startswith("v_mfma"):
            continue
        products += 1
        _, ops = operands(s)
        src = set().union(*[regs(o) for o in ops[1:]])
        ws = 0
        for j in range(i - 1, max(-1, i - 16), -1):
            t = ins[j][1]
            top, tops = operands(t)
            if top.startswith("s_cbranch") or top.startswith("s_branch"):
                break
            if top.startswith("v_") and not top.startswith("v_mfma") and tops and regs(tops[0]) & src:
                assert ws >= VALU_MFMA_WAIT_STATES, (KERNELS[key], t, s, ws)
                break
            ws += wait_states(t)
    assert products > 0, KERNELS[key]


WRITERS = ("v_", "ds_read", "buffer_load", "global_load", "scratch_load", "flat_load")


@pytest.mark.parametrize("key", sorted(KERNELS))
def test_chain_start_c_operand_not_overwritten_early(kernels, key):
    ins = instructions(kernels[key][0])
    starts = 0
    for i, s, in_asm in ins:
        if not (in_asm and s.startswith("v_mfma")):
            continue
        _, ops = operands(s)
        c, d = regs(ops[3]), regs(ops[0])
        if not c or c == d:
            continue
        starts += 1
        ws = 0
        for j in range(i + 1, min(len(ins), i + 80)):
            t = ins[j][1]
            top, tops = operands(t)
            if top.startswith(("s_cbranch", "s_branch", "s_endpgm")) or ws >= SRCC_WAR_WAIT_STATES:
                break
            if tops and top.startswith(WRITERS) and regs(tops[0]) & c:
                assert False, (KERNELS[key], s, t, ws)
            ws += wait_states(t)
    if "int8" in KERNELS[key] or "fused" in KERNELS[key] or "scores" in KERNELS[key]:
        assert starts > 0, KERNELS[key]
