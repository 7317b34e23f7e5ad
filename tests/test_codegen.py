"""The compiled kernels keep the code shape they were tuned for: the
prefill kernel's matrix-phase operand pipeline, and no register spills in
any prefill or backward kernel beyond the few bytes listed below.

The steady matrix phase of the ping-pong prefill kernel issues 32 MFMAs,
each with its A operand (a K or V fragment) read from LDS a few MFMAs
ahead into its own registers.  If the scheduler drops that order, every
MFMA takes its operand from the same four registers and waits for the
read before it (``s_waitcnt lgkmcnt(0)``): same results, about 20 % slower.
This has happened after unrelated edits, so the gfx950 assembly of the
kernel (compiled here, on the CPU) is checked: every basic block with 32
MFMAs and no exponentials must draw its A operands from several register
ranges and wait for the LDS only a few times in full.
"""
import os
import re
import subprocess
import tempfile

import pytest

from exact_attention_09_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "exact_attention_09_amd", "csrc", "attn_prefill_pp.hip")
MFMA = re.compile(r"^\s+v_mfma_f32_32x32x16_bf16 \S+, (v\[\d+:\d+\])")


def _functions(asm: str):
    """(template arguments, list of basic blocks as line lists) per kernel."""
    out = {}
    for m in re.finditer(r"^(_ZN4attn\S*prefill_pp_kernel\S*):\s*;", asm, re.M):
        name = m.group(1)
        end = asm.index(".Lfunc_end", m.end())
        body = asm[m.end():end].split("\n")
        blocks, cur = [], []
        for line in body:
            if re.match(r"^\.LBB\d+_\d+:", line):
                blocks.append(cur)
                cur = []
            else:
                cur.append(line)
        blocks.append(cur)
        args = re.search(r"kernelI(.*)EEvNS", name).group(1)
        out[args.replace("Li", "").replace("ELb", ",").replace("E", "")] = blocks
    return out


@pytest.fixture(scope="module")
def prefill_asm():
    try:
        cc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "pp.s")
        cmd = [cc, *[f for f in b.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S", SRC, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def test_matrix_phase_operand_ring(prefill_asm):
    funcs = _functions(prefill_asm)
    assert len(funcs) == 24, sorted(funcs)  # d x causal x varlen x window x layout
    checked = 0
    for args, blocks in funcs.items():
        for blk in blocks:
            srcs = [m.group(1) for m in map(MFMA.match, blk) if m]
            if len(srcs) != 32 or any("v_exp_f32" in line for line in blk):
                continue
            full_waits = sum("lgkmcnt(0)" in line for line in blk)
            assert len(set(srcs)) >= 4 and full_waits <= 4, (
                f"prefill_pp_kernel<{args}>: a steady matrix phase takes its A operands from "
                f"{len(set(srcs))} register ranges and waits for the LDS in full {full_waits} times "
                "(the operand reads are no longer issued ahead of the MFMAs)")
            checked += 1
    assert checked >= 48, checked  # several steady matrix phases per instantiation


def _scratch(asm: str):
    """Private (scratch) bytes per kernel from the code object metadata."""
    out = {}
    for block in asm.split("- .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        size = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        if name and size:
            out[name.group(1)] = int(size.group(1))
    return out


@pytest.fixture(scope="module")
def backward_asm():
    try:
        cc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = os.path.join(ROOT, "exact_attention_09_amd", "csrc", "attn_backward.hip")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "bwd.s")
        cmd = [cc, *[f for f in b.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def test_no_register_spills(prefill_asm, backward_asm):
    """Every prefill and backward kernel keeps its values in registers: a
    spill to scratch memory in a tile loop has cost 4-70 % before.  A few
    instantiations are allowed the bytes they have long had, none of them in
    a tile loop: the packed-sequence d = 128 prefill kernels (12 bytes: two
    values stored at setup and reloaded once per item, in the item lookup)
    and the windowed d = 128 dQ kernels (one value outside the key-tile
    loop; in the packed-sequence one, one 8-byte reload per tile)."""
    spills = {**_scratch(prefill_asm), **_scratch(backward_asm)}
    assert len(spills) >= 24 + 24, f"kernels found: {len(spills)}"
    allowed = {"prefill_pp_kernelILi128ELb1ELb1ELb0E": 12, "prefill_pp_kernelILi128ELb0ELb1ELb0E": 12,
               "dq_kernelILi128ELb1ELb0ELb1E": 8, "dq_kernelILi128ELb1ELb1ELb1E": 16}
    for name, size in spills.items():
        limit = next((v for k, v in allowed.items() if k in name), 0)
        assert size <= limit, f"{name}: {size} bytes of scratch (allowed {limit})"
