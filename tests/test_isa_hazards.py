"""Static check of the compiled chunk kernels (gfx950 assembly, CPU only).

On gfx950 an MFMA whose accumulator input is the result of an MFMA of a
different shape (16x16x32 into 16x16x16, or back) needs at least five
independent issue slots between the two; chains of one shape are interlocked
by the hardware.  The compiler does not always insert those slots, and a
shorter gap silently reads a stale accumulator.  The kernels are written so
that no accumulator chain mixes shapes; this test compiles them and checks
the scheduled code, so that a change of source or compiler that brings such
a chain back within five slots fails here rather than as rare wrong results.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_prefill_amd", "csrc")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
MIN_SLOTS = 5


def _vrange(tok):
    m = re.match(r"^v\[(\d+):(\d+)\]$", tok)
    if m:
        return int(m.group(1)), int(m.group(2))
    m = re.match(r"^v(\d+)$", tok)
    return (int(m.group(1)),) * 2 if m else None


def _writes(line):
    """VGPR range written by a vector instruction (its first operand)."""
    parts = line.split(None, 1)
    if len(parts) < 2 or not parts[0].startswith(("v_", "ds_read", "global_load", "buffer_load")):
        return None
    if parts[0].startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
        return None
    return _vrange(parts[1].split(",")[0].strip())


def _overlap(a, b):
    return a is not None and b is not None and not (a[1] < b[0] or b[1] < a[0])


def mixed_chains(asm: str):
    """(kernel, slots, producer, consumer) for every MFMA whose accumulator
    input was last written by an MFMA of another opcode, scanning back within
    the basic block; slots counts issued instructions, s_nop N as N + 1."""
    found = []
    for m in re.finditer(r"\n(_Z\w+):", asm):
        end = asm.find(".Lfunc_end", m.end())
        lines = [l.strip() for l in asm[m.end():end].split("\n")
                 if l.strip() and not l.strip().startswith(";")]
        for i, line in enumerate(lines):
            if not line.startswith("v_mfma"):
                continue
            args = [t.strip() for t in line.split(None, 1)[1].split(",")]
            acc = _vrange(args[3])
            if acc is None:
                continue
            slots = 0
            for j in range(i - 1, -1, -1):
                prev = lines[j]
                if prev.startswith(".") or prev.startswith("s_cbranch") or prev.startswith("s_branch"):
                    break
                op = prev.split()[0]
                w = _writes(prev)
                if _overlap(w, acc):
                    if op.startswith("v_mfma") and op != line.split()[0]:
                        found.append((m.group(1), slots, op, line.split()[0]))
                    break
                slots += int(prev.split()[1]) + 1 if op == "s_nop" else 1
    return found


def _compile(src):
    # the per-source flags of the library build (the scheduler choice of the
    # pipelined kernel's four-slice units), so that the checked code is the
    # code that ships
    from gated_deltanet_prefill_amd.build import EXTRA
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", *EXTRA.get(src, []), "-I", os.path.join(ROOT, "include"),
           "-x", "hip", "--cuda-device-only", "-S", "-o", "-", os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


def test_scan_finds_a_planted_chain():
    """The scanner itself: a 16x16x32 result consumed by a 16x16x16 one slot
    later is reported, a same-shape chain and a far-apart one are not."""
    asm = "\n".join([
        "", "_Zkernel:",
        "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
        "v_add_u32_e32 v20, 1, v20",
        "v_mfma_f32_16x16x16_bf16 v[0:3], v[12:13], v[14:15], v[0:3]",
        "v_mfma_f32_16x16x32_bf16 v[16:19], v[4:7], v[8:11], v[16:19]",
        "v_mfma_f32_16x16x32_bf16 v[16:19], v[4:7], v[8:11], v[16:19]",
        "v_mfma_f32_16x16x32_bf16 v[24:27], v[4:7], v[8:11], 0",
        "s_nop 7",
        "v_mfma_f32_16x16x16_bf16 v[24:27], v[12:13], v[14:15], v[24:27]",
        ".Lfunc_end0:", ""])
    got = mixed_chains(asm)
    assert [(s, p, c) for _, s, p, c in got] == [
        (1, "v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16"),
        (8, "v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16")]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_close_mixed_shape_accumulator_chains():
    srcs = ["gdn_chunk_bf16.hip", "gdn_chunk_f16.hip", "gdn_chunk_f32.hip",
            "gdn_chunk_wy2_bf16.hip", "gdn_chunk_wy2_f16.hip",
            "gdn_chunk_vg_bf16.hip", "gdn_chunk_vg_f16.hip", "gdn_chunk_vg_f32.hip"]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        asms = list(ex.map(_compile, srcs))
    bad = [(src, k[:70], s, p, c) for src, asm in zip(srcs, asms)
           for k, s, p, c in mixed_chains(asm) if s < MIN_SLOTS]
    assert not bad, f"MFMA accumulator chains across shapes closer than {MIN_SLOTS} slots: {bad}"
