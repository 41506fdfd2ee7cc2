"""Instruction budget of the ring kernels' main loops (CPU only: hipcc compiles the kernels to
gfx950 assembly; nothing runs on a GPU).

A wave holding 256 accumulators has every register its SIMD offers one wave, so it is alone on
its SIMD, and whatever it issues besides the MFMAs competes with them for issue cycles.  These
checks pin each kernel's main loop: its instructions per MFMA, no spill traffic in it, and no
compiler wait for every memory operation in flight (which would drain the ring's loads)."""
import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from group_gemm_amd import build as B

# name: (source, mangled-name prefix of the instantiation, most instructions per MFMA allowed,
#        most scratch bytes per lane: spilled registers, whose reloads wait for every load in flight)
LOOPS = {
    "bf16 forward": ("ragged_m_bf16.hip", "_ZN2gg2mb6kernelILi256ELi2ELi3ELi4ELb0ELb0EtEE", 3.55, 128),
    "bf16 data gradient": ("ragged_m_bf16.hip", "_ZN2gg2mb6kernelILi256ELi2ELi3ELi4ELb1ELb0EtEE", 3.4, 64),
    "MXFP8 forward": ("ragged_m_mx.hip", "_ZN2gg2mx6kernelILb1ELb0EtEE", 8.5, 64),
    "weight gradient": ("ragged_k_bf16.hip", "_ZN2gg2kr6kernelILb0EfLb0EEE", 3.8, 0),
    "gated": ("ragged_m_gated.hip", "_ZN2gg2mg6kernelILi0EtEE", 3.5, 0),
}


@pytest.fixture(scope="module")
def asm():
    out = tempfile.mkdtemp(prefix="gg_isa_")
    srcs = sorted({v[0] for v in LOOPS.values()})

    def compile_one(src):
        dst = os.path.join(out, src + ".s")
        flags = [f for f in B.FLAGS if f != "-fPIC"]
        r = subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", dst],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, open(dst).read()

    with cf.ThreadPoolExecutor(len(srcs)) as ex:
        return dict(ex.map(compile_one, srcs))


def innermost_loops(text, prefix):
    """(label, instructions) of every innermost loop of the function: the blocks from a branch
    target up to a branch back to it, with no other such branch inside"""
    m = re.search(r"^(" + prefix + r"\w*):", text, re.M)
    assert m, prefix
    body = text[m.start():text.index(".Lfunc_end", m.start())].splitlines()
    blocks = []
    for raw in body:
        line = raw.strip()
        if line.startswith(".LBB") or line.startswith("; %bb"):
            blocks.append((line.split(":")[0], []))
        elif blocks and line and not line.startswith(";") and not line.startswith("."):
            blocks[-1][1].append(line)
    where = {label: i for i, (label, _) in enumerate(blocks)}
    spans = []
    for i, (_, ins) in enumerate(blocks):
        for x in ins:
            br = re.match(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", x)
            if br and where.get(br.group(1), i + 1) <= i:
                spans.append((where[br.group(1)], i))
    inner = [(a, b) for a, b in spans if not any((a, b) != (c, e) and a <= c and e <= b for c, e in spans)]
    return [(blocks[a][0], [x for _, ins in blocks[a:b + 1] for x in ins]) for a, b in inner]


@pytest.mark.parametrize("name", list(LOOPS))
def test_main_loop_budget(asm, name):
    src, prefix, budget, scratch = LOOPS[name]
    loops = innermost_loops(asm[src], prefix)
    assert loops, f"{name}: no loop found"
    nm = lambda ins: sum(1 for x in ins if x.startswith("v_mfma"))
    top = max(nm(ins) for _, ins in loops)
    assert top > 0, f"{name}: no MFMA in any loop"
    # the main loop: the loop with the most MFMAs and, among those, the fewest instructions
    label, ins = min(((l, i) for l, i in loops if nm(i) == top), key=lambda li: len(li[1]))
    ratio = len(ins) / top
    assert ratio <= budget, f"{name}: {len(ins)} instructions for {top} MFMAs ({ratio:.2f} per MFMA) in {label}"
    assert not any(x.startswith("scratch_") for x in ins), f"{name}: spill traffic in the main loop {label}"
    assert not any(re.match(r"s_waitcnt\s+vmcnt\(0\)", x) for x in ins), f"{name}: vmcnt(0) in the main loop {label}"
    m = re.search(r"^" + prefix + r"\w*:", asm[src], re.M)
    size = re.search(r"; ScratchSize: (\d+)", asm[src][asm[src].index(".Lfunc_end", m.start()):])
    assert size and int(size.group(1)) <= scratch, f"{name}: {size and size.group(1)} scratch bytes per lane"
