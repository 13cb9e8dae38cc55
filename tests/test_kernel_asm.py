"""Checks on the gfx950 assembly of the library's kernels (compiled here with
the library's own flags; no GPU needed).

A 16x16x16 bf16 MFMA that took its accumulator from the result of a
16x16x32 bf16 MFMA issued just before it (only an s_waitcnt between them,
which the compiler treats as enough for an exactly overlapping accumulator)
returned wrong values in two of the four result rows on gfx950.  No kernel may
feed one MFMA shape's result into another shape's accumulator with fewer than
MIN_WAIT wait states between them."""
import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from weight_recurrent_sequence_amd import _build

MIN_WAIT = 8
MFMA = re.compile(r"^(v_mfma\w*)\s+([va]\[\d+:\d+\]|[va]\d+),\s*(\S+),\s*(\S+),\s*([va]\[\d+:\d+\]|[va]\d+|0)")


def regs(r):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", r)
    if m:
        return m.group(1), int(m.group(2)), int(m.group(3))
    m = re.match(r"([va])(\d+)$", r)
    return (m.group(1), int(m.group(2)), int(m.group(2))) if m else None


def overlap(a, b):
    return a is not None and b is not None and a[0] == b[0] and not (a[2] < b[1] or b[2] < a[1])


def mixed_chains(asm):
    """(kernel, producer, consumer, wait states) of every accumulator handed
    from one MFMA opcode to another within MIN_WAIT wait states, in program
    order within each function."""
    found, fn, hist, clock = [], None, [], 0
    for line in asm.split("\n"):
        if re.match(r"^_Z\w+:", line):
            fn, hist, clock = line.split(":")[0], [], 0
            continue
        t = line.strip()
        if not t or t[0] in ";." or t.endswith(":"):
            continue
        m = MFMA.match(t)
        if m and fn:
            op, dst, src_c = m.group(1), regs(m.group(2)), regs(m.group(5))
            for end, pop, pdst in reversed(hist):
                if overlap(pdst, src_c):
                    if pop != op and clock - end - 1 < MIN_WAIT:
                        found.append((fn, pop, op, clock - end - 1))
                    break
            hist = (hist + [(clock, op, dst)])[-32:]
        clock += int(t.split()[1], 0) + 1 if t.startswith("s_nop") else 1
    return found


def test_scanner_finds_a_planted_chain():
    asm = ("_Zkernel:\n"
           "\tv_mfma_f32_16x16x32_bf16 v[2:5], v[6:9], v[10:13], v[2:5]\n"
           "\ts_waitcnt lgkmcnt(0)\n"
           "\tv_mfma_f32_16x16x16_bf16 v[2:5], v[14:15], v[16:17], v[2:5]\n"
           "\tv_mfma_f32_16x16x32_bf16 v[20:23], v[6:9], v[10:13], v[20:23]\n"
           "\ts_nop 7\n"
           "\tv_mfma_f32_16x16x16_bf16 v[20:23], v[14:15], v[16:17], v[20:23]\n"
           "\tv_mfma_f32_16x16x32_bf16 v[30:33], v[6:9], v[10:13], 0\n"
           "\tv_mfma_f32_16x16x32_bf16 v[30:33], v[6:9], v[10:13], v[30:33]\n")
    assert mixed_chains(asm) == [("_Zkernel", "v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16", 1)]


@pytest.fixture(scope="module")
def device_asm():
    srcs = sorted(f for f in os.listdir(_build.CSRC) if f.endswith(".hip") and f in _build.SOURCES)
    assert srcs
    with tempfile.TemporaryDirectory() as d:
        def compile_one(src):
            out = os.path.join(d, src + ".s")
            cmd = [_build.hipcc(), *_build.flags(), "--cuda-device-only", "-S",
                   os.path.join(_build.CSRC, src), "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            return src, open(out).read()
        with cf.ThreadPoolExecutor(len(srcs)) as ex:
            return dict(ex.map(compile_one, srcs))


def test_no_mixed_mfma_accumulator_chains(device_asm):
    bad = {src: mixed_chains(asm) for src, asm in device_asm.items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, bad


def test_every_kernel_has_mfma_code(device_asm):
    # the scan above sees the kernels' MFMA code at all
    assert sum(len(re.findall(r"\bv_mfma_", a)) for a in device_asm.values()) > 100
