"""Static check of the attention kernels' tile-loop barriers in the gfx950 assembly hipcc emits.

Each wave copies its share of the next K and V tiles into LDS (global->LDS loads counted by
vmcnt) and the other waves read those regions after the tile's workgroup barrier.  A wave must
therefore have waited for every copy it issued (vmcnt(0)) before it reaches the barrier: a
partial wait such as vmcnt(1) is only safe if the load left in flight was issued last, and the
compiler is free to reorder a tile's independent loads.  The test compiles fa_fwd.hip with the
library's flags and checks every barrier inside a loop of every attention kernel:
  * the nearest preceding wait on vector memory is vmcnt(0);
  * no global->LDS copy is issued between that wait and the barrier (one register load, the
    bitmask words of a later tile, may be).
CPU only (hipcc cross-compiles); skipped where hipcc is absent."""

import os
import re
import subprocess
import tempfile

import pytest

from attention_forward_fwd_amd import build


def _hipcc():
    try:
        return build.hipcc()
    except RuntimeError:
        return None


@pytest.fixture(scope="module")
def asm():
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "fa_fwd.s")
        cmd = [cc, *flags, "--cuda-device-only", "-S", f"-I{build.INCLUDE}", "-o", out, build.SOURCES[0]]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def _kernels(text):
    for m in re.finditer(r"^(_ZN\w*fa_fwd_kernel\w*):", text, re.M):
        end = text.find(".Lfunc_end", m.end())
        yield m.group(1), text[m.end():end].split("\n")


def _loop_barriers(lines):
    """Indices of s_barrier instructions in blocks that LLVM marks as part of a loop."""
    in_loop = False
    out = []
    for k, line in enumerate(lines):
        s = line.strip()
        if re.match(r"^\.LBB\w+:", line) or s.startswith("; %bb."):
            in_loop = "in Loop" in line or "Loop Header" in line
        elif s.startswith("s_barrier") and in_loop:
            out.append(k)
    return out


def _check_barrier(lines, k):
    issued = []
    for j in range(k - 1, -1, -1):
        s = lines[j].strip()
        if re.match(r"(buffer_load|global_load|buffer_store|global_store)", s):
            issued.append(s)
        m = re.match(r"s_waitcnt\b.*\bvmcnt\((\d+)\)", s)
        if m:
            n = int(m.group(1))
            dma = [x for x in issued if re.search(r"\blds\b", x) or x.startswith("global_load_lds")]
            loads = [x for x in issued if x.startswith(("buffer_load", "global_load"))]
            return n, dma, loads
    return None, [], []


def test_tile_loop_barriers_wait_for_every_copy(asm):
    checked = 0
    kernels = list(_kernels(asm))
    assert len(kernels) >= 48, f"expected every attention kernel instance, found {len(kernels)}"
    for name, lines in kernels:
        bars = _loop_barriers(lines)
        assert bars, f"{name}: no barrier found inside a loop"
        for k in bars:
            n, dma, loads = _check_barrier(lines, k)
            assert n == 0, f"{name}: barrier at line {k} follows s_waitcnt vmcnt({n})"
            assert not dma, f"{name}: barrier at line {k} follows a global->LDS copy issued after the wait: {dma}"
            assert len(loads) <= 1, f"{name}: barrier at line {k}: {len(loads)} loads issued after the wait"
            checked += 1
    assert checked >= 2 * len(kernels)
