"""The register-W matmul's explicit waits cover the X copies they stand for.

gemm_rw.hip copies X from global memory straight into LDS and, before the
barrier between a stage's halves, waits with `s_waitcnt vmcnt(N) lgkmcnt(0)`
until the copy of the next stage has landed.  The copy was issued two copy
groups back; N must be at most the number of memory instructions issued after
it, or the barrier can open with that copy still in flight.  N is written by
hand from the issue order, and the compiler may drop or move loads (it drops
loads whose results are dead), so the count is checked here against the
instructions the compiler actually emits, with the library's own flags.
Runs on the CPU (hipcc cross-compiles gfx950).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "q4_weight_only_amd"))
import build as jq4k_build  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(jq4k_build.HIPCC),
                                reason="hipcc is not installed")

COPY_GROUP = 8   # X copy instructions per wave per stage (kRwXChunks)


def device_asm(src, tmp_path):
    out = tmp_path / "k.s"
    cmd = [jq4k_build.HIPCC, *jq4k_build.CFLAGS, *jq4k_build.EXTRA_FLAGS.get(src, []),
           "--cuda-device-only", "-S", os.path.join(jq4k_build.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return [l.strip() for l in out.read_text().splitlines()
            if l.strip() and not l.strip().startswith((";", "."))]


def test_register_w_waits_cover_the_copy(tmp_path):
    lines = device_asm("gemm_rw.hip", tmp_path)
    kinds, waits = [], []
    for l in lines:
        op = l.split()[0]
        if op.startswith("buffer_load") and " lds" in l:
            kinds.append("copy")
        elif op.startswith(("global_load", "buffer_load", "global_store", "buffer_store",
                            "flat_")):
            kinds.append("mem")
        elif op == "s_waitcnt" and "vmcnt(" in l and "lgkmcnt(0)" in l:
            waits.append((len(kinds), int(l.split("vmcnt(")[1].split(")")[0])))
    # copy instruction k belongs to group k // COPY_GROUP
    group, ncopy = [], 0
    for k in kinds:
        group.append(ncopy // COPY_GROUP if k == "copy" else None)
        ncopy += k == "copy"
    assert ncopy % COPY_GROUP == 0
    checked = 0
    for pos, n in waits:
        groups = [g for g in group[:pos] if g is not None]
        if len(groups) < 2 * COPY_GROUP:
            continue   # the prologue's copies, waited for by a full count
        target = max(groups) - 1
        last = max(i for i, g in enumerate(group[:pos]) if g == target)
        after = pos - 1 - last
        assert n <= after, (f"vmcnt({n}) before a barrier, but only {after} memory "
                            f"instructions follow the copy it waits for")
        checked += 1
    # one wait per stage, four stages per iteration of the main loop
    assert checked >= 4
