"""The M = 1 GEMV keeps six waves per SIMD and spills nothing.

The GEMV shares the SIMDs' vector instructions with its weight stream, and
its speed depends on six waves per SIMD hiding each other's latency: at most
80 VGPRs per lane (a SIMD holds 512).  Its registers are set by the compiler
from the load pipeline (two sets of weight loads taking the rounds in turn)
and the x staging, so a change to either can silently cost a wave, or spill
to scratch memory.  This compiles gemv.hip with the library's own flags and
reads the register counts and scratch sizes the compiler reports.  Runs on
the CPU (hipcc cross-compiles gfx950).
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

# kernel (mangled-name fragment) -> most VGPRs allowed
BUDGET = {
    "q4k_gemv_kernel": 80,          # six waves per SIMD
    "q4k_gemv_batched_kernel": 80,
    "q4k_gemv_swiglu_kernel": 96,   # five
    "q4k_gemv_rmsnorm_kernel": 128, # four (the norm's x registers)
}


def kernel_resources(tmp_path):
    out = tmp_path / "gemv.s"
    cmd = [jq4k_build.HIPCC, *jq4k_build.CFLAGS, *jq4k_build.EXTRA_FLAGS.get("gemv.hip", []),
           "--cuda-device-only", "-S", os.path.join(jq4k_build.CSRC, "gemv.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    res, name = {}, None
    for line in out.read_text().splitlines():
        f = line.split()
        if not f:
            continue
        if f[0] == ".amdhsa_kernel":
            name = f[1]
            res[name] = {}
        elif name and f[0] in (".amdhsa_next_free_vgpr", ".amdhsa_private_segment_fixed_size"):
            res[name][f[0]] = int(f[1])
        elif f[0] == ".end_amdhsa_kernel":
            name = None
    return res


def test_gemv_registers_and_scratch(tmp_path):
    res = kernel_resources(tmp_path)
    for frag, budget in BUDGET.items():
        hits = [k for k in res if frag in k]
        assert hits, f"no kernel named like {frag}"
        for k in hits:
            vgprs = res[k][".amdhsa_next_free_vgpr"]
            scratch = res[k][".amdhsa_private_segment_fixed_size"]
            assert scratch == 0, f"{k} spills {scratch} bytes to scratch"
            assert vgprs <= budget, f"{k} takes {vgprs} VGPRs, more than {budget}"
