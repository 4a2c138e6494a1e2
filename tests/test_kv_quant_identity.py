"""The KV quantiser's codes without a division per value are the codes of
the definition, for every input a vector can hold.

kv_quant_kernel forms rint(v / s) as rint(q0 + (v - q0 s) y) with y = 1/s
rounded once, q0 = v y rounded and both corrections one fma each.  The
inputs of one value are only its binary16 v and the binary16 max |v| of its
vector, so the identity is checked exhaustively on the CPU over all of them
(kv_quant_identity.c: about 10^9 pairs, a few seconds on the host's cores).
The GPU's fp32 multiply, fma, division and rint are the IEEE operations the C
program uses (the kernels keep denormals; no value here is denormal in fp32).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")


def test_reciprocal_codes_equal_division_codes(tmp_path):
    exe = tmp_path / "kv_quant_identity"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe),
                    os.path.join(HERE, "kv_quant_identity.c"), "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    pairs, bad = (int(w) for w in out.stdout.split()[1::2])
    assert bad == 0 and pairs > 10**9, out.stdout
