"""Host checks of bench.py: its entry points exist and a multi-GPU request
exits with a message instead of running."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_entry_points_defined():
    b = _bench_module()
    for name in ("decode_leg", "lm_head_leg", "prefill_leg", "prefill_m33_leg", "lm_head_m512_leg", "swiglu_leg", "rmsnorm_leg",
                 "profile_run", "measured_traffic",
                 "cpu_baseline", "cpu_baseline_prefill", "main"):
        assert callable(getattr(b, name)), name
    assert b.PREFILL_KERNEL.startswith("jq4k::q4k_gemm_")


def test_multi_gpu_request_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
