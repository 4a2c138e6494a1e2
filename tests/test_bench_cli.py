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
    for name in ("single_leg", "decode_leg", "lm_head_leg", "prefill_leg", "m33_leg",
                 "lm_head_m512_leg", "swiglu_leg", "rmsnorm_leg", "kv_leg", "ceilings_leg",
                 "profile_run", "kernel_trace", "roofline", "cpu_baseline",
                 "cpu_baseline_prefill", "main"):
        assert callable(getattr(b, name)), name
    assert set(b.LEGS) >= {"single", "decode", "m33", "prefill", "lm_head", "lm_head_m512"}
    assert b.RW_KERNEL.startswith("jq4k::q4k_gemm_")


def test_roofline_object_from_events_and_trace():
    """The roofline object: achieved = algorithmic amount / event time per
    launch; with a current kernel-trace entry for the leg, trace_frac and the
    traffic (fetch + write bytes) come from it."""
    b = _bench_module()
    r = b.roofline("hbm", 8e9, 2.0, "k", "leg", {}, "bytes_per_launch")
    assert r["achieved"] == 4.0 and r["frac"] == round(4.0 / 8000.0, 4)
    assert r["trace_frac"] is None and r["traffic"] is None
    tr = {"leg": {"k": {"avg_us": 1e6, "fetch_bytes": 10, "write_bytes": 5}}}
    r = b.roofline("hbm", 8e9, 2.0, "k", "leg", tr, "bytes_per_launch")
    assert r["trace_avg_us"] == 1e6 and r["trace_frac"] == round(8.0 / 8000.0, 4)
    assert r["traffic"] == 15
    r = b.roofline("mfma", 5e15, 2.0, "k", "x", tr, "flops_per_launch")
    assert r["unit"] == "TFLOP/s" and r["frac"] == 1.0 and r["flops_per_launch"] == 5e15


def test_multi_gpu_request_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
