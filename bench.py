"""Benchmark of the Q4_K weight-only matmul on one MI355X.

Headline (value): M = 1 weight bandwidth over one Qwen3-4B decode layer -- the
seven Q4_K projections q, k, v, o, gate, up, down at one token, each a GEMV
(0.5625 bytes per weight), one grouped launch per step (the synthetic inputs
of the seven are independent).  The same layer in dependency order (q|k|v,
o, gate|up, down: four launches) is reported beside it as the decode-step
figure.  Every other workload of the benchmark suite is a leg of the same
run: the single 2560 x 2560 GEMV, the 33-token prefill through 36 layers,
the 2048-token layer, the LM head at M = 1 and M = 512, the fused SwiGLU and
RMSNorm variants, the KV-cache convert, and the measured ceilings of this
GPU (streaming reads in two patterns and a matrix-instruction loop).

Protocol.  Inputs are seeded synthetic tensors resident in HBM before timing.
Weights rotate over enough identical copies (>= 1 GiB) that no step finds its
weights in the 256 MB last-level cache.  W warm-up steps run untimed; the K
timed steps are captured in a HIP graph (launch overhead out of the timed
region, kernels back to back) and bracketed by HIP events recorded on the
stream the kernels run on.  Kernel-trace durations of the same kernels, from
a rocprofv3 run of `bench.py --profile` kept under profiles/, are reported
beside the event times while the kernel sources are unchanged.  The CPU
oracle is timed on a bounded sample of the same workloads (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--prefill-steps P] [--no-cpu]
                    [--only LEG,...] [--profile]
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import q4k_inputs as qi  # noqa: E402

METRIC = "Q4_K matmul: M=1 weight GB/s (% HBM peak); M=2048 TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
BYTES_PER_WEIGHT = 144 / 256
ROTATION_BYTES = 1 << 30
DEPENDENCY_GROUPS = [[0, 1, 2], [3], [4, 5], [6]]   # q|k|v, o, gate|up, down

# The kernel each timed leg's launches run (for the kernel-trace lookup).
GEMV_KERNEL = "jq4k::q4k_gemv_kernel"
GEMV_BATCHED_KERNEL = "jq4k::q4k_gemv_batched_kernel"
RW_KERNEL = "jq4k::q4k_gemm_rw_kernel"
# Untimed launches before a matrix-core leg's timed ones: after the leg's
# set-up the GPU needs a few hundred microseconds of load to reach its
# sustained clock (the M = 2048 layer measured 483 us per launch over 10
# steps after 2 warm-up launches, 422 us over 40).
MFMA_WARMUP = 10
SKINNY_KERNEL = "jq4k::q4k_gemm_skinny_kernel<3>"
# Marker launches of the probe kernel separate the legs of a --profile run:
# a read of 16 bytes with PROFILE_MARKER + leg index workgroups.
PROFILE_MARKER = 1000
PROFILE_LEGS = ["copy_512MiB", "single", "decode", "lm_head", "m33", "prefill", "lm_head_m512",
                "warmup"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=30)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches, no graph")
    ap.add_argument("--only", default="",
                    help="comma-separated legs to time (single,decode,lm_head,m33,prefill,"
                         "lm_head_m512,swiglu,rmsnorm,kv,ceilings); prints them as one JSON "
                         "object instead of the benchmark line")
    ap.add_argument("--profile", action="store_true",
                    help="a few eager launches of each measured kernel for rocprofv3, legs "
                         "separated by marker launches; no JSON line")
    return ap.parse_args()


def graph_ok(args, graph):
    """Whether a leg replays its launches from a HIP graph (the default).
    The M = 1 LM head is timed eagerly: its graph replays measured ~8 us per
    launch longer than eager launches and than its kernel trace (45.6 us),
    while launch overhead at that length is negligible.  The matrix-core
    legs measure the same either way."""
    return graph and not args.eager


def timed(torch, fn, steps, warmup, use_graph):
    """Run fn(i) for warm-up, then time `steps` calls; returns seconds."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    if use_graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(steps):
                    fn(warmup + i)
        torch.cuda.synchronize()
        g.replay()                              # first replay uploads the graph
        torch.cuda.synchronize()
        run = g.replay
    else:
        def run():
            for i in range(steps):
                fn(warmup + i)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    run()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3


def stream_ptr(torch):
    return torch.cuda.current_stream().cuda_stream


def check(jq4k, rc):
    if rc:
        raise RuntimeError(jq4k.strerror(rc))


def copies_for(nbytes):
    return max(2, math.ceil(ROTATION_BYTES / nbytes))


def to_dev(torch, a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda:0")


# ---------------------------------------------------------------- traces

def kernel_trace():
    """Per-leg kernel-trace averages (and traffic) from
    profiles/kernel_trace.json, or {} when the file is missing or was taken on
    other kernel sources."""
    from profile_summary import kernel_source_hash
    path = os.path.join(ROOT, "profiles", "kernel_trace.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        doc = json.load(f)
    if doc.get("kernel_sources_sha256") != kernel_source_hash():
        return {}
    return doc.get("legs", {})


def roofline(bound, amount, seconds_per_launch, kernel, leg, traces, unit_amount):
    """Roofline object: `amount` algorithmic bytes (hbm) or flops (mfma) per
    launch of `kernel`; achieved from the event time per launch, and from the
    kernel-trace average of the same leg when it is current."""
    peak, unit = (HBM_PEAK_GBS, "GB/s") if bound == "hbm" else (MFMA_BF16_PEAK_TFLOPS, "TFLOP/s")
    scale = 1e9 if bound == "hbm" else 1e12
    achieved = amount / seconds_per_launch / scale
    out = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4), "traffic": None, "kernel": kernel,
           "avg_launch_us": round(seconds_per_launch * 1e6, 3), unit_amount: amount,
           "trace_avg_us": None, "trace_frac": None}
    t = traces.get(leg, {}).get(kernel)
    if t:
        out["trace_avg_us"] = t["avg_us"]
        out["trace_frac"] = round(amount / (t["avg_us"] * 1e-6) / scale / peak, 4)
        if t.get("fetch_bytes") is not None and t.get("write_bytes") is not None:
            out["traffic"] = t["fetch_bytes"] + t["write_bytes"]
    return out


# ------------------------------------------------------------------- legs

def single_leg(torch, jq4k, args, traces):
    """The single 2560 x 2560 Q4_K GEMV at M = 1 (seed 0), rotated over copies
    (3.7 MB each, >= 1 GiB in all)."""
    W, X = qi.single_gemv(0)
    N = K = 2560
    copies = copies_for(W.nbytes)
    Wd = [to_dev(torch, W)]
    Wd += [Wd[0].clone() for _ in range(copies - 1)]
    Xd = to_dev(torch, X.view(np.int16))
    Yd = torch.empty(N, dtype=torch.float32, device="cuda:0")
    L = jq4k.raw()

    def one(i):
        check(jq4k, L.jq4k_gemv(Wd[i % copies].data_ptr(), Xd.data_ptr(), Yd.data_ptr(), 1, N,
                                K, stream_ptr(torch)))
    t = timed(torch, one, args.steps, args.warmup, not args.eager) / args.steps
    return {"workload": "single Q4_K GEMV, N=2560 x K=2560, M=1, seed 0; one jq4k_gemv "
                        "launch per step", "N": N, "K": K, "weight_bytes": int(W.nbytes),
            "rotation_copies": copies, "us": round(t * 1e6, 3),
            "GB_s": round(W.nbytes / t / 1e9, 1),
            "roofline": roofline("hbm", int(W.nbytes), t, GEMV_KERNEL, "single", traces,
                                 "bytes_per_launch")}


def decode_leg(torch, jq4k, args, traces):
    """Seven Q4_K GEMVs of one decode layer, timed three ways:
    batched_1     one jq4k_gemv_batched launch for all seven (independent in
                  this workload) -- the headline value;
    dependency_4  the launches a real decode step makes (q|k|v, o, gate|up,
                  down: later groups consume earlier outputs);
    separate_7    seven jq4k_gemv launches;
    and each projection alone."""
    layer = qi.decode_layer(1, 0, 1)
    layer_bytes = sum(W.nbytes for _, _, _, W, _ in layer)
    copies = copies_for(layer_bytes)
    Ws = [[to_dev(torch, W) for _, _, _, W, _ in layer]]
    for _ in range(copies - 1):
        Ws.append([w.clone() for w in Ws[0]])
    Xs = [to_dev(torch, X.view(np.int16)) for _, _, _, _, X in layer]
    Ys = [torch.empty((1, N), dtype=torch.float32, device="cuda:0") for _, N, _, _, _ in layer]
    L = jq4k.raw()

    def descs(c, idx):
        arr = (jq4k.GemvDesc * len(idx))()
        for j, p in enumerate(idx):
            _, N, K, _, _ = layer[p]
            arr[j] = jq4k.GemvDesc(Ws[c][p].data_ptr(), Xs[p].data_ptr(), Ys[p].data_ptr(), N, K)
        return arr
    all7 = [descs(c, range(7)) for c in range(copies)]
    grouped = [[descs(c, gi) for gi in DEPENDENCY_GROUPS] for c in range(copies)]

    def step_batched(i):
        check(jq4k, L.jq4k_gemv_batched(ctypes.addressof(all7[i % copies]), 7, stream_ptr(torch)))

    def step_grouped(i):
        s = stream_ptr(torch)
        for arr, gi in zip(grouped[i % copies], DEPENDENCY_GROUPS):
            check(jq4k, L.jq4k_gemv_batched(ctypes.addressof(arr), len(gi), s))

    def step_separate(i):
        Wc = Ws[i % copies]
        s = stream_ptr(torch)
        for p, (_, N, K, _, _) in enumerate(layer):
            check(jq4k, L.jq4k_gemv(Wc[p].data_ptr(), Xs[p].data_ptr(), Ys[p].data_ptr(), 1, N,
                                    K, s))

    graph = not args.eager
    secs = timed(torch, step_batched, args.steps, args.warmup, graph)
    modes = {}
    for name, fn, launches in (("batched_1", None, 1), ("dependency_4", step_grouped, 4),
                               ("separate_7", step_separate, 7)):
        t = secs if fn is None else timed(torch, fn, args.steps, args.warmup, graph)
        gbs = layer_bytes * args.steps / t / 1e9
        modes[name] = {"launches_per_step": launches, "us_per_step": round(t / args.steps * 1e6, 2),
                       "GB_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    per_proj = {}
    for p, (name, N, K, W, _) in enumerate(layer):
        def one(i, p=p, N=N, K=K):
            check(jq4k, L.jq4k_gemv(Ws[i % copies][p].data_ptr(), Xs[p].data_ptr(),
                                    Ys[p].data_ptr(), 1, N, K, stream_ptr(torch)))
        t = timed(torch, one, args.steps, 4, graph)
        per_proj[name] = {"N": N, "K": K, "us": round(t / args.steps * 1e6, 3),
                          "GB_s": round(W.nbytes * args.steps / t / 1e9, 1)}
    t1 = secs / args.steps
    return {"workload": "Qwen3-4B decode layer, 7 Q4_K projections at M=1 (q 4096x2560, "
                        "k/v 1024x2560, o 2560x4096, gate/up 9728x2560, down 2560x9728), "
                        "seeds [1,0,p]",
            "weight_bytes_per_step": layer_bytes, "rotation_copies": copies,
            "us": round(t1 * 1e6, 3), "GB_s": round(layer_bytes / t1 / 1e9, 1),
            "modes": modes, "per_projection": per_proj,
            "roofline": roofline("hbm", layer_bytes, t1, GEMV_BATCHED_KERNEL, "decode", traces,
                                 "bytes_per_launch")}


def lm_head_leg(torch, jq4k, args, traces):
    """The 151936 x 2560 Q4_K LM head at M = 1: one 219 MB GEMV, rotated over
    five copies."""
    W, X = qi.lm_head(4, 1)
    N, K = 151936, 2560
    copies = copies_for(W.nbytes)
    Wd = [to_dev(torch, W)]
    Wd += [Wd[0].clone() for _ in range(copies - 1)]
    Xd = to_dev(torch, X.view(np.int16))
    Yd = torch.empty(N, dtype=torch.float32, device="cuda:0")
    L = jq4k.raw()

    def one(i):
        check(jq4k, L.jq4k_gemv(Wd[i % copies].data_ptr(), Xd.data_ptr(), Yd.data_ptr(), 1, N, K,
                                stream_ptr(torch)))
    steps = max(10, args.steps // 10)
    t = timed(torch, one, steps, 3, graph_ok(args, False)) / steps
    return {"workload": "Qwen3-4B-shaped LM head as Q4_K, N=151936 x K=2560, M=1, seed 4",
            "N": N, "K": K, "weight_bytes": int(W.nbytes), "rotation_copies": copies,
            "launch": "eager" if not graph_ok(args, False) else "hip-graph",
            "us": round(t * 1e6, 2), "GB_s": round(W.nbytes / t / 1e9, 1),
            "roofline": roofline("hbm", int(W.nbytes), t, GEMV_KERNEL, "lm_head", traces,
                                 "bytes_per_launch")}


def prefill_leg(torch, jq4k, args, traces):
    """The seven projections of one layer at M = 2048 tokens on the MFMA path,
    W rotated over copies (>= 1 GiB), timed as batched_1 (one
    jq4k_gemm_batched launch; the prefill figure), dependency_4 and
    separate_7, and each projection alone."""
    M = 2048
    projs = [qi.prefill_projection(3, 0, p, M) for p in range(7)]
    flops = sum(2.0 * M * N * K for _, N, K, _, _ in projs)
    wbytes = sum(W.nbytes for _, _, _, W, _ in projs)
    copies = copies_for(wbytes)
    Ws = [[to_dev(torch, W) for _, _, _, W, _ in projs]]
    for _ in range(copies - 1):
        Ws.append([w.clone() for w in Ws[0]])
    Xs = [to_dev(torch, X.view(np.int16)) for _, _, _, _, X in projs]
    Ys = [torch.empty((M, N), dtype=torch.float32, device="cuda:0") for _, N, _, _, _ in projs]
    L = jq4k.raw()

    def descs(c, idx):
        arr = (jq4k.GemmDesc * len(idx))()
        for j, p in enumerate(idx):
            _, N, K, _, _ = projs[p]
            arr[j] = jq4k.GemmDesc(Ws[c][p].data_ptr(), Xs[p].data_ptr(), Ys[p].data_ptr(),
                                   M, N, K)
        return arr
    all7 = [descs(c, range(7)) for c in range(copies)]
    grouped = [[descs(c, gi) for gi in DEPENDENCY_GROUPS] for c in range(copies)]

    def step_batched(i):
        check(jq4k, L.jq4k_gemm_batched(ctypes.addressof(all7[i % copies]), 7, stream_ptr(torch)))

    def step_grouped(i):
        s = stream_ptr(torch)
        for arr, gi in zip(grouped[i % copies], DEPENDENCY_GROUPS):
            check(jq4k, L.jq4k_gemm_batched(ctypes.addressof(arr), len(gi), s))

    def step_separate(i):
        Wc = Ws[i % copies]
        s = stream_ptr(torch)
        for p, (_, N, K, _, _) in enumerate(projs):
            check(jq4k, L.jq4k_gemm(Wc[p].data_ptr(), Xs[p].data_ptr(), Ys[p].data_ptr(), M, N,
                                    K, s))

    graph = graph_ok(args, True)
    steps = args.prefill_steps
    secs = timed(torch, step_batched, steps, MFMA_WARMUP, graph)
    modes = {}
    for name, fn, launches in (("batched_1", None, 1), ("dependency_4", step_grouped, 4),
                               ("separate_7", step_separate, 7)):
        t = secs if fn is None else timed(torch, fn, steps, MFMA_WARMUP, graph)
        modes[name] = {"launches_per_step": launches, "us_per_step": round(t / steps * 1e6, 1),
                       "TFLOP_s": round(flops * steps / t / 1e12, 1)}
    per_proj = {}
    for p, (name, N, K, _, _) in enumerate(projs):
        def one(i, p=p, N=N, K=K):
            check(jq4k, L.jq4k_gemm(Ws[i % copies][p].data_ptr(), Xs[p].data_ptr(),
                                    Ys[p].data_ptr(), M, N, K, stream_ptr(torch)))
        t = timed(torch, one, steps, MFMA_WARMUP, graph)
        per_proj[name] = {"N": N, "K": K, "us": round(t / steps * 1e6, 2),
                          "TFLOP_s": round(2.0 * M * N * K * steps / t / 1e12, 1)}
    t1 = secs / steps
    return {"workload": "Qwen3-4B layer, 7 Q4_K projections at M=2048, seeds [3,0,p]; one "
                        "jq4k_gemm_batched launch per step (the seven are independent here)",
            "value": round(flops / t1 / 1e12, 1), "unit": "TFLOP/s", "steps": steps,
            "ms_per_step": round(t1 * 1e3, 4), "rotation_copies": copies,
            "roofline": roofline("mfma", flops, t1, RW_KERNEL, "prefill", traces,
                                 "flops_per_launch"),
            "modes": modes, "per_projection": per_proj}


def m33_leg(torch, jq4k, args, traces):
    """M = 33 through all 36 layers' seven projections (252 matmuls, 2.04 GB of
    Q4_K weights, child seeds [2, layer, p]): one jq4k_gemm_batched_ws launch
    per layer (split K), 36 per pass, one workspace reused layer after layer.
    HBM-bound: the attainable roofline counts W, X and Y bytes at 8 TB/s.  The
    same pass through jq4k_gemm_batched (whole K per tile) is timed beside
    it."""
    M, L = 33, jq4k.raw()
    keep, arrs = [], []
    wbytes = xybytes = flops = 0
    for layer in range(36):
        arr = (jq4k.GemmDesc * 7)()
        for p in range(7):
            _, N, K, W, X = qi.prefill_projection(2, layer, p, M)
            Wd = to_dev(torch, W)
            Xd = to_dev(torch, X.view(np.int16))
            Yd = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
            keep.append((Wd, Xd, Yd))
            arr[p] = jq4k.GemmDesc(Wd.data_ptr(), Xd.data_ptr(), Yd.data_ptr(), M, N, K)
            wbytes += W.nbytes
            xybytes += X.nbytes + M * N * 4
            flops += 2.0 * M * N * K
        arrs.append(arr)
    need = ctypes.c_size_t(0)
    check(jq4k, L.jq4k_gemm_workspace_size(ctypes.addressof(arrs[0]), 7, ctypes.byref(need)))
    ws = torch.zeros(max(need.value, 256), dtype=torch.uint8, device="cuda:0")

    def pass_ws(i):
        s = stream_ptr(torch)
        for arr in arrs:
            check(jq4k, L.jq4k_gemm_batched_ws(ctypes.addressof(arr), 7, ws.data_ptr(),
                                               ws.numel(), s))

    def pass_whole_k(i):
        s = stream_ptr(torch)
        for arr in arrs:
            check(jq4k, L.jq4k_gemm_batched(ctypes.addressof(arr), 7, s))
    steps = max(3, args.prefill_steps // 2)
    t = timed(torch, pass_ws, steps, 1, not args.eager) / steps
    t_whole = timed(torch, pass_whole_k, steps, 1, not args.eager) / steps
    allb = wbytes + xybytes
    rl = roofline("hbm", allb / 36, t / 36, SKINNY_KERNEL, "m33", traces, "bytes_per_launch")
    rl["bytes_per_pass"] = allb
    return {"workload": "Qwen3-4B cold prefill, M=33 through 36 layers x 7 Q4_K projections "
                        "(252 matmuls), seeds [2,l,p]; one jq4k_gemm_batched_ws (split-K) "
                        "launch per layer",
            "launches_per_pass": 36, "us_per_pass": round(t * 1e6, 1),
            "workspace_bytes": int(need.value), "weight_GB_s": round(wbytes / t / 1e9, 1),
            "roofline": rl, "TFLOP_s": round(flops / t / 1e12, 2),
            "whole_k_us_per_pass": round(t_whole * 1e6, 1)}


def lm_head_m512_leg(torch, jq4k, args, traces):
    """The 151936 x 2560 Q4_K LM head at M = 512 (a prefill chunk): one
    jq4k_gemm launch, MFMA-bound, W rotated over five copies."""
    W, X = qi.lm_head(4, 512)
    N, K, M = 151936, 2560, 512
    copies = copies_for(W.nbytes)
    Wd = [to_dev(torch, W)]
    Wd += [Wd[0].clone() for _ in range(copies - 1)]
    Xd = to_dev(torch, X.view(np.int16))
    Yd = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    L = jq4k.raw()

    def one(i):
        check(jq4k, L.jq4k_gemm(Wd[i % copies].data_ptr(), Xd.data_ptr(), Yd.data_ptr(), M, N, K,
                                stream_ptr(torch)))
    steps = max(5, args.prefill_steps)
    t = timed(torch, one, steps, MFMA_WARMUP, graph_ok(args, True)) / steps
    flops = 2.0 * M * N * K
    return {"workload": "Qwen3-4B-shaped LM head as Q4_K, N=151936 x K=2560, M=512, seed 4",
            "N": N, "K": K, "M": M, "rotation_copies": copies, "us": round(t * 1e6, 1),
            "TFLOP_s": round(flops / t / 1e12, 1),
            "roofline": roofline("mfma", flops, t, RW_KERNEL, "lm_head_m512", traces,
                                 "flops_per_launch")}


def swiglu_leg(torch, jq4k, args, traces):
    """gate|up of a layer with the SwiGLU epilogue fused (jq4k_gemm_swiglu):
    M = 1 (the decode gate/up) and M = 2048, weights rotated over copies;
    beside each, the same two matmuls as one grouped launch without the
    epilogue."""
    L = jq4k.raw()
    out = {}
    for M, seed in ((1, 1), (2048, 3)):
        if M == 1:
            layer = qi.decode_layer(1, 0, 1)
            (_, N, K, Wg, X), (_, _, _, Wu, _) = layer[4], layer[5]
        else:
            _, N, K, Wg, X = qi.prefill_projection(seed, 0, 4, M)
            _, _, _, Wu, _ = qi.prefill_projection(seed, 0, 5, M)
        wbytes = Wg.nbytes + Wu.nbytes
        copies = copies_for(wbytes)
        Wgs = [to_dev(torch, Wg)]
        Wus = [to_dev(torch, Wu)]
        for _ in range(copies - 1):
            Wgs.append(Wgs[0].clone())
            Wus.append(Wus[0].clone())
        Xd = to_dev(torch, X.view(np.int16))
        H = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        Yg = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        Yu = torch.empty((M, N), dtype=torch.float32, device="cuda:0")

        def fused(i):
            check(jq4k, L.jq4k_gemm_swiglu(Wgs[i % copies].data_ptr(), Wus[i % copies].data_ptr(),
                                           Xd.data_ptr(), H.data_ptr(), M, N, K,
                                           stream_ptr(torch)))
        descs = []
        for c in range(copies):
            if M == 1:
                arr = (jq4k.GemvDesc * 2)()
                arr[0] = jq4k.GemvDesc(Wgs[c].data_ptr(), Xd.data_ptr(), Yg.data_ptr(), N, K)
                arr[1] = jq4k.GemvDesc(Wus[c].data_ptr(), Xd.data_ptr(), Yu.data_ptr(), N, K)
            else:
                arr = (jq4k.GemmDesc * 2)()
                arr[0] = jq4k.GemmDesc(Wgs[c].data_ptr(), Xd.data_ptr(), Yg.data_ptr(), M, N, K)
                arr[1] = jq4k.GemmDesc(Wus[c].data_ptr(), Xd.data_ptr(), Yu.data_ptr(), M, N, K)
            descs.append(arr)
        grouped_fn = L.jq4k_gemv_batched if M == 1 else L.jq4k_gemm_batched

        def grouped(i):
            check(jq4k, grouped_fn(ctypes.addressof(descs[i % copies]), 2, stream_ptr(torch)))
        steps = args.steps if M == 1 else args.prefill_steps
        w = 3 if M == 1 else MFMA_WARMUP
        tf = timed(torch, fused, steps, w, graph_ok(args, True)) / steps
        tg = timed(torch, grouped, steps, w, graph_ok(args, True)) / steps
        if M == 1:
            out["m1"] = {"N": N, "K": K, "weight_bytes": wbytes, "fused_us": round(tf * 1e6, 2),
                         "fused_GB_s": round(wbytes / tf / 1e9, 1),
                         "grouped_no_epilogue_us": round(tg * 1e6, 2)}
        else:
            fl = 2.0 * 2 * M * N * K
            out[f"m{M}"] = {"N": N, "K": K, "M": M, "fused_us": round(tf * 1e6, 1),
                            "fused_TFLOP_s": round(fl / tf / 1e12, 1),
                            "grouped_no_epilogue_us": round(tg * 1e6, 1)}
    return out


def rmsnorm_leg(torch, jq4k, args, traces):
    """The decode gate projection (9728 x 2560) with its RMSNorm fused into the
    x staging (jq4k_gemv_rmsnorm), beside the plain GEMV of the same matrix;
    then the row norm of a 2048 x 2560 prefill (jq4k_rmsnorm_bf16)."""
    layer = qi.decode_layer(1, 0, 1)
    _, N, K, W, X = layer[4]
    g = qi.rng(7)
    gamma = qi.f32_to_bf16_bits((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
    copies = copies_for(W.nbytes)
    Ws = [to_dev(torch, W)]
    Ws += [Ws[0].clone() for _ in range(copies - 1)]
    Xd = to_dev(torch, X.view(np.int16))
    Gd = to_dev(torch, gamma.view(np.int16))
    Y = torch.empty(N, dtype=torch.float32, device="cuda:0")
    L = jq4k.raw()

    def fused(i):
        check(jq4k, L.jq4k_gemv_rmsnorm(Ws[i % copies].data_ptr(), Xd.data_ptr(), Gd.data_ptr(),
                                        1e-6, Y.data_ptr(), N, K, stream_ptr(torch)))

    def plain(i):
        check(jq4k, L.jq4k_gemv(Ws[i % copies].data_ptr(), Xd.data_ptr(), Y.data_ptr(), 1, N, K,
                                stream_ptr(torch)))
    tf = timed(torch, fused, args.steps, 4, not args.eager) / args.steps
    tp = timed(torch, plain, args.steps, 4, not args.eager) / args.steps
    out = {"N": N, "K": K, "fused_us": round(tf * 1e6, 2),
           "fused_GB_s": round(W.nbytes / tf / 1e9, 1), "plain_gemv_us": round(tp * 1e6, 2)}
    M = 2048
    Xp = qi.activations(qi.rng(8), M, K)
    xcopies = copies_for(2 * Xp.nbytes)
    Xs = [to_dev(torch, Xp.view(np.int16))]
    Xs += [Xs[0].clone() for _ in range(xcopies - 1)]
    Xh = [torch.empty_like(x) for x in Xs]

    def rows(i):
        c = i % xcopies
        check(jq4k, L.jq4k_rmsnorm_bf16(Xs[c].data_ptr(), Gd.data_ptr(), 1e-6, Xh[c].data_ptr(),
                                        M, K, stream_ptr(torch)))
    tr = timed(torch, rows, args.steps, 4, not args.eager) / args.steps
    moved = 2 * Xp.nbytes   # read X, write x_hat (gamma: 5 KB, L2-resident)
    out["rows_m2048"] = {"M": M, "K": K, "us": round(tr * 1e6, 2),
                         "roofline": {"bound": "hbm", "achieved": round(moved / tr / 1e9, 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(moved / tr / 1e9 / HBM_PEAK_GBS, 4),
                                      "bytes_per_launch": moved}}
    return out


def kv_leg(torch, jq4k, args, traces):
    """FP16 <-> INT8 KV-cache convert over the whole 1024-token cache of the
    workload (36 layers x K, V x 8 heads x 1024 tokens = 589,824 vectors of
    128 values, 151 MB in fp16): one jq4k_kv_quant_i8 launch and one
    jq4k_kv_dequant_f16 launch, each over rotating copies (>= 1 GiB).
    HBM-bound: bytes = 2 B read + 1 B written per value + 4 B per vector (or
    the reverse)."""
    L = jq4k.raw()
    v = qi.kv_cache(5)
    nvec, dim = v.shape
    nbytes = nvec * dim * 3 + nvec * 4
    copies = copies_for(nbytes)
    vs = [to_dev(torch, v.view(np.int16))]
    vs += [vs[0].clone() for _ in range(copies - 1)]
    qs = [torch.empty((nvec, dim), dtype=torch.int8, device="cuda:0") for _ in range(copies)]
    ss = [torch.empty(nvec, dtype=torch.float32, device="cuda:0") for _ in range(copies)]
    outs = [torch.empty((nvec, dim), dtype=torch.int16, device="cuda:0") for _ in range(copies)]
    s0 = stream_ptr(torch)
    for i in range(copies):
        check(jq4k, L.jq4k_kv_quant_i8(vs[i].data_ptr(), qs[i].data_ptr(), ss[i].data_ptr(), nvec,
                                       dim, s0))

    def quant(i):
        c = i % copies
        check(jq4k, L.jq4k_kv_quant_i8(vs[c].data_ptr(), qs[c].data_ptr(), ss[c].data_ptr(), nvec,
                                       dim, stream_ptr(torch)))

    def dequant(i):
        c = i % copies
        check(jq4k, L.jq4k_kv_dequant_f16(qs[c].data_ptr(), ss[c].data_ptr(), outs[c].data_ptr(),
                                          nvec, dim, stream_ptr(torch)))
    steps = max(10, args.prefill_steps)
    res = {"workload": "Qwen3-4B KV cache at 1024 tokens: 589,824 vectors x 128 fp16 "
                       "(36 layers x K,V x 8 heads), seed 5; one launch per direction",
           "bytes_per_launch": nbytes, "rotation_copies": copies}
    for name, fn in (("fp16_to_int8", quant), ("int8_to_fp16", dequant)):
        t = timed(torch, fn, steps, 2, not args.eager) / steps
        gbs = nbytes / t / 1e9
        res[name] = {"us": round(t * 1e6, 2), "GB_s": round(gbs, 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    return res


def ceilings_leg(torch, jq4k, args, traces):
    """What this GPU reaches, beside the published peaks: streaming reads of
    1 GiB, and of the decode layer's and the LM head's sizes rotated through
    1 GiB, in two patterns (read_*: jq4k_probe_read, a grid striding over the
    buffer with plain 16-byte loads; stream_*: jq4k_probe_stream, one
    short-lived workgroup per 36 KB with non-temporal loads, the faster one
    here), and a loop of v_mfma_f32_32x32x16_bf16 on register operands
    (jq4k_probe_mfma)."""
    L = jq4k.raw()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 8 * cus
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda:0")
    buf = torch.empty(ROTATION_BYTES, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)
    out = {}
    for name, nbytes in (("read_1GiB", ROTATION_BYTES), ("read_56.8MB", 56770560),
                         ("read_218.8MB", 218787840)):
        pieces = max(1, ROTATION_BYTES // nbytes)

        def rd(i, nbytes=nbytes, pieces=pieces):
            off = (i % pieces) * nbytes
            check(jq4k, L.jq4k_probe_read(buf.data_ptr() + off, nbytes, sink.data_ptr(), wgs,
                                          stream_ptr(torch)))
        def st(i, nbytes=nbytes, pieces=pieces):
            off = (i % pieces) * nbytes
            check(jq4k, L.jq4k_probe_stream(buf.data_ptr() + off, nbytes, sink.data_ptr(),
                                            stream_ptr(torch)))
        steps = 20 if nbytes == ROTATION_BYTES else 100
        for key, fn in ((name, rd), (name.replace("read_", "stream_"), st)):
            t = timed(torch, fn, steps, 3, not args.eager) / steps
            out[key] = {"bytes": nbytes, "us": round(t * 1e6, 2), "GB_s": round(nbytes / t / 1e9, 1),
                        "frac_of_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
    iters = 4096
    mwgs = 4 * cus       # four workgroups of four waves per CU: four waves per SIMD

    def mf(i):
        check(jq4k, L.jq4k_probe_mfma(iters, sink.data_ptr(), mwgs, stream_ptr(torch)))
    t = timed(torch, mf, 5, 1, False) / 5
    fl = iters * 8 * 2.0 * 32 * 32 * 16 * mwgs * 4
    out["mfma_bf16_loop"] = {"workgroups": mwgs, "us": round(t * 1e6, 1),
                             "TFLOP_s": round(fl / t / 1e12, 1),
                             "frac_of_mfma_peak": round(fl / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    # the int8-activation MMQ variant's inner loop (MFMA + per-sub-block
    # rescale) from registers: an upper bound on its rate
    qwgs = 2 * cus

    def mq(i):
        check(jq4k, L.jq4k_probe_mmq(iters, sink.data_ptr(), qwgs, stream_ptr(torch)))
    t = timed(torch, mq, 5, 1, False) / 5
    ops = iters * 2.0 * 64 * 64 * 32 * qwgs * 4
    out["mmq_i8_inner_loop"] = {
        "workgroups": qwgs, "us": round(t * 1e6, 1), "TOPS": round(ops / t / 1e12, 1),
        "frac_of_int8_peak": round(ops / t / 1e12 / 5000.0, 4),
        "frac_of_bf16_peak": round(ops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "note": "16 v_mfma_i32_16x16x32_i8 per sub-block of a 64x64 wave tile plus the fp32 "
                "rescale of every int32 sum, operands in registers; compare with the bf16 "
                "path's full kernel (prefill.value)"}
    del buf
    return out


LEGS = {"single": single_leg, "decode": decode_leg, "lm_head": lm_head_leg, "m33": m33_leg,
        "prefill": prefill_leg, "lm_head_m512": lm_head_m512_leg, "swiglu": swiglu_leg,
        "rmsnorm": rmsnorm_leg, "kv": kv_leg, "ceilings": ceilings_leg}


# ---------------------------------------------------------------- profile

def profile_run(torch, jq4k):
    """Launches for rocprofv3 runs: for each leg of PROFILE_LEGS a marker and
    eager launches of what the leg times, over the same rotation of weight
    copies (>= 1 GiB, so that no launch finds its weights in the last-level
    cache), synchronised.  The first leg is a 512 MiB device copy, the
    reference for scaling FETCH_SIZE and WRITE_SIZE.  The marker is
    jq4k_probe_read over 16 bytes with PROFILE_MARKER + leg index
    workgroups, so that profile_summary.py can tell the legs apart."""
    L = jq4k.raw()
    s = stream_ptr(torch)
    msink = torch.empty((PROFILE_MARKER + len(PROFILE_LEGS)) * 256, dtype=torch.int32,
                        device="cuda:0")
    mbuf = torch.zeros(16, dtype=torch.uint8, device="cuda:0")

    def marker(name):
        torch.cuda.synchronize()
        check(jq4k, L.jq4k_probe_read(mbuf.data_ptr(), 16, msink.data_ptr(),
                                      PROFILE_MARKER + PROFILE_LEGS.index(name), s))
        torch.cuda.synchronize()

    def rotated(Ws):
        """Copies of the list of weight tensors Ws, >= 1 GiB in all."""
        c = copies_for(sum(w.numel() for w in Ws))
        return [Ws] + [[w.clone() for w in Ws] for _ in range(c - 1)]

    a = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    marker("copy_512MiB")
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b

    W, X = qi.single_gemv(0)
    Wr = rotated([to_dev(torch, W)])
    Xd = to_dev(torch, X.view(np.int16))
    Yd = torch.empty(2560, dtype=torch.float32, device="cuda:0")
    marker("single")
    for i in range(40):
        check(jq4k, L.jq4k_gemv(Wr[i % len(Wr)][0].data_ptr(), Xd.data_ptr(), Yd.data_ptr(), 1,
                                2560, 2560, s))
    torch.cuda.synchronize()
    del Wr

    layer = qi.decode_layer(1, 0, 1)
    Wr = rotated([to_dev(torch, W) for _, _, _, W, _ in layer])
    Xs = [to_dev(torch, X.view(np.int16)) for _, _, _, _, X in layer]
    Ys = [torch.empty(N, dtype=torch.float32, device="cuda:0") for _, N, _, _, _ in layer]
    arrs = []
    for Wc in Wr:
        arr = (jq4k.GemvDesc * 7)()
        for p, (_, N, K, _, _) in enumerate(layer):
            arr[p] = jq4k.GemvDesc(Wc[p].data_ptr(), Xs[p].data_ptr(), Ys[p].data_ptr(), N, K)
        arrs.append(arr)
    marker("decode")
    for i in range(20):
        check(jq4k, L.jq4k_gemv_batched(ctypes.addressof(arrs[i % len(arrs)]), 7, s))
    torch.cuda.synchronize()
    del Wr, arrs

    W, X = qi.lm_head(4, 512)
    Wr = rotated([to_dev(torch, W)])
    X1 = to_dev(torch, X[:1].view(np.int16))
    Y1 = torch.empty(151936, dtype=torch.float32, device="cuda:0")
    marker("lm_head")
    for i in range(10):
        check(jq4k, L.jq4k_gemv(Wr[i % len(Wr)][0].data_ptr(), X1.data_ptr(), Y1.data_ptr(), 1,
                                151936, 2560, s))
    torch.cuda.synchronize()

    # M = 33: one pass through the 36 layers, as the benchmark runs it
    keep, sarrs = [], []
    for layer_i in range(36):
        sarr = (jq4k.GemmDesc * 7)()
        for p in range(7):
            _, N, K, Wp, Xp = qi.prefill_projection(2, layer_i, p, 33)
            t = (to_dev(torch, Wp), to_dev(torch, Xp.view(np.int16)),
                 torch.empty((33, N), dtype=torch.float32, device="cuda:0"))
            keep.append(t)
            sarr[p] = jq4k.GemmDesc(t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), 33, N, K)
        sarrs.append(sarr)
    need = ctypes.c_size_t(0)
    check(jq4k, L.jq4k_gemm_workspace_size(ctypes.addressof(sarrs[0]), 7, ctypes.byref(need)))
    ws = torch.zeros(max(need.value, 256), dtype=torch.uint8, device="cuda:0")
    marker("m33")
    for sarr in sarrs:
        check(jq4k, L.jq4k_gemm_batched_ws(ctypes.addressof(sarr), 7, ws.data_ptr(), ws.numel(),
                                           s))
    torch.cuda.synchronize()
    del keep, sarrs, ws

    projs = [qi.prefill_projection(3, 0, p, 2048) for p in range(7)]
    Wg = rotated([to_dev(torch, Wp) for _, _, _, Wp, _ in projs])
    Xg = [to_dev(torch, Xp.view(np.int16)) for _, _, _, _, Xp in projs]
    Yg = [torch.empty((2048, N), dtype=torch.float32, device="cuda:0") for _, N, _, _, _ in projs]
    garrs = []
    for Wc in Wg:
        garr = (jq4k.GemmDesc * 7)()
        for p, (_, N, K, _, _) in enumerate(projs):
            garr[p] = jq4k.GemmDesc(Wc[p].data_ptr(), Xg[p].data_ptr(), Yg[p].data_ptr(), 2048,
                                    N, K)
        garrs.append(garr)
    # the matrix-core legs start warm, as the benchmark times them (the
    # warm-up launches under a marker of their own)
    marker("warmup")
    for i in range(MFMA_WARMUP):
        check(jq4k, L.jq4k_gemm_batched(ctypes.addressof(garrs[i % len(garrs)]), 7, s))
    marker("prefill")
    for i in range(8):
        check(jq4k, L.jq4k_gemm_batched(ctypes.addressof(garrs[i % len(garrs)]), 7, s))
    torch.cuda.synchronize()
    del Wg, Xg, Yg, garrs

    X512 = to_dev(torch, X.view(np.int16))
    Y512 = torch.empty((512, 151936), dtype=torch.float32, device="cuda:0")
    marker("warmup")
    for i in range(MFMA_WARMUP):
        check(jq4k, L.jq4k_gemm(Wr[i % len(Wr)][0].data_ptr(), X512.data_ptr(), Y512.data_ptr(),
                                512, 151936, 2560, s))
    marker("lm_head_m512")
    for i in range(8):
        check(jq4k, L.jq4k_gemm(Wr[i % len(Wr)][0].data_ptr(), X512.data_ptr(), Y512.data_ptr(),
                                512, 151936, 2560, s))
    torch.cuda.synchronize()
    print("profile run done", flush=True)


# ---------------------------------------------------------------- CPU

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _omp_threads(n):
    """Set the OpenMP thread count of the (already loaded) oracle library."""
    import oracle
    oracle.lib()
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
        return True
    except (OSError, AttributeError):
        return False


def cpu_baseline(layer, budget_s=12.0):
    """The oracle (C, OpenMP over rows, fp32 dequant + fp64 accumulation) on
    the host: whole decode-layer passes for about budget_s seconds on every
    host thread, then the single 2560 x 2560 GEMV on one thread for a
    per-core rate."""
    import oracle
    threads = oracle.num_threads()
    reps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for _, N, K, W, X in layer:
            oracle.gemm(W, X, N, K)
        reps += 1
    secs = time.perf_counter() - t0
    weights = sum(N * K for _, N, K, _, _ in layer) * reps
    out = {"value": round(weights * BYTES_PER_WEIGHT / secs / 1e9, 3), "unit": "GB/s",
           "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"{reps} passes of the full decode layer (7 projections, M=1) in "
                     f"{secs:.1f} s on {threads} threads, fp32 dequant + fp64 accumulate"}
    W, X = qi.single_gemv(0)
    if _omp_threads(1):
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 3.0:
            oracle.gemm(W, X, 2560, 2560)
            n += 1
        s1 = time.perf_counter() - t0
        _omp_threads(threads)
        out["single_thread_cfg0"] = {"value": round(n * W.nbytes / s1 / 1e9, 4), "unit": "GB/s",
                                     "sample": f"{n} runs of the 2560x2560 GEMV in {s1:.1f} s "
                                               "on 1 thread"}
    return out


def cpu_baseline_prefill(budget_rows=64):
    import oracle
    M = 2048
    t0 = time.perf_counter()
    flops = 0.0
    for p in range(7):
        _, N, K, W, X = qi.prefill_projection(3, 0, p, M)
        oracle.gemm(W[:budget_rows], X, budget_rows, K)
        flops += 2.0 * M * budget_rows * K
    secs = time.perf_counter() - t0
    return {"value": round(flops / secs / 1e12, 5), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {budget_rows} rows of each of the 7 projections at M=2048 "
                      f"({flops / 1e9:.1f} GFLOP in {secs:.1f} s)"}


# ------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the matmul shards by rows of W, see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch
    import q4_weight_only_amd as jq4k
    jq4k.raw()
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    torch.cuda.set_device(0)

    if args.profile:
        profile_run(torch, jq4k)
        return
    traces = kernel_trace()
    if args.only:
        out = {name: LEGS[name](torch, jq4k, args, traces) for name in args.only.split(",")}
        print(json.dumps(out), flush=True)
        return

    legs = {}
    for name, fn in LEGS.items():
        legs[name] = fn(torch, jq4k, args, traces)
        print(f"bench: {name} done", file=sys.stderr, flush=True)
    dec = legs["decode"]
    out = {
        "metric": METRIC,
        "value": dec["GB_s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["us"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": dec["workload"] + "; one jq4k_gemv_batched launch per step (the seven "
                                          "are independent here)",
            "weight_bytes_per_step": dec["weight_bytes_per_step"],
            "rotation_copies": dec["rotation_copies"],
            "launch": "eager" if args.eager else "hip-graph",
            "arithmetic": "bf16 activations staged as binary16 (exact), 4-bit codes as "
                          "binary16 in v_dot2_f32_f16, fp32 sums, per-row certified bound",
            "device": torch.cuda.get_device_name(0),
        },
        "roofline": dec["roofline"],
        "decode_step_dependency_ordered": dict(
            dec["modes"]["dependency_4"],
            note="q|k|v, o, gate|up, down as four grouped launches, each consuming the "
                 "previous outputs in a real decode step"),
        "prefill": legs["prefill"],
        "configs": {"single_2560x2560_m1": legs["single"], "decode_layer_m1": dec,
                    "prefill_m33_36_layers": legs["m33"], "prefill_m2048_layer": legs["prefill"],
                    "lm_head_m1": legs["lm_head"], "lm_head_m512": legs["lm_head_m512"]},
        "next": {"swiglu_gate_up": legs["swiglu"], "rmsnorm": legs["rmsnorm"],
                 "kv_convert": legs["kv"]},
        "ceilings": legs["ceilings"],
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(qi.decode_layer(1, 0, 1))
        out["prefill"]["cpu_baseline"] = cpu_baseline_prefill()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
