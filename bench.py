"""Benchmark of the Q4_K weight-only matmul on one MI355X.

Headline (value): M = 1 weight bandwidth over one Qwen3-4B decode layer -- the
seven Q4_K projections q, k, v, o, gate, up, down at one token, each a GEMV
(0.5625 bytes per weight).  A step is one pass over the seven projections.
Second figure (prefill): TFLOP/s of the same seven projections at M = 2048
tokens on the MFMA path.

Protocol.  Inputs are seeded synthetic tensors resident in HBM before timing.
Weights rotate over enough identical copies (>= 1 GiB) that no step finds its
weights in the 256 MB last-level cache.  W warm-up steps run untimed; the K
timed steps are captured in a HIP graph (launch overhead out of the timed
region, kernels back to back) and bracketed by HIP events recorded on the
stream the kernels run on.  The CPU oracle is timed on a bounded sample of the
same workload for the cpu_baseline field.

    python bench.py [--steps K] [--warmup W] [--prefill-steps P] [--no-cpu]
"""
import argparse
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches, no graph")
    ap.add_argument("--only", default="",
                    help="comma-separated legs to time (decode,lm_head,...); prints them "
                         "as one JSON object instead of the benchmark line")
    ap.add_argument("--profile", action="store_true",
                    help="a few eager launches of each kernel for rocprofv3, no JSON line")
    return ap.parse_args()


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


DEPENDENCY_GROUPS = [[0, 1, 2], [3], [4, 5], [6]]   # q|k|v, o, gate|up, down
PREFILL_KERNEL = "jq4k::q4k_gemm_ws_kernel<false>"   # jq4k_gemm_batched at M = 2048 (256-row tile)
SKINNY_KERNEL = "jq4k::q4k_gemm_skinny_kernel<3>"    # jq4k_gemm_batched_ws at M = 33


def decode_leg(torch, jq4k, args):
    """Seven Q4_K GEMVs of one decode layer, timed three ways:
    batched_1     one jq4k_gemv_batched launch for all seven (they are
                  independent in this workload) -- the headline value;
    dependency_4  the launches a real decode step can make (q|k|v, o, gate|up,
                  down: later groups consume earlier outputs);
    separate_7    seven jq4k_gemv launches."""
    import ctypes
    layer = qi.decode_layer(1, 0, 1)
    layer_bytes = sum(W.nbytes for _, _, _, W, _ in layer)
    copies = max(2, math.ceil(ROTATION_BYTES / layer_bytes))
    Ws = [[torch.from_numpy(W).to("cuda:0") for _, _, _, W, _ in layer]]
    for _ in range(copies - 1):
        Ws.append([w.clone() for w in Ws[0]])
    Xs = [torch.from_numpy(X.view(np.int16)).to("cuda:0").view(torch.bfloat16)
          for _, _, _, _, X in layer]
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

    def check(rc):
        if rc:
            raise RuntimeError(jq4k.strerror(rc))

    def step_batched(i):
        check(L.jq4k_gemv_batched(ctypes.addressof(all7[i % copies]), 7,
                                  torch.cuda.current_stream().cuda_stream))

    def step_grouped(i):
        s = torch.cuda.current_stream().cuda_stream
        for arr, gi in zip(grouped[i % copies], DEPENDENCY_GROUPS):
            check(L.jq4k_gemv_batched(ctypes.addressof(arr), len(gi), s))

    def step_separate(i):
        Wc = Ws[i % copies]
        s = torch.cuda.current_stream().cuda_stream
        for p, (_, N, K, _, _) in enumerate(layer):
            check(L.jq4k_gemv(Wc[p].data_ptr(), Xs[p].data_ptr(), Ys[p].data_ptr(), 1, N, K, s))

    graph = not args.eager
    secs = timed(torch, step_batched, args.steps, args.warmup, graph)
    modes = {}
    for name, fn, launches in (("batched_1", None, 1), ("dependency_4", step_grouped, 4),
                               ("separate_7", step_separate, 7)):
        t = secs if fn is None else timed(torch, fn, args.steps, args.warmup, graph)
        modes[name] = {"launches_per_step": launches, "us_per_step": round(t / args.steps * 1e6, 2),
                       "GB_s": round(layer_bytes * args.steps / t / 1e9, 1)}
    per_proj = {}
    for p, (name, N, K, W, _) in enumerate(layer):
        def one(i, p=p, N=N, K=K):
            s = torch.cuda.current_stream().cuda_stream
            check(L.jq4k_gemv(Ws[i % copies][p].data_ptr(), Xs[p].data_ptr(), Ys[p].data_ptr(),
                              1, N, K, s))
        t = timed(torch, one, args.steps, 4, graph)
        per_proj[name] = {"N": N, "K": K, "us": round(t / args.steps * 1e6, 3),
                          "GB_s": round(W.nbytes * args.steps / t / 1e9, 1)}
    return layer, layer_bytes, copies, secs, modes, per_proj


def lm_head_leg(torch, jq4k, args):
    """The 151936 x 2560 Q4_K LM head at M = 1: one 219 MB GEMV, the largest
    single-kernel bandwidth case (context for the headline)."""
    W, X = qi.lm_head(4, 1)
    N, K = 151936, 2560
    copies = max(2, math.ceil(ROTATION_BYTES / W.nbytes))
    Wd = [torch.from_numpy(W).to("cuda:0")]
    Wd += [Wd[0].clone() for _ in range(copies - 1)]
    Xd = torch.from_numpy(X.view(np.int16)).to("cuda:0")
    Yd = torch.empty(N, dtype=torch.float32, device="cuda:0")
    L = jq4k.raw()

    def one(i):
        rc = L.jq4k_gemv(Wd[i % copies].data_ptr(), Xd.data_ptr(), Yd.data_ptr(), 1, N, K,
                         torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(jq4k.strerror(rc))
    steps = max(10, args.steps // 10)
    t = timed(torch, one, steps, 3, not args.eager)
    return {"N": N, "K": K, "weight_bytes": int(W.nbytes), "us": round(t / steps * 1e6, 2),
            "GB_s": round(W.nbytes * steps / t / 1e9, 1),
            "frac_of_hbm_peak": round(W.nbytes * steps / t / 1e9 / HBM_PEAK_GBS, 4)}


def prefill_leg(torch, jq4k, args):
    """The seven projections of one layer at M = 2048 tokens on the MFMA path,
    timed as batched_1 (one jq4k_gemm_batched launch; the headline prefill
    figure), dependency_4 (q|k|v, o, gate|up, down) and separate_7 (seven
    jq4k_gemm launches)."""
    import ctypes
    M = 2048
    projs = [qi.prefill_projection(3, 0, p, M) for p in range(7)]
    flops = sum(2.0 * M * N * K for _, N, K, _, _ in projs)
    copies = 2
    Ws = [[torch.from_numpy(W).to("cuda:0") for _, _, _, W, _ in projs]]
    Ws.append([w.clone() for w in Ws[0]])
    Xs = [torch.from_numpy(X.view(np.int16)).to("cuda:0").view(torch.bfloat16)
          for _, _, _, _, X in projs]
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

    def check(rc):
        if rc:
            raise RuntimeError(jq4k.strerror(rc))

    def step_batched(i):
        check(L.jq4k_gemm_batched(ctypes.addressof(all7[i % copies]), 7,
                                  torch.cuda.current_stream().cuda_stream))

    def step_grouped(i):
        s = torch.cuda.current_stream().cuda_stream
        for arr, gi in zip(grouped[i % copies], DEPENDENCY_GROUPS):
            check(L.jq4k_gemm_batched(ctypes.addressof(arr), len(gi), s))

    def step_separate(i):
        Wc = Ws[i % copies]
        s = torch.cuda.current_stream().cuda_stream
        for p, (_, N, K, _, _) in enumerate(projs):
            check(L.jq4k_gemm(Wc[p].data_ptr(), Xs[p].data_ptr(), Ys[p].data_ptr(), M, N, K, s))

    graph = not args.eager
    secs = timed(torch, step_batched, args.prefill_steps, 2, graph)
    modes = {}
    for name, fn, launches in (("batched_1", None, 1), ("dependency_4", step_grouped, 4),
                               ("separate_7", step_separate, 7)):
        t = secs if fn is None else timed(torch, fn, args.prefill_steps, 2, graph)
        modes[name] = {"launches_per_step": launches,
                       "us_per_step": round(t / args.prefill_steps * 1e6, 1),
                       "TFLOP_s": round(flops * args.prefill_steps / t / 1e12, 1)}
    per_proj = {}
    for p, (name, N, K, _, _) in enumerate(projs):
        def one(i, p=p, N=N, K=K):
            s = torch.cuda.current_stream().cuda_stream
            check(L.jq4k_gemm(Ws[i % copies][p].data_ptr(), Xs[p].data_ptr(), Ys[p].data_ptr(),
                              M, N, K, s))
        t = timed(torch, one, args.prefill_steps, 1, graph)
        per_proj[name] = {"N": N, "K": K, "us": round(t / args.prefill_steps * 1e6, 2),
                          "TFLOP_s": round(2.0 * M * N * K * args.prefill_steps / t / 1e12, 1)}
    return flops, secs, modes, per_proj


def prefill_m33_leg(torch, jq4k, args):
    """M = 33 through all 36 layers' seven projections (252 matmuls, 2.04 GB of
    Q4_K weights, child seeds [2, layer, p]): one jq4k_gemm_batched_ws launch
    per layer (split K: down in 2 K ranges), 36 per pass, one
    workspace reused layer after layer.  HBM-bound: the attainable roofline
    counts W, X and Y bytes at 8 TB/s.  The same pass through
    jq4k_gemm_batched (whole K per tile) is timed beside it."""
    import ctypes
    M, L = 33, jq4k.raw()
    keep, arrs = [], []
    wbytes = xybytes = flops = 0
    for layer in range(36):
        arr = (jq4k.GemmDesc * 7)()
        for p in range(7):
            _, N, K, W, X = qi.prefill_projection(2, layer, p, M)
            Wd = torch.from_numpy(W).to("cuda:0")
            Xd = torch.from_numpy(X.view(np.int16)).to("cuda:0")
            Yd = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
            keep.append((Wd, Xd, Yd))
            arr[p] = jq4k.GemmDesc(Wd.data_ptr(), Xd.data_ptr(), Yd.data_ptr(), M, N, K)
            wbytes += W.nbytes
            xybytes += X.nbytes + M * N * 4
            flops += 2.0 * M * N * K
        arrs.append(arr)
    need = ctypes.c_size_t(0)
    rc = L.jq4k_gemm_workspace_size(ctypes.addressof(arrs[0]), 7, ctypes.byref(need))
    if rc:
        raise RuntimeError(jq4k.strerror(rc))
    ws = torch.zeros(max(need.value, 256), dtype=torch.uint8, device="cuda:0")

    def pass_ws(i):
        s = torch.cuda.current_stream().cuda_stream
        for arr in arrs:
            rc = L.jq4k_gemm_batched_ws(ctypes.addressof(arr), 7, ws.data_ptr(), ws.numel(), s)
            if rc:
                raise RuntimeError(jq4k.strerror(rc))

    def pass_whole_k(i):
        s = torch.cuda.current_stream().cuda_stream
        for arr in arrs:
            rc = L.jq4k_gemm_batched(ctypes.addressof(arr), 7, s)
            if rc:
                raise RuntimeError(jq4k.strerror(rc))
    steps = max(3, args.prefill_steps // 2)
    t = timed(torch, pass_ws, steps, 1, not args.eager) / steps
    t_whole = timed(torch, pass_whole_k, steps, 1, not args.eager) / steps
    allb = wbytes + xybytes
    return {"workload": "Qwen3-4B cold prefill, M=33 through 36 layers x 7 Q4_K projections "
                        "(252 matmuls), seeds [2,l,p]; one jq4k_gemm_batched_ws (split-K) "
                        "launch per layer",
            "launches_per_pass": 36, "us_per_pass": round(t * 1e6, 1),
            "workspace_bytes": int(need.value),
            "weight_GB_s": round(wbytes / t / 1e9, 1),
            "roofline": {"bound": "hbm", "achieved": round(allb / t / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(allb / t / 1e9 / HBM_PEAK_GBS, 4),
                         "bytes_per_pass": allb,
                         "traffic_per_launch": measured_traffic(SKINNY_KERNEL),
                         "kernel": SKINNY_KERNEL},
            "TFLOP_s": round(flops / t / 1e12, 2),
            "whole_k_us_per_pass": round(t_whole * 1e6, 1)}


def kv_convert_leg(torch, jq4k, args):
    """FP16 <-> INT8 KV-cache convert over the whole 1024-token cache of the
    workload (36 layers x K, V x 8 heads x 1024 tokens = 589,824 vectors of
    128 values, 151 MB in fp16): one jq4k_kv_quant_i8 launch and one
    jq4k_kv_dequant_f16 launch, each timed over two rotating copies (456 MB,
    above the last-level cache).  HBM-bound: bytes = 2 B read + 1 B written
    per value + 4 B per vector (or the reverse)."""
    import ctypes
    L = jq4k.raw()
    v = qi.kv_cache(5)
    nvec, dim = v.shape
    vs = [torch.from_numpy(v.view(np.int16)).to("cuda:0")]
    vs.append(vs[0].clone())
    qs = [torch.empty((nvec, dim), dtype=torch.int8, device="cuda:0") for _ in range(2)]
    ss = [torch.empty(nvec, dtype=torch.float32, device="cuda:0") for _ in range(2)]
    outs = [torch.empty((nvec, dim), dtype=torch.int16, device="cuda:0") for _ in range(2)]
    s0 = torch.cuda.current_stream().cuda_stream
    for i in range(2):
        assert L.jq4k_kv_quant_i8(vs[i].data_ptr(), qs[i].data_ptr(), ss[i].data_ptr(), nvec, dim,
                                  s0) == 0

    def quant(i):
        s = torch.cuda.current_stream().cuda_stream
        rc = L.jq4k_kv_quant_i8(vs[i % 2].data_ptr(), qs[i % 2].data_ptr(), ss[i % 2].data_ptr(),
                                nvec, dim, s)
        if rc:
            raise RuntimeError(jq4k.strerror(rc))

    def dequant(i):
        s = torch.cuda.current_stream().cuda_stream
        rc = L.jq4k_kv_dequant_f16(qs[i % 2].data_ptr(), ss[i % 2].data_ptr(),
                                   outs[i % 2].data_ptr(), nvec, dim, s)
        if rc:
            raise RuntimeError(jq4k.strerror(rc))
    steps = max(10, args.prefill_steps)
    nbytes = nvec * dim * 3 + nvec * 4
    res = {"workload": "Qwen3-4B KV cache at 1024 tokens: 589,824 vectors x 128 fp16 "
                       "(36 layers x K,V x 8 heads), seed 5; one launch per direction",
           "bytes_per_launch": nbytes}
    for name, fn in (("fp16_to_int8", quant), ("int8_to_fp16", dequant)):
        t = timed(torch, fn, steps, 2, not args.eager) / steps
        gbs = nbytes / t / 1e9
        res[name] = {"us": round(t * 1e6, 2), "GB_s": round(gbs, 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    return res


def lm_head_m512_leg(torch, jq4k, args):
    """The 151936 x 2560 Q4_K LM head at M = 512 (a prefill chunk): one
    jq4k_gemm launch, MFMA-bound."""
    W, X = qi.lm_head(4, 512)
    N, K, M = 151936, 2560, 512
    Wd = torch.from_numpy(W).to("cuda:0")
    Xd = torch.from_numpy(X.view(np.int16)).to("cuda:0")
    Yd = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    L = jq4k.raw()

    def one(i):
        rc = L.jq4k_gemm(Wd.data_ptr(), Xd.data_ptr(), Yd.data_ptr(), M, N, K,
                         torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(jq4k.strerror(rc))
    steps = max(3, args.prefill_steps)
    t = timed(torch, one, steps, 2, not args.eager) / steps
    tf = 2.0 * M * N * K / t / 1e12
    return {"N": N, "K": K, "M": M, "us": round(t * 1e6, 1), "TFLOP_s": round(tf, 1),
            "frac_of_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}


def swiglu_leg(torch, jq4k, args):
    """gate|up of a layer with the SwiGLU epilogue fused (jq4k_gemm_swiglu):
    M = 1 (the decode gate/up, rotated over copies like the decode leg) and
    M = 2048; beside each, the same two matmuls as one grouped launch without
    the epilogue."""
    import ctypes
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
        copies = max(2, math.ceil(ROTATION_BYTES / wbytes)) if M == 1 else 1
        Wgs = [torch.from_numpy(Wg).to("cuda:0")]
        Wus = [torch.from_numpy(Wu).to("cuda:0")]
        for _ in range(copies - 1):
            Wgs.append(Wgs[0].clone())
            Wus.append(Wus[0].clone())
        Xd = torch.from_numpy(X.view(np.int16)).to("cuda:0")
        H = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        Yg = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        Yu = torch.empty((M, N), dtype=torch.float32, device="cuda:0")

        def fused(i):
            rc = L.jq4k_gemm_swiglu(Wgs[i % copies].data_ptr(), Wus[i % copies].data_ptr(),
                                    Xd.data_ptr(), H.data_ptr(), M, N, K,
                                    torch.cuda.current_stream().cuda_stream)
            if rc:
                raise RuntimeError(jq4k.strerror(rc))
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
            rc = grouped_fn(ctypes.addressof(descs[i % copies]), 2,
                            torch.cuda.current_stream().cuda_stream)
            if rc:
                raise RuntimeError(jq4k.strerror(rc))
        steps = args.steps if M == 1 else args.prefill_steps
        tf = timed(torch, fused, steps, 3, not args.eager) / steps
        tg = timed(torch, grouped, steps, 3, not args.eager) / steps
        key = "m1" if M == 1 else f"m{M}"
        if M == 1:
            out[key] = {"N": N, "K": K, "weight_bytes": wbytes, "fused_us": round(tf * 1e6, 2),
                        "fused_GB_s": round(wbytes / tf / 1e9, 1),
                        "grouped_no_epilogue_us": round(tg * 1e6, 2)}
        else:
            fl = 2.0 * 2 * M * N * K
            out[key] = {"N": N, "K": K, "M": M, "fused_us": round(tf * 1e6, 1),
                        "fused_TFLOP_s": round(fl / tf / 1e12, 1),
                        "grouped_no_epilogue_us": round(tg * 1e6, 1)}
    return out


def rmsnorm_leg(torch, jq4k, args):
    """The decode gate projection (9728 x 2560) with its RMSNorm fused into the
    x staging (jq4k_gemv_rmsnorm), beside the plain GEMV of the same matrix;
    weights rotate over copies like the decode leg."""
    layer = qi.decode_layer(1, 0, 1)
    _, N, K, W, X = layer[4]
    g = qi.rng(7)
    gamma = qi.f32_to_bf16_bits((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
    copies = max(2, math.ceil(ROTATION_BYTES / W.nbytes))
    Ws = [torch.from_numpy(W).to("cuda:0")]
    Ws += [Ws[0].clone() for _ in range(copies - 1)]
    Xd = torch.from_numpy(X.view(np.int16)).to("cuda:0")
    Gd = torch.from_numpy(gamma.view(np.int16)).to("cuda:0")
    Y = torch.empty(N, dtype=torch.float32, device="cuda:0")
    L = jq4k.raw()

    def fused(i):
        rc = L.jq4k_gemv_rmsnorm(Ws[i % copies].data_ptr(), Xd.data_ptr(), Gd.data_ptr(), 1e-6,
                                 Y.data_ptr(), N, K, torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(jq4k.strerror(rc))

    def plain(i):
        rc = L.jq4k_gemv(Ws[i % copies].data_ptr(), Xd.data_ptr(), Y.data_ptr(), 1, N, K,
                         torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(jq4k.strerror(rc))
    tf = timed(torch, fused, args.steps, 4, not args.eager) / args.steps
    tp = timed(torch, plain, args.steps, 4, not args.eager) / args.steps
    out = {"N": N, "K": K, "fused_us": round(tf * 1e6, 2),
           "fused_GB_s": round(W.nbytes / tf / 1e9, 1), "plain_gemv_us": round(tp * 1e6, 2)}
    # M > 1: the rows normalised once (jq4k_rmsnorm_bf16) ahead of the
    # prefill matmuls, 2048 x 2560 bf16, rotating over copies of X
    M = 2048
    Xp = qi.activations(qi.rng(8), M, K)
    xcopies = max(2, math.ceil(ROTATION_BYTES / (2 * Xp.nbytes)))
    Xs = [torch.from_numpy(Xp.view(np.int16)).to("cuda:0")]
    Xs += [Xs[0].clone() for _ in range(xcopies - 1)]
    Xh = [torch.empty_like(x) for x in Xs]

    def rows(i):
        c = i % xcopies
        rc = L.jq4k_rmsnorm_bf16(Xs[c].data_ptr(), Gd.data_ptr(), 1e-6, Xh[c].data_ptr(), M, K,
                                 torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(jq4k.strerror(rc))
    tr = timed(torch, rows, args.steps, 4, not args.eager) / args.steps
    moved = 2 * Xp.nbytes   # read X, write x_hat (gamma: 5 KB, L2-resident)
    out["rows_m2048"] = {"M": M, "K": K, "us": round(tr * 1e6, 2),
                         "roofline": {"bound": "hbm", "achieved": round(moved / tr / 1e9, 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(moved / tr / 1e9 / HBM_PEAK_GBS, 4),
                                      "bytes_per_launch": moved}}
    return out


def profile_run(torch, jq4k):
    """Launches for rocprofv3 runs: a 512 MiB device copy (the reference for
    scaling FETCH_SIZE / WRITE_SIZE), then 20 batched decode-layer GEMVs, 20
    LM-head GEMVs, 3 batched launches of the M=2048 layer and 5 split-K
    launches of one M=33 layer, eagerly, synchronised."""
    import ctypes
    a = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    L = jq4k.raw()
    s = torch.cuda.current_stream().cuda_stream
    layer = qi.decode_layer(1, 0, 1)
    dev = [(torch.from_numpy(W).to("cuda:0"), torch.from_numpy(X.view(np.int16)).to("cuda:0"),
            torch.empty(N, dtype=torch.float32, device="cuda:0")) for _, N, K, W, X in layer]
    arr = (jq4k.GemvDesc * 7)()
    for p, ((_, N, K, _, _), (W, X, Y)) in enumerate(zip(layer, dev)):
        arr[p] = jq4k.GemvDesc(W.data_ptr(), X.data_ptr(), Y.data_ptr(), N, K)
    for _ in range(20):
        assert L.jq4k_gemv_batched(ctypes.addressof(arr), 7, s) == 0
    torch.cuda.synchronize()
    W, X = qi.lm_head(4, 1)
    Wd = torch.from_numpy(W).to("cuda:0")
    Xd = torch.from_numpy(X.view(np.int16)).to("cuda:0")
    Yd = torch.empty(151936, dtype=torch.float32, device="cuda:0")
    for _ in range(20):
        assert L.jq4k_gemv(Wd.data_ptr(), Xd.data_ptr(), Yd.data_ptr(), 1, 151936, 2560, s) == 0
    torch.cuda.synchronize()
    M = 2048
    keep = []
    garr = (jq4k.GemmDesc * 7)()
    for p in range(7):
        _, N, K, W, X = qi.prefill_projection(3, 0, p, M)
        Wd = torch.from_numpy(W).to("cuda:0")
        Xd = torch.from_numpy(X.view(np.int16)).to("cuda:0")
        Yd = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        keep.append((Wd, Xd, Yd))
        garr[p] = jq4k.GemmDesc(Wd.data_ptr(), Xd.data_ptr(), Yd.data_ptr(), M, N, K)
    for _ in range(3):
        assert L.jq4k_gemm_batched(ctypes.addressof(garr), 7, s) == 0
    torch.cuda.synchronize()
    del keep
    M = 33
    keep = []
    sarr = (jq4k.GemmDesc * 7)()
    for p in range(7):
        _, N, K, W, X = qi.prefill_projection(2, 0, p, M)
        Wd = torch.from_numpy(W).to("cuda:0")
        Xd = torch.from_numpy(X.view(np.int16)).to("cuda:0")
        Yd = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        keep.append((Wd, Xd, Yd))
        sarr[p] = jq4k.GemmDesc(Wd.data_ptr(), Xd.data_ptr(), Yd.data_ptr(), M, N, K)
    need = ctypes.c_size_t(0)
    assert L.jq4k_gemm_workspace_size(ctypes.addressof(sarr), 7, ctypes.byref(need)) == 0
    ws = torch.zeros(max(need.value, 256), dtype=torch.uint8, device="cuda:0")
    for _ in range(5):
        assert L.jq4k_gemm_batched_ws(ctypes.addressof(sarr), 7, ws.data_ptr(), ws.numel(), s) == 0
    torch.cuda.synchronize()
    print("profile run done", flush=True)


def measured_traffic(kernel):
    """Mean HBM bytes (fetch + write) per dispatch of `kernel` from
    profiles/traffic.json, or None when the file is missing or was measured on
    other kernel sources."""
    from profile_summary import kernel_source_hash
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    if doc.get("kernel_sources_sha256") != kernel_source_hash():
        return None
    hits = [e for e in doc["kernels"].values() if e["kernel"] == kernel]
    n = sum(e["dispatches"] for e in hits)
    if not n:
        return None
    return round(sum((e["fetch_bytes"] + e["write_bytes"]) * e["dispatches"] for e in hits) / n)


def cpu_baseline(layer, budget_s=12.0):
    import oracle
    reps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for _, N, K, W, X in layer:
            oracle.gemm(W, X, N, K)
        reps += 1
    secs = time.perf_counter() - t0
    weights = sum(N * K for _, N, K, _, _ in layer) * reps
    return {"value": round(weights * BYTES_PER_WEIGHT / secs / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} passes of the full decode layer (7 projections, M=1) "
                      f"in {secs:.1f} s, fp32 dequant + fp64 accumulate"}


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
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {budget_rows} rows of each of the 7 projections at M=2048 "
                      f"({flops / 1e9:.1f} GFLOP in {secs:.1f} s)"}


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
    if args.only:
        legs = {"decode": lambda: decode_leg(torch, jq4k, args)[3:],
                "lm_head": lambda: lm_head_leg(torch, jq4k, args),
                "prefill": lambda: prefill_leg(torch, jq4k, args)[1:],
                "m33": lambda: prefill_m33_leg(torch, jq4k, args),
                "lm_head_m512": lambda: lm_head_m512_leg(torch, jq4k, args),
                "swiglu": lambda: swiglu_leg(torch, jq4k, args),
                "rmsnorm": lambda: rmsnorm_leg(torch, jq4k, args),
                "kv": lambda: kv_convert_leg(torch, jq4k, args)}
        out = {}
        for name in args.only.split(","):
            out[name] = legs[name]()
        print(json.dumps(out, default=str), flush=True)
        return
    layer, layer_bytes, copies, secs, modes, per_proj = decode_leg(torch, jq4k, args)
    gbs = layer_bytes * args.steps / secs / 1e9
    lm = lm_head_leg(torch, jq4k, args)
    flops, psecs, p_modes, p_per = prefill_leg(torch, jq4k, args)
    m33 = prefill_m33_leg(torch, jq4k, args)
    lm512 = lm_head_m512_leg(torch, jq4k, args)
    swiglu = swiglu_leg(torch, jq4k, args)
    rmsnorm = rmsnorm_leg(torch, jq4k, args)
    kv = kv_convert_leg(torch, jq4k, args)
    tflops = flops * args.prefill_steps / psecs / 1e12

    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(secs / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-4B decode layer, 7 Q4_K projections at M=1 "
                        "(q 4096x2560, k/v 1024x2560, o 2560x4096, gate/up 9728x2560, "
                        "down 2560x9728), seeds [1,0,p]; one jq4k_gemv_batched launch "
                        "per step (the seven are independent here)",
            "weight_bytes_per_step": layer_bytes,
            "rotation_copies": copies,
            "launch": "eager" if args.eager else "hip-graph",
            "device": torch.cuda.get_device_name(0),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("jq4k::q4k_gemv_batched_kernel"),
            "kernel": "q4k_gemv_batched_kernel",
            "avg_launch_us": round(secs / args.steps * 1e6, 3),
            "bytes_per_launch": layer_bytes,
        },
        "decode_modes": modes,
        "per_projection": per_proj,
        "lm_head_m1": lm,
        "prefill": {
            "workload": "Qwen3-4B layer, 7 Q4_K projections at M=2048, seeds [3,0,p]; one "
                        "jq4k_gemm_batched launch per step (the seven are independent here)",
            "value": round(tflops, 1), "unit": "TFLOP/s", "steps": args.prefill_steps,
            "ms_per_step": round(psecs / args.prefill_steps * 1e3, 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(PREFILL_KERNEL),
                         "kernel": PREFILL_KERNEL,
                         "avg_launch_us": round(psecs / args.prefill_steps * 1e6, 2),
                         "flops_per_launch": flops},
            "modes": p_modes,
            "per_projection": p_per,
        },
        "prefill_m33_36_layers": m33,
        "lm_head_m512": lm512,
        "swiglu_gate_up": swiglu,
        "rmsnorm_gate_m1": rmsnorm,
        "kv_convert": kv,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(layer)
        out["prefill"]["cpu_baseline"] = cpu_baseline_prefill()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
