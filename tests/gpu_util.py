"""Helpers for the GPU parity tests: device copies, oracle comparison."""
import sys

import numpy as np

import oracle


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda:0")


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run_gemm(W, X, N, K, path=None):
    """Run jq4k on host arrays W (uint8 N x nb*144), X (uint16 M x K); return Y."""
    import torch
    import q4_weight_only_amd as jq4k
    M = X.shape[0]
    Wd = dev(W.reshape(N, -1))
    Xd = dev(X.reshape(M, K)).view(torch.bfloat16)
    Yd = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    if path is None:
        jq4k.gemm(Wd, Xd, Yd)
    elif path == "gemv":
        jq4k.gemv(Wd, Xd, Yd)
    else:
        jq4k.gemm(Wd, Xd, Yd, path=path)
    return host(Yd)


def parity(y, Y_ref, A, what):
    """Assert every element meets |y - y_ref| <= 2e-3 * A + 1e-5; return the
    worst ratio of error to bound."""
    y = np.asarray(y, np.float64)
    ok = oracle.within_tolerance(y, Y_ref, A)
    ratio = np.abs(y - Y_ref) / oracle.tolerance(A)
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(
            f"{what}: {len(bad)} of {ok.size} elements out of tolerance; first at {i}: "
            f"gpu={y[i]!r} ref={Y_ref[i]!r} A={A[i]!r}; worst ratio {worst:.3g}")
    return worst
