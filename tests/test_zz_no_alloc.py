"""The allocation-free grouped matmul (jq4k_gemm_batched_noalloc), for
callers that cannot allocate: through the C ABI, two calls in a row (the
second on smaller problems), each output bit-identical to the existing
jq4k_gemm_batched_ws with a caller workspace on the same problems, and
within the oracle bound; a request beyond the static buffer is refused with
nothing launched."""
import ctypes

import numpy as np
import pytest

import oracle
import q4k_inputs as qi
from tests.gpu_util import announce, dev, host, parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import q4_weight_only_amd as jq4k
    jq4k.raw()
    return jq4k


def _problems(g, shapes):
    return [(M, N, K, qi.weight_bytes(g, N, K), qi.activations(g, M, K)) for M, N, K in shapes]


def _run(gpu, probs, noalloc):
    Wd = [dev(W) for *_, W, _ in probs]
    Xd = [dev(X).view(torch.bfloat16) for *_, X in probs]
    Yd = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
          for M, N, *_ in probs]
    arr = gpu.gemm_descs(list(zip(Wd, Xd, Yd)))
    L = gpu.raw()
    s = torch.cuda.current_stream().cuda_stream
    if noalloc:
        rc = L.jq4k_gemm_batched_noalloc(ctypes.addressof(arr), len(probs), s)
    else:
        n = gpu.gemm_workspace_size(list(zip(Wd, Xd, Yd)))
        ws = torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda:0")
        rc = L.jq4k_gemm_batched_ws(ctypes.addressof(arr), len(probs), ws.data_ptr(), n, s)
    assert rc == 0, gpu.strerror(rc)
    return [host(y) for y in Yd]


def test_noalloc_matches_workspace_entry_point(gpu):
    g = np.random.default_rng(600)
    # first call: a Qwen3-4B layer at M = 33 (down split in K ranges)
    layer = [qi.prefill_projection(2, 0, p, 33) for p in range(7)]
    first = [(33, N, K, W, X) for _, N, K, W, X in layer]
    # second call: smaller problems, one of them split (K = 9728)
    second = _problems(g, [(5, 300, 9728), (3, 77, 2560), (1, 129, 4096)])
    for name, probs in (("layer M=33", first), ("smaller", second)):
        announce(f"noalloc vs workspace: {name}")
        ref = _run(gpu, probs, noalloc=False)
        got = _run(gpu, probs, noalloc=True)
        for (M, N, K, W, X), a, b in zip(probs, got, ref):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (name, M, N, K)
            if name == "smaller" or N <= 1024:
                Y, A = oracle.gemm(W, X, N, K)
                parity(a, Y, A, f"noalloc {name} M={M} N={N} K={K}")


def test_noalloc_refuses_more_than_the_scratch(gpu):
    """Problems whose split-K workspace exceeds JQ4K_SCRATCH_BYTES: -3 and no
    launch (the pointers are never read); the buffer still works after."""
    big = (gpu.GemmDesc * 4)()
    for i in range(4):
        big[i] = gpu.GemmDesc(16, 16, 16, 64, 2560, 9728)   # 4 x 6.6 MB needed
    n = ctypes.c_size_t(0)
    assert gpu.raw().jq4k_gemm_workspace_size(ctypes.addressof(big), 4, ctypes.byref(n)) == 0
    assert n.value > gpu.SCRATCH_BYTES
    rc = gpu.raw().jq4k_gemm_batched_noalloc(ctypes.addressof(big), 4, None)
    assert rc == gpu.ESCRATCH
    g = np.random.default_rng(601)
    probs = _problems(g, [(17, 200, 9728)])
    assert np.array_equal(_run(gpu, probs, True)[0].view(np.uint32),
                          _run(gpu, probs, False)[0].view(np.uint32))
