"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer fields and the fp32 / bf16 dequantised weights must match bit for
bit; matmul outputs must meet |y - y_ref| <= 2e-3 * sum|w*x| + 1e-5 on every
element.  Inputs are the seeded synthetic workloads (Qwen3-4B shapes; the
genie-ai-runtime README's CLI banner gives 36 layers and a 2560 hidden size)
plus structured blocks built by the oracle-side encoder.
"""
import numpy as np
import pytest

import oracle
import q4k_inputs as qi
from oracle import q4k_pack as pk
from tests import golden_blocks
from tests.gpu_util import announce, dev, host, parity, run_gemm

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import q4_weight_only_amd as jq4k
    jq4k.raw()                                      # fails loudly if not built
    return jq4k


def _special_blocks(g, nb):
    """Random blocks whose d/dmin cover subnormal, negative, zero and large
    binary16 values (finite)."""
    W = g.integers(0, 256, (nb, 144), dtype=np.uint8)
    hdr = g.integers(0, 0x7C00, (nb, 2)).astype(np.uint16)
    hdr |= (g.integers(0, 2, (nb, 2)) << 15).astype(np.uint16)
    hdr[0:8] = [[0x0001, 0x0001], [0x03FF, 0x8001], [0x0000, 0x0000], [0x8000, 0x7BFF],
                [0x7BFF, 0x7BFF], [0x0400, 0x03FF], [0x3C00, 0x0000], [0x0000, 0x3C00]]
    W[:, 0:4] = hdr.view(np.uint8).reshape(nb, 4)
    return W


# ------------------------------------------------------------ exports

def _assert_same_weights(got_bits, ref_bits, zero_mask_got, zero_mask_ref, W, what):
    """Bit equality, with +0 and -0 taken as the same weight: the exact value
    d*sc*q - dmin*m = 0 has no sign (the GPU's fma can return -0 when d < 0)."""
    same = (got_bits == ref_bits) | (zero_mask_got & zero_mask_ref)
    if not same.all():
        idx = np.flatnonzero(~same)[:8]
        rows = [(int(i) // 256, int(i) % 256, hex(int(W[i // 256, 0]) | int(W[i // 256, 1]) << 8),
                 hex(int(W[i // 256, 2]) | int(W[i // 256, 3]) << 8), hex(int(got_bits[i])),
                 hex(int(ref_bits[i]))) for i in idx]
        raise AssertionError(f"{what}: {int((~same).sum())} weights differ; "
                             f"(block, i, d, dmin, gpu, ref): {rows}")

def test_unpack_fields_bit_exact(gpu):
    g = np.random.default_rng(100)
    W = np.concatenate([g.integers(0, 256, (3000, 144), dtype=np.uint8)] +
                       [b["bytes"][None] for b in golden_blocks.load()])
    nb = W.shape[0]
    announce(f"unpack_fields nblocks={nb}")
    q = torch.zeros(nb * 256, dtype=torch.uint8, device="cuda:0")
    sc = torch.zeros(nb * 8, dtype=torch.uint8, device="cuda:0")
    m = torch.zeros(nb * 8, dtype=torch.uint8, device="cuda:0")
    gpu.unpack_fields(dev(W), q, sc, m)
    rq, rsc, rm, _, _ = oracle.unpack_fields(W)
    assert np.array_equal(host(q).reshape(nb, 256), rq)
    assert np.array_equal(host(sc).reshape(nb, 8), rsc)
    assert np.array_equal(host(m).reshape(nb, 8), rm)


def test_dequant_f32_bit_exact(gpu):
    g = np.random.default_rng(101)
    W = np.concatenate([_special_blocks(g, 2000), qi.weight_bytes(g, 64, 2560).reshape(-1, 144)]
                       + [b["bytes"][None] for b in golden_blocks.load()])
    nb = W.shape[0]
    announce(f"dequant_f32 nblocks={nb}")
    w = torch.zeros(nb * 256, dtype=torch.float32, device="cuda:0")
    gpu.dequant_f32(dev(W), w)
    ref = oracle.dequant_f32(W)
    got = host(w)
    _assert_same_weights(got.view(np.uint32), ref.view(np.uint32), got == 0, ref == 0, W,
                         "dequant_f32")


def test_dequant_bf16_bit_exact(gpu):
    g = np.random.default_rng(102)
    W = np.concatenate([_special_blocks(g, 2000), qi.weight_bytes(g, 64, 2560).reshape(-1, 144)])
    nb = W.shape[0]
    announce(f"dequant_bf16 nblocks={nb}")
    w = torch.zeros(nb * 256, dtype=torch.int16, device="cuda:0")
    gpu.dequant_bf16(dev(W), w)
    got = host(w).view(np.uint16)
    ref = oracle.dequant_bf16(W)
    _assert_same_weights(got, ref, (got & 0x7FFF) == 0, (ref & 0x7FFF) == 0, W, "dequant_bf16")


# ------------------------------------------------------------ M = 1

def test_gemv_single_2560x2560(gpu):
    W, X = qi.single_gemv(0)
    announce("gemv 2560x2560 seed 0")
    y = run_gemm(W, X, 2560, 2560, path="gemv")
    Y, A = oracle.gemm(W, X, 2560, 2560)
    parity(y, Y, A, "gemv 2560x2560")


@pytest.mark.parametrize("N,K", [(1, 256), (3, 256), (17, 512), (255, 768), (1000, 2560),
                                 (129, 4096), (333, 9728), (64, 16384), (5, 1280)])
def test_gemv_ragged_shapes(gpu, N, K):
    g = np.random.default_rng([103, N, K])
    W = qi.weight_bytes(g, N, K)
    X = qi.activations(g, 1, K)
    announce(f"gemv N={N} K={K}")
    y = run_gemm(W, X, N, K, path="gemv")
    Y, A = oracle.gemm(W, X, N, K)
    parity(y, Y, A, f"gemv N={N} K={K}")


def test_gemv_decode_layer(gpu):
    for name, N, K, W, X in qi.decode_layer(1, 0, 1):
        announce(f"gemv decode layer {name} {N}x{K}")
        y = run_gemm(W, X, N, K, path="gemv")
        Y, A = oracle.gemm(W, X, N, K)
        parity(y, Y, A, f"decode {name}")


def test_gemv_one_hot_isolates_weights(gpu):
    """x = e_k gives y = column k of the fp32 weights, exactly: the only
    non-zero sub-block sum is S1 = q, S0 = 1, and d*sc*q - dmin*m is rounded
    once (fast path and exact recomputation alike).  Pins the kernel's
    mapping of k to block, quarter, nibble, sub-block and matrix-core operand
    position."""
    g = np.random.default_rng(104)
    N, K = 40, 512
    W = qi.weight_bytes(g, N, K)
    w = oracle.dequant_f32(W).reshape(N, K)
    for k in (0, 31, 32, 63, 64, 255, 256, 300, 511):
        X = np.zeros((1, K), np.uint16)
        X[0, k] = 0x3F80
        announce(f"gemv one-hot k={k}")
        y = run_gemm(W, X, N, K, path="gemv")
        assert np.array_equal(y[0], w[:, k]), k


def _zero_weight_matrix(g, N, K, d, kind):
    """N x K blocks that mix exactly-zero weights with ordinary ones, built by
    the oracle-side encoder.  kind 'zero': q = 0 and m = 0 with sc = 63 and
    dmin = d (a valid Q4_K block whose weights are all 0); 'cancel': in every
    sub-block q is a constant c and m = c*sc with dmin = d, so d*sc*q - dmin*m
    = 0 although both terms are large.  Rows 0..N/2 are entirely such blocks;
    in the other rows 7 of every block's 8 sub-blocks are, and one is random
    (the workload's d, sc, m, q)."""
    nb = N * (K // 256)
    dbits = pk.half_bits(np.full(nb, d))
    sc = np.full((nb, 8), 63)
    m = np.zeros((nb, 8), np.int64)
    q = np.zeros((nb, 8, 32), np.int64)
    if kind == "cancel":
        c = g.integers(1, 4, (nb, 8))
        sc = g.integers(1, 64, (nb, 8)) // c
        sc[sc == 0] = 1
        m = sc * c
        q[:] = c[:, :, None]
    rows_zero = N // 2
    live = np.arange(nb) >= rows_zero * (K // 256)
    s_live = g.integers(0, 8, nb)
    idx = np.flatnonzero(live)
    sc[idx, s_live[idx]] = g.integers(0, 64, idx.size)
    m[idx, s_live[idx]] = g.integers(0, 64, idx.size)
    q[idx, s_live[idx]] = g.integers(0, 16, (idx.size, 32))
    return pk.pack_blocks(dbits, dbits, sc, m, q.reshape(nb, 256)).reshape(N, -1), rows_zero


@pytest.mark.parametrize("kind", ["zero", "cancel"])
@pytest.mark.parametrize("d", [2e-3, 1e-2, 1.0])
@pytest.mark.parametrize("K", [2560, 9728])
def test_gemv_zero_weight_rows(gpu, kind, d, K):
    """Rows whose weights are exactly zero (and rows mostly so) with dense
    N(0,1) activations, through every M = 1 entry point: jq4k_gemv,
    jq4k_gemv_batched, jq4k_gemv_rmsnorm and jq4k_gemm_swiglu.  The oracle
    gives y = 0 and sum|w*x| = 0 there, so the bound leaves 1e-5; the kernel's
    binary16 weights are exactly 0, so y is exactly 0."""
    g = np.random.default_rng([140, K, int(d * 1e4), kind == "cancel"])
    N = 300
    W, rows_zero = _zero_weight_matrix(g, N, K, d, kind)
    X = qi.activations(g, 1, K)
    assert np.all(oracle.dequant_f32(W).reshape(N, K)[:rows_zero] == 0)
    Y, A = oracle.gemm(W, X, N, K)
    announce(f"gemv zero-weight rows kind={kind} d={d} K={K}")
    y = run_gemm(W, X, N, K, path="gemv")
    parity(y, Y, A, f"gemv zero rows {kind} d={d} K={K}")
    assert np.all(y[0, :rows_zero] == 0)
    # the grouped launch, with an ordinary problem beside it
    Wr = qi.weight_bytes(g, 77, 2560)
    Xr = qi.activations(g, 1, 2560)
    Yb = [torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda:0"),
          torch.full((1, 77), float("nan"), dtype=torch.float32, device="cuda:0")]
    gpu.gemv_batched([(dev(W), dev(X).view(torch.bfloat16), Yb[0]),
                      (dev(Wr), dev(Xr).view(torch.bfloat16), Yb[1])])
    parity(host(Yb[0]), Y, A, f"gemv batched zero rows {kind} d={d} K={K}")
    # with the RMSNorm prologue
    gamma = qi.f32_to_bf16_bits((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
    Yn = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda:0")
    gpu.gemv_rmsnorm(dev(W), dev(X).view(torch.bfloat16), dev(gamma).view(torch.bfloat16),
                     1e-6, Yn)
    Yr, Ar, _ = oracle.gemm_rmsnorm(W, X, gamma, 1e-6, N, K)
    yn = host(Yn)
    parity(yn, Yr, Ar, f"gemv rmsnorm zero rows {kind} d={d} K={K}")
    assert np.all(yn[0, :rows_zero] == 0)
    # SwiGLU with the zero-weight matrix as gate and as up
    Wo = qi.weight_bytes(g, N, K)
    _swiglu_check(gpu, W, Wo, X, N, K, f"zero-weight gate {kind} d={d}")
    _swiglu_check(gpu, Wo, W, X, N, K, f"zero-weight up {kind} d={d}")


def test_gemv_large_and_special_scales(gpu):
    """Blocks with d, dmin of both signs from binary16 subnormals up to 69
    (the largest weights, 69*63*15 = 65205, stay finite in binary16), and the
    golden blocks: every output within the bound."""
    g = np.random.default_rng(141)
    N, K = 200, 2560
    nb = N * K // 256
    W = g.integers(0, 256, (nb, 144), dtype=np.uint8)
    hdr = g.integers(0, 0x5450, (nb, 2)).astype(np.uint16)
    hdr |= (g.integers(0, 2, (nb, 2)) << 15).astype(np.uint16)
    W[:, 0:4] = hdr.view(np.uint8).reshape(nb, 4)
    W = W.reshape(N, -1)
    X = qi.activations(g, 1, K)
    announce("gemv large and special scales")
    y = run_gemm(W, X, N, K, path="gemv")
    Y, A = oracle.gemm(W, X, N, K)
    parity(y, Y, A, "gemv special scales")


def test_gemv_largest_weights(gpu):
    """The largest weights Q4_K can encode (d = dmin = +-65504, sc = m = 63:
    |w| up to 65504 * 63 * 16, beyond binary16's range) in rows of their own
    and beside ordinary rows: every output finite and within the bound."""
    g = np.random.default_rng(142)
    N, K = 64, 512
    W = qi.weight_bytes(g, N, K)
    for row, (d, dmin, q) in enumerate([(65504.0, 0.0, 15), (65504.0, 65504.0, 0),
                                        (-65504.0, 65504.0, 15), (65504.0, -65504.0, 7)]):
        big = pk.pack_blocks(pk.half_bits(np.array([d])), pk.half_bits(np.array([dmin])),
                             np.full((1, 8), 63), np.full((1, 8), 63), np.full((1, 256), q))
        W[5 + 9 * row, 0:144] = big[0]
        W[6 + 9 * row] = np.tile(big[0], K // 256)
    X = qi.activations(g, 1, K)
    announce("gemv largest weights")
    y = run_gemm(W, X, N, K, path="gemv")
    assert np.all(np.isfinite(y))
    Y, A = oracle.gemm(W, X, N, K)
    parity(y, Y, A, "gemv largest weights")


def test_gemv_activation_range(gpu):
    """Activations beyond binary16's range and across many binades inside one
    block of 256 (x is staged as binary16 with a power-of-two scale per
    block), and an all-zero x: every output within the bound."""
    g = np.random.default_rng(143)
    N, K = 300, 2560
    W = qi.weight_bytes(g, N, K)
    z = g.standard_normal(K)
    cases = {
        "huge": z * 1e30,
        "tiny": z * 1e-30,
        "beyond_f16": z * 7e4,
        "binades": z * np.exp2(g.integers(-40, 40, K)),
        "mixed_blocks": z * np.repeat(np.exp2(g.integers(-60, 60, K // 256)), 256),
        "zero": np.zeros(K),
    }
    for name, xv in cases.items():
        X = qi.f32_to_bf16_bits(xv.astype(np.float32))[None]
        announce(f"gemv activation range {name}")
        y = run_gemm(W, X, N, K, path="gemv")
        Y, A = oracle.gemm(W, X, N, K)
        parity(y, Y, A, f"gemv activations {name}")
        if name == "zero":
            assert np.all(y == 0)


def test_gemv_closed_form_constant_blocks(gpu):
    blk = [b for b in golden_blocks.load() if b["name"] == "closed_form"][0]["bytes"]
    N, K = 70, 2560
    W = np.tile(blk, (N, K // 256))
    X = np.full((1, K), 0x3F80, np.uint16)
    announce("gemv closed form")
    y = run_gemm(W, X, N, K, path="gemv")
    assert np.all(y == -10.0)


def test_gemv_batched_decode_layer(gpu):
    """One launch for the seven independent projections: every output equals
    the per-problem GEMV bit for bit, and meets the oracle bound."""
    layer = qi.decode_layer(1, 0, 1)
    g = np.random.default_rng(109)
    extra = [("odd", 77, 768, qi.weight_bytes(g, 77, 768), qi.activations(g, 1, 768)),
             ("empty", 0, 512, np.zeros((0, 288), np.uint8), qi.activations(g, 1, 512))]
    probs = layer + extra
    Wd = [dev(W) for _, N, K, W, _ in probs]
    Xd = [dev(X).view(torch.bfloat16) for *_, X in probs]
    Yb = [torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda:0")
          for _, N, *_ in probs]
    announce(f"gemv batched {len(probs)} problems")
    gpu.gemv_batched(list(zip(Wd, Xd, Yb)))
    for (name, N, K, W, X), wd, xd, yb in zip(probs, Wd, Xd, Yb):
        if N == 0:
            continue
        ys = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
        gpu.gemv(wd, xd, ys)
        got, single = host(yb), host(ys)
        assert np.array_equal(got.view(np.uint32), single.view(np.uint32)), name
        Y, A = oracle.gemm(W, X, N, K)
        parity(got, Y, A, f"batched {name}")
    # the launch queues the problems by K; the caller's order must not matter
    order = np.random.default_rng(110).permutation(len(probs))
    Yp = [torch.full((1, probs[i][1]), float("nan"), dtype=torch.float32, device="cuda:0")
          for i in order]
    announce("gemv batched, problems in another order")
    gpu.gemv_batched([(Wd[i], Xd[i], y) for i, y in zip(order, Yp)])
    for i, y in zip(order, Yp):
        assert np.array_equal(host(y).view(np.uint32), host(Yb[i]).view(np.uint32)), probs[i][0]


def test_gemv_batched_decode_step_groups(gpu):
    """The four dependent launches of a decode step (q|k|v, o, gate|up, down),
    each its own batched launch.  The smaller ones give fewer workgroups than
    CUs at the batch's usual rows and are spread over every CU with fewer
    rows per workgroup; every output still equals the per-problem GEMV bit
    for bit (a row's sums do not depend on the rows per workgroup) and meets
    the oracle bound."""
    layer = qi.decode_layer(1, 0, 1)
    for group in ((0, 1, 2), (3,), (4, 5), (6,)):
        probs = [layer[i] for i in group]
        Wd = [dev(W) for _, N, K, W, _ in probs]
        Xd = [dev(X).view(torch.bfloat16) for *_, X in probs]
        Yb = [torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda:0")
              for _, N, *_ in probs]
        announce(f"gemv batched decode-step group {[p[0] for p in probs]}")
        gpu.gemv_batched(list(zip(Wd, Xd, Yb)))
        for (name, N, K, W, X), wd, xd, yb in zip(probs, Wd, Xd, Yb):
            ys = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
            gpu.gemv(wd, xd, ys)
            got, single = host(yb), host(ys)
            assert np.array_equal(got.view(np.uint32), single.view(np.uint32)), name
            Y, A = oracle.gemm(W, X, N, K)
            parity(got, Y, A, f"decode-step group {name}")


def test_gemv_rows_per_block_any(gpu):
    """jq4k_gemv_rows at row counts from 1 (a workgroup's rounds mostly idle
    lanes, whose stores go to the spare slot) to the LDS budget's range:
    every output equals jq4k_gemv's bit for bit (a row's sums do not depend
    on the rows per workgroup) and meets the oracle bound."""
    import q4_weight_only_amd as jq4k
    g = np.random.default_rng(131)
    # rows within the 96 KiB LDS budget: up to ~560 at K = 2560, ~120 at 9728
    for N, K, rows in ((517, 2560, (1, 3, 16, 51, 200, 500)), (130, 9728, (1, 3, 16, 51, 120))):
        W = qi.weight_bytes(g, N, K)
        X = qi.activations(g, 1, K)
        wd, xd = dev(W), dev(X).view(torch.bfloat16)
        ref = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
        gpu.gemv(wd, xd, ref)
        Y, A = oracle.gemm(W, X, N, K)
        parity(host(ref), Y, A, f"gemv N={N} K={K}")
        for R in rows:
            announce(f"gemv_rows N={N} K={K} R={R}")
            y = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda:0")
            gpu.gemv_rows(wd, xd, y, R)
            assert np.array_equal(host(y).view(np.uint32), host(ref).view(np.uint32)), (N, K, R)
        # past the budget: refused before any launch
        with pytest.raises(jq4k.Jq4kError):
            gpu.gemv_rows(wd, xd, torch.empty((1, N), dtype=torch.float32, device="cuda:0"), 5000)


def test_gemv_batched_sixteen_problems(gpu):
    """A batched launch at its limit of 16 problems, of mixed shapes (rows 1
    to 3000, K 256 to 16384, a repeated x): each output equals the
    per-problem GEMV bit for bit and meets the oracle bound."""
    g = np.random.default_rng(132)
    shapes = [(1, 256), (2, 16384), (3000, 2560), (17, 768), (300, 4096), (64, 9728), (5, 512),
              (1000, 1024), (129, 2560), (7, 7680), (2048, 256), (31, 3072), (256, 5120),
              (90, 2560), (1, 1024), (700, 2304)]
    shared_x = qi.activations(g, 1, 2560)
    probs = []
    for N, K in shapes:
        X = shared_x if K == 2560 else qi.activations(g, 1, K)
        probs.append((N, K, qi.weight_bytes(g, N, K), X))
    Wd = [dev(W) for *_, W, _ in probs]
    Xd = [dev(X).view(torch.bfloat16) for *_, X in probs]
    Yb = [torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda:0")
          for N, *_ in probs]
    announce("gemv batched, 16 problems")
    gpu.gemv_batched(list(zip(Wd, Xd, Yb)))
    for (N, K, W, X), wd, xd, yb in zip(probs, Wd, Xd, Yb):
        ys = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
        gpu.gemv(wd, xd, ys)
        assert np.array_equal(host(yb).view(np.uint32), host(ys).view(np.uint32)), (N, K)
        Y, A = oracle.gemm(W, X, N, K)
        parity(host(yb), Y, A, f"batched N={N} K={K}")


# ------------------------------------------------------------ M > 1 (MFMA)

PATHS = ["mfma64", "mfma128", "mfma256", "mfma_big", "mfma_rw", "skinny"]


def _path(name):
    import q4_weight_only_amd as jq4k
    return {"mfma": jq4k.PATH_MFMA, "mfma64": jq4k.PATH_MFMA_T64,
            "mfma128": jq4k.PATH_MFMA_T128, "mfma256": jq4k.PATH_MFMA_T256,
            "skinny": jq4k.PATH_SKINNY, "mfma_big": jq4k.PATH_MFMA_BIG,
            "mfma_rw": jq4k.PATH_MFMA_RW}[name]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M,N,K", [(1, 37, 256), (2, 128, 256), (3, 130, 512), (17, 256, 768),
                                   (33, 300, 2560), (64, 129, 512), (65, 257, 256),
                                   (128, 64, 1024), (200, 383, 512), (300, 140, 256)])
def test_mfma_paths_ragged(gpu, path, M, N, K):
    g = np.random.default_rng([105, M, N, K])
    W = qi.weight_bytes(g, N, K)
    X = qi.activations(g, M, K)
    announce(f"{path} M={M} N={N} K={K}")
    if path == "skinny" and M > 64:
        # The small-M kernel takes at most 64 rows of X: the host refuses
        # the call with EINVAL before any launch.
        import q4_weight_only_amd as jq4k
        with pytest.raises(jq4k.Jq4kError) as e:
            run_gemm(W, X, N, K, path=_path(path))
        assert e.value.code == jq4k.EINVAL
        return
    y = run_gemm(W, X, N, K, path=_path(path))
    Y, A = oracle.gemm(W, X, N, K)
    parity(y, Y, A, f"{path} M={M} N={N} K={K}")


@pytest.mark.parametrize("path", PATHS)
def test_mfma_identity_probe(gpu, path):
    """X = I_K gives Y = bf16(w)^T exactly: every output is one weight (the
    small-M kernel takes the identity 64 rows at a time)."""
    g = np.random.default_rng(106)
    N, K = 48, 512
    W = qi.weight_bytes(g, N, K)
    wb = oracle.dequant_bf16(W).reshape(N, K)
    ref = (wb.astype(np.uint32) << 16).view(np.float32)
    rows = 64 if path == "skinny" else K
    for k0 in range(0, K, rows):
        X = np.zeros((rows, K), np.uint16)
        X[np.arange(rows), k0 + np.arange(rows)] = 0x3F80
        announce(f"{path} identity probe, k {k0}..{k0 + rows - 1}")
        y = run_gemm(W, X, N, K, path=_path(path))
        assert np.array_equal(y, ref.T[k0:k0 + rows])


@pytest.mark.parametrize("path", PATHS)
def test_mfma_identity_probe_special_blocks(gpu, path):
    """The identity probe on blocks whose d and dmin are subnormal, negative,
    zero or the largest finite binary16 values: every matmul path's own
    dequantisation (the binary16-subnormal form of the quants, widened by
    v_fma_mix_f32) gives the oracle's bf16 weights bit for bit (+0 and -0
    alike)."""
    g = np.random.default_rng(119)
    N, K = 48, 512
    W = _special_blocks(g, N * K // 256).reshape(N, K // 256 * 144)
    wb = oracle.dequant_bf16(W.reshape(-1, 144)).reshape(N, K)
    ref = (wb.astype(np.uint32) << 16).view(np.float32)
    rows = 64 if path == "skinny" else K
    for k0 in range(0, K, rows):
        X = np.zeros((rows, K), np.uint16)
        X[np.arange(rows), k0 + np.arange(rows)] = 0x3F80
        announce(f"{path} identity probe on special blocks, k {k0}..{k0 + rows - 1}")
        y = run_gemm(W, X, N, K, path=_path(path))
        assert np.all(np.isfinite(y))
        assert np.array_equal(y, ref.T[k0:k0 + rows])


@pytest.mark.parametrize("M", [2, 33, 300])
def test_gemm_auto_and_determinism(gpu, M):
    g = np.random.default_rng([107, M])
    N, K = 520, 2560
    W = qi.weight_bytes(g, N, K)
    X = qi.activations(g, M, K)
    announce(f"gemm auto M={M} twice")
    y1 = run_gemm(W, X, N, K)
    y2 = run_gemm(W, X, N, K)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    Y, A = oracle.gemm(W, X, N, K)
    parity(y1, Y, A, f"auto M={M}")


@pytest.mark.parametrize("seed,shapes,path", [
    # largest M below 512: the 128-row tile
    (110, [(300, 130, 512), (77, 384, 768), (129, 65, 256), (0, 64, 256), (256, 1000, 2560)],
     "PATH_MFMA_T128"),
    # largest M from 512: the 256-row wave-specialised kernel, ragged in M and N
    (111, [(600, 200, 512), (512, 130, 768), (1, 64, 256), (37, 300, 256), (259, 0, 512)],
     "PATH_MFMA_T256"),
    # largest M up to 64: the small-M kernel, whole K (no workspace)
    (112, [(33, 130, 2560), (64, 64, 768), (1, 300, 256), (17, 1000, 9728), (0, 64, 256)],
     "PATH_SKINNY"),
])
def test_gemm_batched_mixed_problems(gpu, seed, shapes, path):
    """One MFMA launch for independent problems of different shapes: each
    output meets the bound and equals the single-problem result on the same
    tile bit for bit."""
    g = np.random.default_rng(seed)
    probs = []
    for M, N, K in shapes:
        probs.append((M, N, K, qi.weight_bytes(g, N, K), qi.activations(g, M, K)))
    Wd = [dev(W) for *_, W, _ in probs]
    Xd = [dev(X).view(torch.bfloat16) for *_, X in probs]
    Yb = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
          for M, N, *_ in probs]
    announce(f"gemm batched {len(probs)} problems")
    gpu.gemm_batched(list(zip(Wd, Xd, Yb)))
    for (M, N, K, W, X), wd, xd, yb in zip(probs, Wd, Xd, Yb):
        if M == 0 or N == 0:
            continue
        ys = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        gpu.gemm(wd, xd, ys, path=getattr(gpu, path))
        got = host(yb)
        assert np.array_equal(got.view(np.uint32), host(ys).view(np.uint32)), (M, N, K)
        Y, A = oracle.gemm(W, X, N, K)
        parity(got, Y, A, f"gemm batched M={M} N={N} K={K}")


# ---------------------------------------------------------------------------
# Split K with a workspace (jq4k_gemm_batched_ws, M <= 64)

@pytest.mark.parametrize("seed,shapes", [
    # the down projection alone at M = 33: 40 tiles x 10 K ranges of 3 or 4 blocks
    (120, [(33, 2560, 9728)]),
    # small M, ragged N, K from one block to 64 (ragged ranges), an empty problem
    (121, [(1, 37, 2560), (5, 300, 4096), (64, 129, 9728), (17, 64, 256), (0, 64, 512),
           (33, 70, 16384)]),
])
def test_gemm_batched_ws_split_k(gpu, seed, shapes):
    """Every output of a split-K launch meets the bound.  The workspace
    starts with zero counters and NaN in the partial-tile storage (which is
    always written before it is read); a second identical call, with the
    counters left at zero by the first and last call's partials in place,
    gives the same bits."""
    g = np.random.default_rng(seed)
    probs = [(M, N, K, qi.weight_bytes(g, N, K), qi.activations(g, M, K)) for M, N, K in shapes]
    Wd = [dev(W) for *_, W, _ in probs]
    Xd = [dev(X).view(torch.bfloat16) for *_, X in probs]
    Yd = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
          for M, N, *_ in probs]
    triples = list(zip(Wd, Xd, Yd))
    n = gpu.gemm_workspace_size(triples)
    assert n > 0 and n % 4 == 0
    # an upper bound on the counter bytes: one int per tile of every problem
    tiles = sum(-(-M // 64) * -(-N // 64) for M, N, *_ in shapes)
    cbytes = min(n, (4 * tiles + 255) // 256 * 256)
    ws = torch.full((n // 4,), float("nan"), dtype=torch.float32, device="cuda:0")
    ws[:cbytes // 4] = 0
    ws = ws.view(torch.uint8)
    announce(f"gemm batched split-K {len(probs)} problems, workspace {n} bytes")
    gpu.gemm_batched_ws(triples, ws)
    first = [host(y) for y in Yd]
    for (M, N, K, W, X), got in zip(probs, first):
        if M == 0 or N == 0:
            continue
        Y, A = oracle.gemm(W, X, N, K)
        parity(got, Y, A, f"split-K M={M} N={N} K={K}")
    for y in Yd:
        y.fill_(float("nan"))
    announce("gemm batched split-K, second call on the same workspace")
    gpu.gemm_batched_ws(triples, ws)
    for y, f in zip(Yd, first):
        assert np.array_equal(host(y).view(np.uint32), f.view(np.uint32))


def test_prefill_m33_one_layer(gpu):
    for p in range(7):
        name, N, K, W, X = qi.prefill_projection(2, 0, p, 33)
        announce(f"prefill M=33 layer 0 {name} {N}x{K}")
        y = run_gemm(W, X, N, K)
        Y, A = oracle.gemm(W, X, N, K)
        parity(y, Y, A, f"M=33 {name}")


def _grouped_layer(gpu, projs, M, ws=False):
    """The seven projections of a layer in one grouped launch (as the
    benchmark times them: with a workspace, split K, at M <= 64); returns the
    host outputs."""
    Wd = [dev(W) for _, _, _, W, _ in projs]
    Xd = [dev(X).view(torch.bfloat16) for _, _, _, _, X in projs]
    Yd = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
          for _, N, _, _, _ in projs]
    triples = list(zip(Wd, Xd, Yd))
    if ws:
        n = gpu.gemm_workspace_size(triples)
        assert n > 0
        gpu.gemm_batched_ws(triples, torch.zeros(n, dtype=torch.uint8, device="cuda:0"))
    else:
        gpu.gemm_batched(triples)
    return [host(y) for y in Yd]


_ORACLE = {}


def _oracle_cached(key, W, X, N, K):
    """oracle.gemm of a full-size workload, computed once per test session
    (the M = 2048 projections serve the grouped layer, the 256 x 256 tile and
    the SwiGLU checks)."""
    if key not in _ORACLE:
        _ORACLE[key] = oracle.gemm(W, X, N, K)
    return _ORACLE[key]


def test_prefill_m2048_full(gpu):
    """M = 2048, one layer, one grouped launch (the 256-row tile): every
    output of every projection against the oracle."""
    projs = [qi.prefill_projection(3, 0, p, 2048) for p in range(7)]
    announce("prefill M=2048 layer 0, one grouped launch, every output")
    ys = _grouped_layer(gpu, projs, 2048)
    for p, ((name, N, K, W, X), y) in enumerate(zip(projs, ys)):
        Y, A = _oracle_cached(("m2048", p), W, X, N, K)
        parity(y, Y, A, f"M=2048 {name}")


def test_big_tile_m2048_full(gpu):
    """The 256 x 256 tile kernel at M = 2048 on the gate (K = 2560) and down
    (K = 9728) projections: every output against the oracle."""
    for p in (4, 6):
        name, N, K, W, X = qi.prefill_projection(3, 0, p, 2048)
        announce(f"big tile M=2048 {name}, every output")
        y = run_gemm(W, X, N, K, path=_path("mfma_big"))
        Y, A = _oracle_cached(("m2048", p), W, X, N, K)
        parity(y, Y, A, f"big tile M=2048 {name}")


def test_register_w_m2048_full(gpu):
    """The register-W kernel (256 x 256 tiles, W dequantised into operand registers) at
    M = 2048 on the gate (K = 2560) and down (K = 9728) projections: every
    output against the oracle."""
    for p in (4, 6):
        name, N, K, W, X = qi.prefill_projection(3, 0, p, 2048)
        announce(f"register-W tile M=2048 {name}, every output")
        y = run_gemm(W, X, N, K, path=_path("mfma_rw"))
        Y, A = _oracle_cached(("m2048", p), W, X, N, K)
        parity(y, Y, A, f"register-W tile M=2048 {name}")


def test_prefill_m33_all_layers_full(gpu):
    """M = 33 through all 36 layers (252 matmuls), each layer one grouped
    split-K launch with a workspace (down and v in 2 K ranges): every output of
    every projection against the oracle."""
    for layer in range(36):
        projs = [qi.prefill_projection(2, layer, p, 33) for p in range(7)]
        announce(f"prefill M=33 layer {layer}, one grouped split-K launch, every output")
        ys = _grouped_layer(gpu, projs, 33, ws=True)
        for (name, N, K, W, X), y in zip(projs, ys):
            Y, A = oracle.gemm(W, X, N, K)
            parity(y, Y, A, f"M=33 layer {layer} {name}")


@pytest.mark.parametrize("M", [1, 512])
def test_lm_head_full(gpu, M):
    """The 151936 x 2560 LM head at M = 1 (the GEMV) and M = 512 (X1 is row 0
    of X512): every output against the oracle."""
    W, X = qi.lm_head(4, 512)
    X = X[:M]
    N, K = 151936, 2560
    announce(f"LM head M={M}, every output")
    y = run_gemm(W, X, N, K)
    Y, A = oracle.gemm(W, X, N, K)
    parity(y, Y, A, f"LM head M={M}")


# ---------------------------------------------------------------------------
# SwiGLU of a gate/up pair (jq4k_gemm_swiglu)

def _swiglu_check(gpu, Wg, Wu, X, N, K, what, rows=None, ms=None):
    M = X.shape[0]
    H = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    announce(f"swiglu {what} M={M} N={N} K={K}")
    gpu.gemm_swiglu(dev(Wg), dev(Wu), dev(X).view(torch.bfloat16), H)
    h = host(H)
    assert np.all(np.isfinite(h)), what
    rows = np.arange(N) if rows is None else rows
    ms = np.arange(M) if ms is None else ms
    Href, G, U, Ag, Au = oracle.gemm_swiglu(Wg[rows], Wu[rows], X[ms], len(rows), K)
    tol = oracle.swiglu_tolerance(G, U, Ag, Au)
    err = np.abs(h[np.ix_(ms, rows)].astype(np.float64) - Href)
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} out of the SwiGLU bound"


@pytest.mark.parametrize("M,N,K", [(1, 1000, 512), (1, 300, 16384), (1, 77, 2560),
                                   (2, 200, 512), (33, 130, 768), (64, 64, 256),
                                   (65, 300, 512), (300, 129, 1024)])
def test_swiglu_ragged(gpu, M, N, K):
    g = np.random.default_rng(300 + M + N)
    Wg, Wu = qi.weight_bytes(g, N, K), qi.weight_bytes(g, N, K)
    _swiglu_check(gpu, Wg, Wu, qi.activations(g, M, K), N, K, "ragged")


def test_swiglu_decode_gate_up(gpu):
    """The decode layer's gate and up projections (9728 x 2560) at M = 1."""
    layer = qi.decode_layer(1, 0, 1)
    (_, N, K, Wg, X), (_, _, _, Wu, _) = layer[4], layer[5]
    _swiglu_check(gpu, Wg, Wu, X, N, K, "decode gate|up")


@pytest.mark.parametrize("M", [33, 2048])
def test_swiglu_prefill_gate_up_full(gpu, M):
    """gate|up of a layer at M = 33 (the 64-row tiles) and M = 2048 (the
    256-row kernel): every output against the oracle's silu(g) * u."""
    seed = 2 if M == 33 else 3
    _, N, K, Wg, X = qi.prefill_projection(seed, 0, 4, M)
    _, _, _, Wu, _ = qi.prefill_projection(seed, 0, 5, M)
    H = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    announce(f"swiglu prefill gate|up M={M}, every output")
    gpu.gemm_swiglu(dev(Wg), dev(Wu), dev(X).view(torch.bfloat16), H)
    h = host(H)
    # both matrices multiply the gate projection's X (the up projection's own
    # X of the workload is not used here)
    if M == 2048:
        G, Ag = _oracle_cached(("m2048", 4), Wg, X, N, K)
    else:
        G, Ag = oracle.gemm(Wg, X, N, K)
    U, Au = oracle.gemm(Wu, X, N, K)
    Href = oracle.silu(G) * U
    tol = oracle.swiglu_tolerance(G, U, Ag, Au)
    bad = np.abs(h.astype(np.float64) - Href) > tol
    assert not bad.any(), f"swiglu M={M}: {bad.sum()} of {bad.size} out of the SwiGLU bound"


def test_swiglu_quick_returns(gpu):
    """M == 0 or N == 0: nothing is launched, whatever the pointers."""
    assert gpu.raw().jq4k_gemm_swiglu(0, 0, 0, 0, 0, 5, 256, None) == 0
    assert gpu.raw().jq4k_gemm_swiglu(0, 0, 0, 0, 7, 0, 256, None) == 0


# ---------------------------------------------------------------------------
# RMSNorm fused ahead of the decode GEMV (jq4k_gemv_rmsnorm)

@pytest.mark.parametrize("N,K", [(2560, 2560), (1000, 512), (300, 16384), (1024, 9728), (7, 256)])
def test_gemv_rmsnorm(gpu, N, K):
    g = np.random.default_rng(500 + N)
    W = qi.weight_bytes(g, N, K)
    X = qi.activations(g, 1, K)
    gamma = qi.f32_to_bf16_bits((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
    eps = 1e-6
    Y = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda:0")
    announce(f"gemv rmsnorm N={N} K={K}")
    gpu.gemv_rmsnorm(dev(W), dev(X).view(torch.bfloat16), dev(gamma).view(torch.bfloat16),
                     eps, Y)
    Yr, A, _ = oracle.gemm_rmsnorm(W, X, gamma, eps, N, K)
    parity(host(Y), Yr, A, f"gemv rmsnorm N={N} K={K}")


def test_gemv_rmsnorm_scale_invariance(gpu):
    """x and 4x normalise to the same x_hat (eps = 0), so the outputs are
    identical bit for bit."""
    g = np.random.default_rng(510)
    N, K = 777, 2560
    W = qi.weight_bytes(g, N, K)
    X = qi.activations(g, 1, K)
    X4 = qi.f32_to_bf16_bits((qi.bf16_bits_to_f32(X) * 4.0).astype(np.float32))
    gamma = qi.f32_to_bf16_bits(np.ones(K, np.float32))
    outs = []
    for x in (X, X4):
        Y = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
        gpu.gemv_rmsnorm(dev(W), dev(x).view(torch.bfloat16), dev(gamma).view(torch.bfloat16),
                         0.0, Y)
        outs.append(host(Y))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def _rmsnorm_rows_gpu(gpu, X, gamma, eps, in_place=False):
    Xd = dev(X).view(torch.bfloat16)
    Xh = Xd if in_place else torch.full_like(Xd, float("nan"))
    gpu.rmsnorm_bf16(Xd, dev(gamma).view(torch.bfloat16), eps, Xh)
    return host(Xh.view(torch.int16)).view(np.uint16)


def _check_xhat(xh, X, gamma, eps, what):
    """x_hat from the GPU (fp32 arithmetic, then RNE to bf16) against the
    oracle's fp64 value: within half a bf16 ulp plus the fp32 error, and
    equal to the oracle's bf16 except where the fp64 value sits within that
    error of a rounding boundary."""
    ref64 = oracle.rmsnorm_f64(X, gamma, eps)
    ref = oracle.rmsnorm_bf16(X, gamma, eps)
    got = oracle.bf16_to_f64(xh).reshape(ref64.shape)
    err = np.abs(got - ref64)
    assert np.all(err <= np.abs(ref64) * (2.0 ** -8 + 2.0 ** -20) + 1e-30), what
    mismatch = np.mean(xh.reshape(ref.shape) != ref)
    assert mismatch < 1e-3, f"{what}: {mismatch:.2e} of x_hat off the oracle's rounding"


@pytest.mark.parametrize("M,K", [(1, 256), (3, 2560), (33, 2560), (64, 9728), (5, 16384),
                                 (2048, 2560)])
def test_rmsnorm_rows(gpu, M, K):
    g = np.random.default_rng([520, M, K])
    X = qi.activations(g, M, K)
    gamma = qi.f32_to_bf16_bits((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
    announce(f"rmsnorm rows M={M} K={K}")
    xh = _rmsnorm_rows_gpu(gpu, X, gamma, 1e-6)
    _check_xhat(xh, X, gamma, 1e-6, f"rmsnorm rows M={M} K={K}")


def test_rmsnorm_rows_in_place_and_edge_values(gpu):
    """In place gives the same bits; a zero row with eps = 0 gives NaN (0/0,
    as the oracle's definition), with eps > 0 zeros; scaling a row by 4
    leaves x_hat unchanged at eps = 0."""
    g = np.random.default_rng(521)
    M, K = 6, 2560
    X = qi.activations(g, M, K)
    X[1] = 0
    X[2] = qi.f32_to_bf16_bits((qi.bf16_bits_to_f32(X[3]) * 4.0).astype(np.float32))
    gamma = qi.f32_to_bf16_bits(np.ones(K, np.float32))
    announce("rmsnorm rows in place, zero row, scaled row")
    a = _rmsnorm_rows_gpu(gpu, X, gamma, 1e-6)
    b = _rmsnorm_rows_gpu(gpu, X, gamma, 1e-6, in_place=True)
    assert np.array_equal(a, b)
    assert np.all(a[1] == 0)
    z = _rmsnorm_rows_gpu(gpu, X, gamma, 0.0)
    assert np.array_equal(z[2], z[3])
    assert np.all(np.isnan(oracle.bf16_to_f64(z[1])))


def test_rmsnorm_rows_then_gemv_equals_fused(gpu):
    """The row norm followed by jq4k_gemv gives jq4k_gemv_rmsnorm's output bit
    for bit: the same x_hat, then the same GEMV."""
    g = np.random.default_rng(522)
    for N, K in ((2560, 2560), (1024, 9728)):
        W = qi.weight_bytes(g, N, K)
        X = qi.activations(g, 1, K)
        gamma = qi.f32_to_bf16_bits((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
        announce(f"rmsnorm rows + gemv vs fused, N={N} K={K}")
        xh = _rmsnorm_rows_gpu(gpu, X, gamma, 1e-6)
        y1 = run_gemm(W, xh.reshape(1, K), N, K)
        Y = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
        gpu.gemv_rmsnorm(dev(W), dev(X).view(torch.bfloat16), dev(gamma).view(torch.bfloat16),
                         1e-6, Y)
        assert np.array_equal(y1.view(np.uint32), host(Y).view(np.uint32))


def test_rmsnorm_rows_then_gemm_prefill_m33(gpu):
    """Prefill with the norm: row norm then the small-M matmul, against the
    oracle's norm-then-matmul (reading of the norm's rounding as for M = 1)."""
    g = np.random.default_rng(523)
    N, K, M = 1000, 2560, 33
    W = qi.weight_bytes(g, N, K)
    X = qi.activations(g, M, K)
    gamma = qi.f32_to_bf16_bits((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
    announce("rmsnorm rows + gemm M=33")
    xh = _rmsnorm_rows_gpu(gpu, X, gamma, 1e-6)
    y = run_gemm(W, xh.reshape(M, K), N, K)
    Yr, A, _ = oracle.gemm_rmsnorm(W, X, gamma, 1e-6, N, K)
    parity(y, Yr, A, "rmsnorm rows + gemm M=33")


# ---------------------------------------------------------------------------
# FP16 <-> INT8 KV-cache convert (jq4k_kv_quant_i8, jq4k_kv_dequant_f16)

def _kv_gpu(gpu, v):
    nvec, dim = v.shape
    vd = dev(v.view(np.int16))
    qd = torch.full((nvec, dim), 99, dtype=torch.int8, device="cuda:0")
    sd = torch.full((nvec,), float("nan"), dtype=torch.float32, device="cuda:0")
    gpu.kv_quant_i8(vd, qd, sd)
    back = torch.full((nvec, dim), -1, dtype=torch.int16, device="cuda:0")
    gpu.kv_dequant_f16(qd, sd, back)
    return host(qd), host(sd), host(back).view(np.uint16)


def _kv_check(gpu, v, what):
    announce(f"kv convert {what} nvec={v.shape[0]} dim={v.shape[1]}")
    q, s, back = _kv_gpu(gpu, v)
    q_ref, s_ref = oracle.kv_quant(v)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), what
    assert np.array_equal(q, q_ref), what
    assert np.array_equal(back, oracle.kv_dequant(q_ref, s_ref)), what


@pytest.mark.parametrize("dim", [8, 24, 64, 128, 136, 512])
@pytest.mark.parametrize("nvec", [1, 3, 17, 1000])
def test_kv_convert_bit_exact(gpu, dim, nvec):
    """Codes, scales and dequantised values bit-identical to the oracle,
    ragged in nvec (partial workgroups) and in dim (idle lanes of a group)."""
    v = qi.kv_vectors(qi.rng([130, dim, nvec]), nvec, dim)
    _kv_check(gpu, v, "ragged")


def test_kv_convert_edge_values(gpu):
    """Zero vectors, signed zeros, the fp16 extremes (65504, subnormals),
    exact ties at power-of-two scales, one nonzero value per vector (all
    finite: non-finite inputs are outside the contract)."""
    dim = 128
    g = qi.rng(131)
    rows = [np.zeros(dim), -np.zeros(dim), np.full(dim, 65504.0), np.full(dim, -6e-8),
            np.clip(g.standard_normal(dim) * 65000 / 4.5, -65504, 65504),
            g.standard_normal(dim) * 1e-6]
    tie = np.tile([127, -127, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5], dim // 8)
    rows += [tie * 2.0 ** k for k in (-10, -3, 0, 5)]
    one = np.zeros(dim)
    one[77] = -3.0
    rows.append(one)
    v = np.array(rows).astype(np.float16).view(np.uint16)
    _kv_check(gpu, v, "edge values")


def test_kv_convert_full_cache(gpu):
    """The whole 1024-token cache of the workload (36 layers x K, V x 8
    heads x 1024 tokens = 589,824 vectors of 128 values), in the launch the
    benchmark times: every code, scale and value against the oracle, then
    the GPU's own round trip (quantising its dequantised cache) gives the
    same codes."""
    v = qi.kv_cache(5)
    _kv_check(gpu, v, "full cache")
    q, s, back = _kv_gpu(gpu, v)
    q2, _, _ = _kv_gpu(gpu, back)
    assert np.array_equal(q2, q)
