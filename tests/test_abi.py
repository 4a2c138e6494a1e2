"""The C ABI of libjq4k on the CPU: the library loads, exports every symbol
include/jq4k.h declares, and rejects bad arguments before any HIP call (so
none of these tests launches anything)."""
import ctypes
import subprocess

import pytest

import q4_weight_only_amd as jq4k

ALIGNED = 0x10000          # fake, 16-byte aligned "device" addresses: never dereferenced
ALIGNED2 = 0x20000
ALIGNED3 = 0x30000
ALIGNED4 = 0x40000


@pytest.fixture(scope="module")
def L():
    return jq4k.raw()


def test_every_declared_symbol_is_exported(L):
    names = jq4k.declared_symbols()
    assert {"jq4k_gemv", "jq4k_gemm", "jq4k_gemm_path", "jq4k_unpack_fields",
            "jq4k_dequant_f32", "jq4k_dequant_bf16", "jq4k_strerror",
            "jq4k_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", jq4k.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_header_compiles_as_c_and_block_is_144_bytes(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "jq4k.h"\n'
                   'int size_ok[sizeof(block_q4_K) == 144 ? 1 : -1];\n'
                   'int main(void) { return 0; }\n')
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", jq4k.HEADER.rsplit("/", 1)[0],
                    str(src), "-o", str(tmp_path / "t")], check=True)


def test_version_and_strerror(L):
    assert jq4k.version() == 100
    assert jq4k.strerror(0) == "success"
    assert jq4k.strerror(-1) == "invalid argument"
    assert jq4k.strerror(-2) == "misaligned pointer"
    assert jq4k.strerror(-77) == "unknown error"


@pytest.mark.parametrize("M,N,K", [(1, 8, 0), (1, 8, -256), (1, 8, 100), (1, 8, 257),
                                   (-1, 8, 256), (1, -8, 256)])
def test_bad_sizes_are_rejected(L, M, N, K):
    for f in (L.jq4k_gemm, L.jq4k_gemv):
        assert f(ALIGNED, ALIGNED2, ALIGNED3, M, N, K, None) == jq4k.EINVAL


def test_gemv_requires_one_token_and_bounded_k(L):
    assert L.jq4k_gemv(ALIGNED, ALIGNED2, ALIGNED3, 2, 8, 256, None) == jq4k.EINVAL
    assert L.jq4k_gemv(ALIGNED, ALIGNED2, ALIGNED3, 0, 8, 256, None) == jq4k.EINVAL
    assert L.jq4k_gemv(ALIGNED, ALIGNED2, ALIGNED3, 1, 8, jq4k.GEMV_MAX_K + 256,
                       None) == jq4k.EINVAL
    assert L.jq4k_gemm_path(ALIGNED, ALIGNED2, ALIGNED3, 2, 8, 256, jq4k.PATH_GEMV,
                            None) == jq4k.EINVAL


def test_unknown_path_is_rejected(L):
    for path in (-1, jq4k.PATH_MFMA_RW + 1, 99):
        assert L.jq4k_gemm_path(ALIGNED, ALIGNED2, ALIGNED3, 4, 8, 256, path,
                                None) == jq4k.EINVAL
    # the small-M kernel takes M <= 64 only
    assert L.jq4k_gemm_path(ALIGNED, ALIGNED2, ALIGNED3, 65, 8, 256, jq4k.PATH_SKINNY,
                            None) == jq4k.EINVAL
    assert L.jq4k_gemm_path(ALIGNED, ALIGNED2, ALIGNED3, 0, 8, 256, jq4k.PATH_SKINNY,
                            None) == jq4k.OK


def test_null_pointers_are_rejected(L):
    for W, X, Y in ((0, ALIGNED2, ALIGNED3), (ALIGNED, 0, ALIGNED3), (ALIGNED, ALIGNED2, 0)):
        assert L.jq4k_gemm(W, X, Y, 3, 8, 256, None) == jq4k.EINVAL
        assert L.jq4k_gemv(W, X, Y, 1, 8, 256, None) == jq4k.EINVAL


def test_misaligned_pointers_are_rejected(L):
    cases = ((ALIGNED + 8, ALIGNED2, ALIGNED3), (ALIGNED, ALIGNED2 + 2, ALIGNED3),
             (ALIGNED, ALIGNED2, ALIGNED3 + 2), (ALIGNED + 1, ALIGNED2, ALIGNED3))
    for W, X, Y in cases:
        assert L.jq4k_gemm(W, X, Y, 3, 8, 256, None) == jq4k.EALIGN
        assert L.jq4k_gemv(W, X, Y, 1, 8, 256, None) == jq4k.EALIGN
    # Y needs only 4-byte alignment
    assert L.jq4k_gemm(ALIGNED, ALIGNED2, ALIGNED3 + 4, 0, 8, 256, None) == jq4k.OK


def test_empty_problems_return_without_launching(L):
    # null pointers are fine when there is nothing to compute
    assert L.jq4k_gemm(0, 0, 0, 0, 8, 256, None) == jq4k.OK
    assert L.jq4k_gemm(0, 0, 0, 5, 0, 256, None) == jq4k.OK
    assert L.jq4k_gemv(0, 0, 0, 1, 0, 256, None) == jq4k.OK
    for path in range(6):
        M = 1 if path == jq4k.PATH_GEMV else 0
        assert L.jq4k_gemm_path(0, 0, 0, M, 0, 512, path, None) == jq4k.OK


def test_export_argument_checks(L):
    assert L.jq4k_unpack_fields(ALIGNED, -1, ALIGNED2, ALIGNED3, ALIGNED3, None) == jq4k.EINVAL
    assert L.jq4k_unpack_fields(0, 0, 0, 0, 0, None) == jq4k.OK
    assert L.jq4k_unpack_fields(0, 3, ALIGNED2, ALIGNED3, ALIGNED3, None) == jq4k.EINVAL
    assert L.jq4k_unpack_fields(ALIGNED, 3, ALIGNED2, 0, ALIGNED3, None) == jq4k.EINVAL
    assert L.jq4k_unpack_fields(ALIGNED + 4, 3, ALIGNED2, ALIGNED3, ALIGNED3,
                                None) == jq4k.EALIGN
    for f in (L.jq4k_dequant_f32, L.jq4k_dequant_bf16):
        assert f(ALIGNED, -5, ALIGNED2, None) == jq4k.EINVAL
        assert f(ALIGNED, 0, 0, None) == jq4k.OK
        assert f(ALIGNED, 2, 0, None) == jq4k.EINVAL
        assert f(ALIGNED, 2, ALIGNED2 + 2, None) == jq4k.EALIGN
        assert f(ALIGNED + 8, 2, ALIGNED2, None) == jq4k.EALIGN


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(jq4k, "_raw", None)
    monkeypatch.setattr(jq4k, "LIB_PATH", "/nonexistent/libjq4k.so")
    with pytest.raises(ImportError):
        jq4k.raw()


def test_gemv_rows_argument_checks(L):
    f = L.jq4k_gemv_rows
    assert f(ALIGNED, ALIGNED2, ALIGNED3, 8, 256, -1, None) == jq4k.EINVAL
    assert f(ALIGNED, ALIGNED2, ALIGNED3, 8, 100, 4, None) == jq4k.EINVAL
    assert f(ALIGNED, ALIGNED2, ALIGNED3, 8, jq4k.GEMV_MAX_K + 256, 4, None) == jq4k.EINVAL
    # 4096 rows of K = 16384 need 1 MiB of partials: beyond the LDS budget
    assert f(ALIGNED, ALIGNED2, ALIGNED3, 8, 16384, 4096, None) == jq4k.EINVAL
    assert f(ALIGNED + 4, ALIGNED2, ALIGNED3, 8, 256, 4, None) == jq4k.EALIGN
    assert f(0, 0, 0, 0, 256, 4, None) == jq4k.OK


def _descs(*rows):
    arr = (jq4k.GemvDesc * max(len(rows), 1))()
    for i, r in enumerate(rows):
        arr[i] = jq4k.GemvDesc(*r)
    return arr


def test_gemv_batched_argument_checks(L):
    f = L.jq4k_gemv_batched
    good = (ALIGNED, ALIGNED2, ALIGNED3, 8, 256)
    assert f(None, 0, None) == jq4k.OK
    assert f(None, 2, None) == jq4k.EINVAL
    assert f(ctypes.addressof(_descs(good)), -1, None) == jq4k.EINVAL
    many = _descs(*([good] * 17))
    assert f(ctypes.addressof(many), 17, None) == jq4k.EINVAL
    for bad, code in (((ALIGNED, ALIGNED2, ALIGNED3, 8, 100), jq4k.EINVAL),
                      ((ALIGNED, ALIGNED2, ALIGNED3, -8, 256), jq4k.EINVAL),
                      ((ALIGNED, ALIGNED2, ALIGNED3, 8, jq4k.GEMV_MAX_K + 256), jq4k.EINVAL),
                      ((0, ALIGNED2, ALIGNED3, 8, 256), jq4k.EINVAL),
                      ((ALIGNED + 8, ALIGNED2, ALIGNED3, 8, 256), jq4k.EALIGN),
                      ((ALIGNED, ALIGNED2, ALIGNED3 + 1, 8, 256), jq4k.EALIGN)):
        arr = _descs(good, bad)          # one bad problem rejects the whole batch
        assert f(ctypes.addressof(arr), 2, None) == code, bad
    empty = _descs((0, 0, 0, 0, 256), (0, 0, 0, 0, 512))
    assert f(ctypes.addressof(empty), 2, None) == jq4k.OK


def test_mfma_k_limit(L):
    for path in (jq4k.PATH_AUTO, jq4k.PATH_MFMA, jq4k.PATH_MFMA_T64, jq4k.PATH_MFMA_T128,
                 jq4k.PATH_MFMA_T256):
        assert L.jq4k_gemm_path(ALIGNED, ALIGNED2, ALIGNED3, 4, 8, jq4k.MFMA_MAX_K + 256, path,
                                None) == jq4k.EINVAL


def test_gemm_batched_argument_checks(L):
    f = L.jq4k_gemm_batched

    def descs(*rows):
        arr = (jq4k.GemmDesc * max(len(rows), 1))()
        for i, r in enumerate(rows):
            arr[i] = jq4k.GemmDesc(*r)
        return arr
    good = (ALIGNED, ALIGNED2, ALIGNED3, 4, 8, 256)
    assert f(None, 0, None) == jq4k.OK
    assert f(None, 1, None) == jq4k.EINVAL
    assert f(ctypes.addressof(descs(good)), -1, None) == jq4k.EINVAL
    many = descs(*([good] * 17))
    assert f(ctypes.addressof(many), 17, None) == jq4k.EINVAL
    for bad, code in (((ALIGNED, ALIGNED2, ALIGNED3, 4, 8, 300), jq4k.EINVAL),
                      ((ALIGNED, ALIGNED2, ALIGNED3, -1, 8, 256), jq4k.EINVAL),
                      ((ALIGNED, 0, ALIGNED3, 4, 8, 256), jq4k.EINVAL),
                      ((ALIGNED, ALIGNED2 + 4, ALIGNED3, 4, 8, 256), jq4k.EALIGN),
                      ((ALIGNED, ALIGNED2, ALIGNED3, 4, 8, jq4k.MFMA_MAX_K + 256), jq4k.EINVAL)):
        assert f(ctypes.addressof(descs(good, bad)), 2, None) == code, bad
    empty = descs((0, 0, 0, 0, 8, 256), (0, 0, 0, 5, 0, 512))
    assert f(ctypes.addressof(empty), 2, None) == jq4k.OK


def _gemm_descs(*rows):
    arr = (jq4k.GemmDesc * max(len(rows), 1))()
    for i, r in enumerate(rows):
        arr[i] = jq4k.GemmDesc(*r)
    return arr


def _ws_size(L, arr, count):
    n = ctypes.c_size_t(12345)
    rc = L.jq4k_gemm_workspace_size(ctypes.addressof(arr) if arr is not None else None, count,
                                    ctypes.byref(n))
    return rc, n.value


def test_gemm_workspace_size(L):
    """Host-side sizing of the split-K workspace: the M = 33 layer splits
    down and v in 2 (with 256 compute units, the count this host assumes without a
    GPU); M > 64 or one short problem needs none."""
    A, B, C = ALIGNED, ALIGNED2, ALIGNED3
    layer = _gemm_descs(*[(A, B, C, 33, n, k) for n, k in
                          ((4096, 2560), (1024, 2560), (1024, 2560), (2560, 4096),
                           (9728, 2560), (9728, 2560), (2560, 9728))])
    rc, n = _ws_size(L, layer, 7)
    assert rc == jq4k.OK
    assert n == (56 * 4 + 255) // 256 * 256 + (16 + 40) * 2 * 64 * 64 * 4
    for rows in (((A, B, C, 65, 4096, 9728),), ((A, B, C, 8, 64, 256),), ()):
        rc, n = _ws_size(L, _gemm_descs(*rows), len(rows))
        assert (rc, n) == (jq4k.OK, 0), rows
    assert _ws_size(L, _gemm_descs((A, B, C, 4, 8, 300)), 1) == (jq4k.EINVAL, 0)
    assert _ws_size(L, _gemm_descs((A, B + 2, C, 4, 8, 256)), 1) == (jq4k.EALIGN, 0)
    assert _ws_size(L, None, 1) == (jq4k.EINVAL, 0)
    assert L.jq4k_gemm_workspace_size(ctypes.addressof(layer), 7, None) == jq4k.EINVAL


def test_gemm_batched_ws_argument_checks(L):
    """A needed workspace must be given, large enough and 256-byte aligned;
    every rejection happens before any launch."""
    f = L.jq4k_gemm_batched_ws
    A, B, C = ALIGNED, ALIGNED2, ALIGNED3
    down = _gemm_descs((A, B, C, 33, 2560, 9728))
    _, need = _ws_size(L, down, 1)
    assert need > 0
    WS = 0x100000000
    assert f(ctypes.addressof(down), 1, None, need, None) == jq4k.EINVAL
    assert f(ctypes.addressof(down), 1, WS, need - 1, None) == jq4k.EINVAL
    assert f(ctypes.addressof(down), 1, WS + 128, need, None) == jq4k.EALIGN
    assert f(None, 0, None, 0, None) == jq4k.OK
    assert f(None, 1, None, 0, None) == jq4k.EINVAL
    bad = _gemm_descs((A, B, C, 33, 2560, 9728), (A, B, C + 2, 33, 8, 256))
    assert f(ctypes.addressof(bad), 2, WS, 1 << 30, None) == jq4k.EALIGN
    empty = _gemm_descs((0, 0, 0, 0, 8, 256), (0, 0, 0, 5, 0, 512))
    assert f(ctypes.addressof(empty), 2, None, 0, None) == jq4k.OK


def test_gemm_swiglu_argument_checks(L):
    f = L.jq4k_gemm_swiglu
    A, B, C, D = ALIGNED, ALIGNED2, ALIGNED3, ALIGNED4
    assert f(A, B, C, D, 4, 8, 300, None) == jq4k.EINVAL          # K not a multiple of 256
    assert f(A, B, C, D, -1, 8, 256, None) == jq4k.EINVAL
    assert f(A, 0, C, D, 4, 8, 256, None) == jq4k.EINVAL           # no up matrix
    assert f(A, B + 4, C, D, 4, 8, 256, None) == jq4k.EALIGN       # up misaligned
    assert f(A + 4, B, C, D, 4, 8, 256, None) == jq4k.EALIGN
    assert f(A, B, C, D, 4, 8, jq4k.MFMA_MAX_K + 256, None) == jq4k.EINVAL
    assert f(0, 0, 0, 0, 0, 8, 256, None) == jq4k.OK               # M == 0
    assert f(0, 0, 0, 0, 3, 0, 256, None) == jq4k.OK               # N == 0


def test_gemv_rmsnorm_argument_checks(L):
    f = L.jq4k_gemv_rmsnorm
    A, B, C, D = ALIGNED, ALIGNED2, ALIGNED3, ALIGNED4
    assert f(A, B, C, 1e-6, D, 8, 300, None) == jq4k.EINVAL        # K not a multiple of 256
    assert f(A, B, C, -1.0, D, 8, 256, None) == jq4k.EINVAL        # eps < 0
    assert f(A, B, C, float("nan"), D, 8, 256, None) == jq4k.EINVAL
    assert f(A, B, C, float("inf"), D, 8, 256, None) == jq4k.EINVAL
    assert f(A, B, 0, 1e-6, D, 8, 256, None) == jq4k.EINVAL        # no gamma
    assert f(A, B, C + 4, 1e-6, D, 8, 256, None) == jq4k.EALIGN    # gamma misaligned
    assert f(A, B, C, 1e-6, D, 8, jq4k.GEMV_MAX_K + 256, None) == jq4k.EINVAL
    assert f(0, 0, 0, 1e-6, 0, 0, 256, None) == jq4k.OK            # N == 0


def test_rmsnorm_rows_argument_checks(L):
    f = L.jq4k_rmsnorm_bf16
    A, B, C = ALIGNED, ALIGNED2, ALIGNED3
    assert f(A, B, 1e-6, C, 4, 300, None) == jq4k.EINVAL          # K not a multiple of 256
    assert f(A, B, 1e-6, C, 4, 0, None) == jq4k.EINVAL
    assert f(A, B, 1e-6, C, 4, jq4k.GEMV_MAX_K + 256, None) == jq4k.EINVAL
    assert f(A, B, 1e-6, C, -1, 256, None) == jq4k.EINVAL         # M < 0
    assert f(A, B, -1.0, C, 4, 256, None) == jq4k.EINVAL          # eps < 0
    assert f(A, B, float("nan"), C, 4, 256, None) == jq4k.EINVAL
    assert f(A, B, float("inf"), C, 4, 256, None) == jq4k.EINVAL
    assert f(0, B, 1e-6, C, 4, 256, None) == jq4k.EINVAL           # null X
    assert f(A, 0, 1e-6, C, 4, 256, None) == jq4k.EINVAL           # null gamma
    assert f(A, B, 1e-6, 0, 4, 256, None) == jq4k.EINVAL           # null Xhat
    assert f(A + 8, B, 1e-6, C, 4, 256, None) == jq4k.EALIGN
    assert f(A, B + 2, 1e-6, C, 4, 256, None) == jq4k.EALIGN
    assert f(A, B, 1e-6, C + 4, 4, 256, None) == jq4k.EALIGN
    assert f(0, 0, 1e-6, 0, 0, 256, None) == jq4k.OK               # M == 0


def test_kv_convert_argument_checks(L):
    """dim a multiple of 8 in 8..512, nvec >= 0, non-null pointers, v
    16-byte / q 8-byte / scale 4-byte alignment; nvec == 0 is a no-op."""
    V, Q, S = ALIGNED, ALIGNED2, ALIGNED3
    for f, args in ((L.jq4k_kv_quant_i8, lambda v, q, s: (v, q, s)),
                    (L.jq4k_kv_dequant_f16, lambda v, q, s: (q, s, v))):
        call = lambda v, q, s, n, d: f(*args(v, q, s), n, d, None)
        for dim in (0, 4, 12, 520, 1024, -8):
            assert call(V, Q, S, 4, dim) == jq4k.EINVAL, dim
        assert call(V, Q, S, -1, 128) == jq4k.EINVAL
        assert call(V, Q, S, 0, 128) == jq4k.OK
        assert call(0, Q, S, 0, 128) == jq4k.OK
        for v, q, s in ((0, Q, S), (V, 0, S), (V, Q, 0)):
            assert call(v, q, s, 4, 128) == jq4k.EINVAL
        assert call(V + 8, Q, S, 4, 128) == jq4k.EALIGN
        assert call(V, Q + 4, S, 4, 128) == jq4k.EALIGN
        assert call(V, Q, S + 2, 4, 128) == jq4k.EALIGN
        assert call(V, Q, S, 1 << 62, 512) == jq4k.EINVAL


def test_binding_rejects_host_tensors_before_any_launch():
    """Host (CPU) tensors reach no kernel: every wrapper raises ValueError
    from its checks, before the C call (the kernels would take a host
    pointer as a device address).  No GPU is needed or touched."""
    torch = pytest.importorskip("torch")
    W = torch.zeros((8, 144), dtype=torch.uint8)
    X = torch.zeros((1, 256), dtype=torch.bfloat16)
    Y = torch.zeros((1, 8), dtype=torch.float32)
    g = torch.zeros(256, dtype=torch.bfloat16)
    cases = [
        ("gemv", lambda: jq4k.gemv(W, X, Y)),
        ("gemm", lambda: jq4k.gemm(W, X, Y)),
        ("gemm path", lambda: jq4k.gemm(W, X, Y, path=jq4k.PATH_SKINNY)),
        ("gemv_batched", lambda: jq4k.gemv_batched([(W, X, Y)])),
        ("gemm_batched", lambda: jq4k.gemm_batched([(W, X, Y)])),
        ("gemm_batched_ws", lambda: jq4k.gemm_batched_ws([(W, X, Y)], None)),
        ("gemv_rmsnorm", lambda: jq4k.gemv_rmsnorm(W, X, g, 1e-6, Y)),
        ("rmsnorm_bf16", lambda: jq4k.rmsnorm_bf16(X, g, 1e-6, X.clone())),
        ("gemm_swiglu", lambda: jq4k.gemm_swiglu(W, W.clone(), X, Y)),
        ("kv_quant_i8", lambda: jq4k.kv_quant_i8(torch.zeros((2, 8), dtype=torch.float16),
                                                 torch.zeros((2, 8), dtype=torch.int8),
                                                 torch.zeros(2))),
        ("kv_dequant_f16", lambda: jq4k.kv_dequant_f16(torch.zeros((2, 8), dtype=torch.int8),
                                                       torch.zeros(2),
                                                       torch.zeros((2, 8), dtype=torch.float16))),
        ("unpack_fields", lambda: jq4k.unpack_fields(W, torch.zeros(8 * 256, dtype=torch.uint8),
                                                     torch.zeros(64, dtype=torch.uint8),
                                                     torch.zeros(64, dtype=torch.uint8))),
        ("dequant_f32", lambda: jq4k.dequant_f32(W, torch.zeros(8 * 256))),
        ("dequant_bf16", lambda: jq4k.dequant_bf16(W, torch.zeros(8 * 256, dtype=torch.int16))),
    ]
    for name, call in cases:
        with pytest.raises(ValueError, match="GPU tensor"):
            call()
    # a non-contiguous view is refused too (checked first)
    with pytest.raises(ValueError, match="contiguous"):
        jq4k.gemv(W.t(), X, Y)


def test_noalloc_argument_checks(L):
    """jq4k_gemm_batched_noalloc rejects what jq4k_gemm_batched_ws rejects,
    and problems needing more than the static buffer, before any launch."""
    assert L.jq4k_gemm_batched_noalloc(None, 0, None) == 0
    assert L.jq4k_gemm_batched_noalloc(None, 1, None) == jq4k.EINVAL
    assert L.jq4k_gemm_batched_noalloc(None, -1, None) == jq4k.EINVAL
    arr = _gemm_descs((16, 16, 16, 33, 8, 100))
    assert L.jq4k_gemm_batched_noalloc(ctypes.addressof(arr), 1, None) == jq4k.EINVAL
    arr = _gemm_descs((17, 16, 16, 33, 8, 256))
    assert L.jq4k_gemm_batched_noalloc(ctypes.addressof(arr), 1, None) == jq4k.EALIGN
    big = _gemm_descs(*[(16, 16, 16, 64, 2560, 9728)] * 4)
    assert L.jq4k_gemm_batched_noalloc(ctypes.addressof(big), 4, None) == jq4k.ESCRATCH
    assert L.jq4k_strerror(jq4k.ESCRATCH).decode().startswith("problems need more")
