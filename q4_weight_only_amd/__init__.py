"""Python binding of libjq4k (Q4_K weight-only matmul for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libjq4k.so; torch supplies device memory and the current stream.
There is no fallback -- if the library is not built, loading fails loudly.

    import q4_weight_only_amd as jq4k
    jq4k.gemm(W, X, Y)     # W uint8 (N, K/256*144), X bf16 (M, K), Y fp32 (M, N)

The C entry points (include/jq4k.h) are also exposed with the same names and
raw integer pointers in ``jq4k.raw``.
"""
import ctypes
import glob
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libjq4k.so")
HEADER = os.path.join(HERE, "..", "include", "jq4k.h")

OK, EINVAL, EALIGN, ESCRATCH = 0, -1, -2, -3
SCRATCH_BYTES = 8 << 20
(PATH_AUTO, PATH_GEMV, PATH_MFMA, PATH_MFMA_T64, PATH_MFMA_T128, PATH_MFMA_T256, PATH_SKINNY,
 PATH_MFMA_BIG, PATH_MFMA_RW) = range(9)
GEMV_MAX_K = 16384
MFMA_MAX_K = 4194304
BLOCK_BYTES = 144
QK = 256


class GemvDesc(ctypes.Structure):
    """jq4k_gemv_desc: one problem of jq4k_gemv_batched."""
    _fields_ = [("W", ctypes.c_void_p), ("X", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("N", ctypes.c_int), ("K", ctypes.c_int)]


GEMV_BATCH_MAX = 16


class GemmDesc(ctypes.Structure):
    """jq4k_gemm_desc: one problem of jq4k_gemm_batched."""
    _fields_ = [("W", ctypes.c_void_p), ("X", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("M", ctypes.c_int), ("N", ctypes.c_int), ("K", ctypes.c_int)]


GEMM_BATCH_MAX = 16


class Jq4kError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


_raw = None


def _load():
    global _raw
    if _raw is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libjq4k.so is not built ({LIB_PATH}); run "
                "`python q4_weight_only_amd/build.py` or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, l = ctypes.c_void_p, ctypes.c_int, ctypes.c_long
        for name in ("jq4k_gemv", "jq4k_gemm"):
            f = getattr(L, name)
            f.argtypes = [vp, vp, vp, i, i, i, vp]
            f.restype = i
        L.jq4k_gemv_rows.argtypes = [vp, vp, vp, i, i, i, vp]
        L.jq4k_gemv_rows.restype = i
        L.jq4k_gemv_batched.argtypes = [vp, i, vp]
        L.jq4k_gemv_batched.restype = i
        L.jq4k_gemm_batched.argtypes = [vp, i, vp]
        L.jq4k_gemm_batched.restype = i
        L.jq4k_gemm_batched_ws.argtypes = [vp, i, vp, ctypes.c_size_t, vp]
        L.jq4k_gemm_batched_ws.restype = i
        L.jq4k_gemm_batched_noalloc.argtypes = [vp, i, vp]
        L.jq4k_gemm_batched_noalloc.restype = i
        L.jq4k_gemm_workspace_size.argtypes = [vp, i, ctypes.POINTER(ctypes.c_size_t)]
        L.jq4k_gemm_workspace_size.restype = i
        L.jq4k_kv_quant_i8.argtypes = [vp, vp, vp, l, i, vp]
        L.jq4k_kv_quant_i8.restype = i
        L.jq4k_kv_dequant_f16.argtypes = [vp, vp, vp, l, i, vp]
        L.jq4k_kv_dequant_f16.restype = i
        L.jq4k_gemm_path.argtypes = [vp, vp, vp, i, i, i, i, vp]
        L.jq4k_gemm_swiglu.argtypes = [vp, vp, vp, vp, i, i, i, vp]
        L.jq4k_gemm_swiglu.restype = i
        L.jq4k_gemv_rmsnorm.argtypes = [vp, vp, vp, ctypes.c_float, vp, i, i, vp]
        L.jq4k_gemv_rmsnorm.restype = i
        L.jq4k_rmsnorm_bf16.argtypes = [vp, vp, ctypes.c_float, vp, i, i, vp]
        L.jq4k_rmsnorm_bf16.restype = i
        L.jq4k_gemm_path.restype = i
        L.jq4k_unpack_fields.argtypes = [vp, l, vp, vp, vp, vp]
        L.jq4k_unpack_fields.restype = i
        L.jq4k_dequant_f32.argtypes = [vp, l, vp, vp]
        L.jq4k_dequant_f32.restype = i
        L.jq4k_dequant_bf16.argtypes = [vp, l, vp, vp]
        L.jq4k_dequant_bf16.restype = i
        L.jq4k_probe_read.argtypes = [vp, ctypes.c_size_t, vp, i, vp]
        L.jq4k_probe_read.restype = i
        L.jq4k_probe_stream.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.jq4k_probe_stream.restype = i
        L.jq4k_probe_mfma.argtypes = [l, vp, i, vp]
        L.jq4k_probe_mfma.restype = i
        L.jq4k_probe_mmq.argtypes = [l, vp, i, vp]
        L.jq4k_probe_mmq.restype = i
        L.jq4k_strerror.argtypes = [i]
        L.jq4k_strerror.restype = ctypes.c_char_p
        L.jq4k_version.argtypes = []
        L.jq4k_version.restype = i
        _raw = L
    return _raw


def raw():
    """The loaded ctypes library (C names, raw pointers)."""
    return _load()


def declared_symbols():
    """Function names that the headers under include/ declare."""
    names = set()
    for path in sorted(glob.glob(os.path.join(os.path.dirname(HEADER), "*.h"))):
        with open(path) as f:
            text = f.read()
        names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(jq4k_\w+)\s*\(", text, re.M))
    return sorted(names)


def strerror(code: int) -> str:
    return _load().jq4k_strerror(int(code)).decode()


def version() -> int:
    return _load().jq4k_version()


def _check(rc, where):
    if rc != 0:
        raise Jq4kError(rc, where)


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _on_device(**tensors):
    """Every tensor must live in the memory of the current GPU: the kernels
    take raw device pointers, and a host or other-device pointer would fault
    the GPU instead of raising here."""
    import torch
    dev = None
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (got one on {t.device})")
        if dev is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the current device is {dev}")


def _dtype(name, t, *allowed):
    if t.dtype not in allowed:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {allowed}")


def _shapes(W, X, Y):
    import torch
    _on_device(W=W, X=X, Y=Y)
    if X.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("X must hold bfloat16 values (bf16 or raw 16-bit)")
    if W.dtype != torch.uint8 or Y.dtype != torch.float32:
        raise TypeError("W must be uint8 block bytes and Y float32")
    for name, t in (("W", W), ("X", X), ("Y", Y)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if X.dim() == 1:
        M, K, N = 1, X.numel(), Y.numel()
    else:
        M, K = X.shape
        N = Y.shape[-1] if Y.dim() == 2 else Y.numel() // max(M, 1)
    if W.numel() != N * (K // QK) * BLOCK_BYTES or Y.numel() != M * N:
        raise ValueError("W, X, Y sizes disagree")
    return int(M), int(N), int(K)


def gemv(W, X, Y, stream=None):
    """Y[0, :] = X[0, :] . W^T for one token (jq4k_gemv)."""
    M, N, K = _shapes(W, X, Y)
    _check(_load().jq4k_gemv(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, N, K,
                             _stream(stream)), "jq4k_gemv")
    return Y


def gemv_rows(W, X, Y, rows_per_block, stream=None):
    """jq4k_gemv with an explicit number of rows of W per workgroup (0: the
    library's choice); the results do not depend on it."""
    M, N, K = _shapes(W, X, Y)
    if M != 1:
        raise ValueError("gemv_rows takes one token (M = 1)")
    _check(_load().jq4k_gemv_rows(W.data_ptr(), X.data_ptr(), Y.data_ptr(), N, K,
                                  int(rows_per_block), _stream(stream)), "jq4k_gemv_rows")
    return Y


def gemv_descs(problems):
    """ctypes array of GemvDesc from (W, X, Y) torch tensor triples."""
    arr = (GemvDesc * max(len(problems), 1))()
    for i, (W, X, Y) in enumerate(problems):
        M, N, K = _shapes(W, X, Y)
        if M != 1:
            raise ValueError("batched GEMV problems have one token")
        arr[i] = GemvDesc(W.data_ptr(), X.data_ptr(), Y.data_ptr(), N, K)
    return arr


def gemv_batched(problems, stream=None):
    """One launch for several independent GEMVs: problems = [(W, X, Y), ...]."""
    arr = gemv_descs(problems)
    _check(_load().jq4k_gemv_batched(ctypes.addressof(arr), len(problems), _stream(stream)),
           "jq4k_gemv_batched")


def gemm_descs(problems):
    """ctypes array of GemmDesc from (W, X, Y) torch tensor triples."""
    arr = (GemmDesc * max(len(problems), 1))()
    for i, (W, X, Y) in enumerate(problems):
        M, N, K = _shapes(W, X, Y)
        arr[i] = GemmDesc(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, N, K)
    return arr


def gemm_batched(problems, stream=None):
    """One MFMA launch for several independent matmuls: [(W, X, Y), ...]."""
    arr = gemm_descs(problems)
    _check(_load().jq4k_gemm_batched(ctypes.addressof(arr), len(problems), _stream(stream)),
           "jq4k_gemm_batched")


def gemm_workspace_size(problems):
    """Bytes of workspace jq4k_gemm_batched_ws needs for [(W, X, Y), ...]."""
    arr = gemm_descs(problems)
    n = ctypes.c_size_t(0)
    _check(_load().jq4k_gemm_workspace_size(ctypes.addressof(arr), len(problems),
                                            ctypes.byref(n)), "jq4k_gemm_workspace_size")
    return n.value


def gemm_batched_ws(problems, workspace, stream=None):
    """jq4k_gemm_batched with a workspace (split K at M <= 64): `workspace`
    is a device tensor of at least gemm_workspace_size(problems) bytes,
    zero-filled before its first use (torch.zeros), or None when that size
    is 0."""
    arr = gemm_descs(problems)
    ptr, nbytes = None, 0
    if workspace is not None:
        _on_device(workspace=workspace)
        ptr, nbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(_load().jq4k_gemm_batched_ws(ctypes.addressof(arr), len(problems), ptr, nbytes,
                                        _stream(stream)), "jq4k_gemm_batched_ws")


def gemm_batched_noalloc(problems, stream=None):
    """jq4k_gemm_batched_ws with the library's static per-GPU scratch buffer
    as the workspace (allocates nothing; calls on one GPU must not overlap)."""
    arr = gemm_descs(problems)
    _check(_load().jq4k_gemm_batched_noalloc(ctypes.addressof(arr), len(problems),
                                             _stream(stream)), "jq4k_gemm_batched_noalloc")


def gemm(W, X, Y, stream=None, path=PATH_AUTO):
    """Y = X . W^T (jq4k_gemm, or jq4k_gemm_path with an explicit kernel path)."""
    M, N, K = _shapes(W, X, Y)
    L = _load()
    if path == PATH_AUTO:
        rc = L.jq4k_gemm(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, N, K, _stream(stream))
    else:
        rc = L.jq4k_gemm_path(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, N, K, int(path),
                              _stream(stream))
    _check(rc, "jq4k_gemm")
    return Y


def gemv_rmsnorm(W, X, gamma, eps, Y, stream=None):
    """Y = W . bf16(rmsnorm(x) * gamma) at M = 1 (jq4k_gemv_rmsnorm)."""
    import torch
    M, N, K = _shapes(W, X, Y)
    _on_device(gamma=gamma)
    _dtype("gamma", gamma, torch.bfloat16, torch.int16, torch.uint16)
    if M != 1 or gamma.numel() != K:
        raise ValueError("gemv_rmsnorm takes one token and K gamma values")
    _check(_load().jq4k_gemv_rmsnorm(W.data_ptr(), X.data_ptr(), gamma.data_ptr(), float(eps),
                                     Y.data_ptr(), N, K, _stream(stream)), "jq4k_gemv_rmsnorm")
    return Y


def rmsnorm_bf16(X, gamma, eps, Xhat, stream=None):
    """Xhat = bf16(rmsnorm(X) * gamma) row by row (jq4k_rmsnorm_bf16); X and
    Xhat are M x K bf16 (Xhat may be X), gamma K bf16 values."""
    import torch
    _on_device(X=X, gamma=gamma, Xhat=Xhat)
    for name, t in (("X", X), ("gamma", gamma), ("Xhat", Xhat)):
        _dtype(name, t, torch.bfloat16, torch.int16, torch.uint16)
    if X.dim() != 2 or Xhat.shape != X.shape or gamma.numel() != X.shape[1]:
        raise ValueError("rmsnorm_bf16 takes X and Xhat of one M x K shape and K gamma values")
    M, K = X.shape
    _check(_load().jq4k_rmsnorm_bf16(X.data_ptr(), gamma.data_ptr(), float(eps), Xhat.data_ptr(),
                                     M, K, _stream(stream)), "jq4k_rmsnorm_bf16")
    return Xhat


def gemm_swiglu(Wg, Wu, X, H, stream=None):
    """H = silu(X . Wg^T) * (X . Wu^T) (jq4k_gemm_swiglu); Wg and Wu alike."""
    import torch
    M, N, K = _shapes(Wg, X, H)
    _on_device(Wu=Wu)
    _dtype("Wu", Wu, torch.uint8)
    if Wu.shape != Wg.shape:
        raise ValueError("gate and up matrices differ in shape")
    _check(_load().jq4k_gemm_swiglu(Wg.data_ptr(), Wu.data_ptr(), X.data_ptr(), H.data_ptr(),
                                    M, N, K, _stream(stream)), "jq4k_gemm_swiglu")
    return H


def kv_quant_i8(v, q, scale, stream=None):
    """FP16 -> INT8 KV convert: v (nvec, dim) float16 or int16/uint16 bit
    patterns, q (nvec, dim) int8, scale (nvec,) float32, all device tensors."""
    import torch
    _on_device(v=v, q=q, scale=scale)
    _dtype("v", v, torch.float16, torch.int16, torch.uint16)
    _dtype("q", q, torch.int8)
    _dtype("scale", scale, torch.float32)
    nvec, dim = v.shape
    if q.shape != v.shape or scale.numel() != nvec:
        raise ValueError("kv_quant_i8 takes v and q of one shape and one scale per vector")
    _check(_load().jq4k_kv_quant_i8(v.data_ptr(), q.data_ptr(), scale.data_ptr(), nvec, dim,
                                    _stream(stream)), "jq4k_kv_quant_i8")


def kv_dequant_f16(q, scale, v, stream=None):
    """INT8 -> FP16 KV convert (the inverse mapping of kv_quant_i8's codes)."""
    import torch
    _on_device(q=q, scale=scale, v=v)
    _dtype("v", v, torch.float16, torch.int16, torch.uint16)
    _dtype("q", q, torch.int8)
    _dtype("scale", scale, torch.float32)
    nvec, dim = q.shape
    if v.shape != q.shape or scale.numel() != nvec:
        raise ValueError("kv_dequant_f16 takes q and v of one shape and one scale per vector")
    _check(_load().jq4k_kv_dequant_f16(q.data_ptr(), scale.data_ptr(), v.data_ptr(), nvec, dim,
                                       _stream(stream)), "jq4k_kv_dequant_f16")


def _nblocks(W, **outs):
    import torch
    _on_device(W=W, **outs)
    _dtype("W", W, torch.uint8)
    if W.numel() % BLOCK_BYTES:
        raise ValueError("W is not a whole number of 144-byte blocks")
    return W.numel() // BLOCK_BYTES


def unpack_fields(W, q, sc, m, stream=None):
    nb = _nblocks(W, q=q, sc=sc, m=m)
    if q.numel() != nb * QK or sc.numel() != nb * 8 or m.numel() != nb * 8:
        raise ValueError("output sizes disagree with W")
    _check(_load().jq4k_unpack_fields(W.data_ptr(), nb, q.data_ptr(), sc.data_ptr(),
                                      m.data_ptr(), _stream(stream)), "jq4k_unpack_fields")


def dequant_f32(W, w, stream=None):
    nb = _nblocks(W, w=w)
    if w.numel() != nb * QK:
        raise ValueError("output size disagrees with W")
    _check(_load().jq4k_dequant_f32(W.data_ptr(), nb, w.data_ptr(), _stream(stream)),
           "jq4k_dequant_f32")


def dequant_bf16(W, w, stream=None):
    nb = _nblocks(W, w=w)
    if w.numel() != nb * QK:
        raise ValueError("output size disagrees with W")
    _check(_load().jq4k_dequant_bf16(W.data_ptr(), nb, w.data_ptr(), _stream(stream)),
           "jq4k_dequant_bf16")

