"""CPU oracle for the Q4_K weight-only matmul -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
imports, links or calls anything here, and this package shares no code with it.

Contents
  * ctypes wrappers over ``q4k_oracle.c`` (fp16/bf16 scalars, field unpack,
    fp32 dequant, bf16 and binary16 of the fp32 weight,
    fp64 contraction with sum |w*x|);
  * ctypes wrappers over ``kv_oracle.c`` (the FP16 <-> INT8 KV-cache convert:
    per-vector absmax scale, round-half-even codes, fp16 dequantisation);
  * ``q4k_pack`` -- an independent bit-writer that packs fields into blocks,
    and the min/max quantiser used for the round-trip invariant.

The format and the arithmetic are stated in the header of ``q4k_oracle.c``
(GGUF's Q4_K block, the format of the Qwen3-4B-Q4_K_M model named in the
genie-ai-runtime README, "At a glance").
"""
import ctypes
import os

import numpy as np

from . import build as _build

BLOCK_BYTES = 144
QK = 256

_lib = None


def lib():
    """Load liboracle_q4k.so, compiling it first only if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_float.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_float.restype = ctypes.c_float
        L.oracle_float_to_bf16_rne.argtypes = [ctypes.c_float]
        L.oracle_float_to_bf16_rne.restype = ctypes.c_uint16
        L.oracle_unpack_fields.argtypes = [u8p, ctypes.c_long, u8p, u8p, u8p,
                                           u16p, u16p]
        L.oracle_unpack_fields.restype = None
        L.oracle_dequant_f32.argtypes = [u8p, ctypes.c_long, f32p]
        L.oracle_dequant_f32.restype = None
        L.oracle_dequant_bf16.argtypes = [u8p, ctypes.c_long, u16p]
        L.oracle_dequant_bf16.restype = None
        L.oracle_gemm.argtypes = [u8p, u16p, f64p, f64p, ctypes.c_long,
                                  ctypes.c_long, ctypes.c_long]
        L.oracle_gemm.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        i8p = ctypes.POINTER(ctypes.c_int8)
        L.oracle_float_to_half_rne.argtypes = [ctypes.c_float]
        L.oracle_float_to_half_rne.restype = ctypes.c_uint16
        L.oracle_half_to_float.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_float.restype = ctypes.c_float
        L.oracle_kv_quant.argtypes = [u16p, ctypes.c_long, ctypes.c_int, i8p, f32p]
        L.oracle_kv_quant.restype = None
        L.oracle_kv_dequant.argtypes = [i8p, f32p, ctypes.c_long, ctypes.c_int, u16p]
        L.oracle_kv_dequant.restype = None
        _lib = L
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _blocks(W):
    W = np.ascontiguousarray(W, dtype=np.uint8)
    if W.size % BLOCK_BYTES:
        raise ValueError("weight bytes are not a whole number of 144-byte blocks")
    return W, W.size // BLOCK_BYTES


def half_to_double(h: int) -> float:
    return lib().oracle_half_to_double(int(h))


def bf16_to_float(b: int) -> float:
    return lib().oracle_bf16_to_float(int(b))


def float_to_bf16_rne(x) -> np.ndarray:
    """Vector of binary32 values -> bf16 bit patterns (uint16)."""
    x = np.asarray(x, dtype=np.float32).ravel()
    f = lib().oracle_float_to_bf16_rne
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def unpack_fields(W):
    """Per-block fields: q[nb,256], sc[nb,8], m[nb,8], d_bits[nb], dmin_bits[nb]."""
    W, nb = _blocks(W)
    q = np.zeros((nb, QK), np.uint8)
    sc = np.zeros((nb, 8), np.uint8)
    m = np.zeros((nb, 8), np.uint8)
    d = np.zeros(nb, np.uint16)
    dm = np.zeros(nb, np.uint16)
    lib().oracle_unpack_fields(_ptr(W, ctypes.c_uint8), nb, _ptr(q, ctypes.c_uint8),
                               _ptr(sc, ctypes.c_uint8), _ptr(m, ctypes.c_uint8),
                               _ptr(d, ctypes.c_uint16), _ptr(dm, ctypes.c_uint16))
    return q, sc, m, d, dm


def dequant_f32(W) -> np.ndarray:
    """fp32 weights, 256 per block, in block order."""
    W, nb = _blocks(W)
    w = np.zeros(nb * QK, np.float32)
    lib().oracle_dequant_f32(_ptr(W, ctypes.c_uint8), nb, _ptr(w, ctypes.c_float))
    return w


def dequant_bf16(W) -> np.ndarray:
    """bf16 (round-to-nearest-even) of the fp32 weights, as uint16 bits."""
    W, nb = _blocks(W)
    w = np.zeros(nb * QK, np.uint16)
    lib().oracle_dequant_bf16(_ptr(W, ctypes.c_uint8), nb, _ptr(w, ctypes.c_uint16))
    return w


def gemm(W, X_bf16, N: int, K: int):
    """Y = X . Wdq^T in fp64 and A = sum |w*x| (M x N each).

    W: uint8 bytes of N rows x K/256 blocks; X_bf16: uint16 array (M, K).
    """
    W, nb = _blocks(W)
    X = np.ascontiguousarray(X_bf16, dtype=np.uint16)
    if X.ndim == 1:
        X = X.reshape(1, -1)
    M = X.shape[0]
    if X.shape[1] != K or nb != N * (K // QK) or K % QK:
        raise ValueError("shape mismatch between W, X, N and K")
    Y = np.zeros((M, N), np.float64)
    A = np.zeros((M, N), np.float64)
    rc = lib().oracle_gemm(_ptr(W, ctypes.c_uint8), _ptr(X, ctypes.c_uint16),
                           _ptr(Y, ctypes.c_double), _ptr(A, ctypes.c_double),
                           M, N, K)
    if rc != 0:
        raise RuntimeError("oracle_gemm failed")
    return Y, A


def num_threads() -> int:
    return lib().oracle_num_threads()


def tolerance(A: np.ndarray) -> np.ndarray:
    """Per-element bound on |y_gpu - y_ref|: 2e-3 * sum|w*x| + 1e-5."""
    return 2e-3 * A + 1e-5


def within_tolerance(y, Y_ref, A) -> np.ndarray:
    """Boolean mask of the elements that satisfy the bound (NaN never does)."""
    y = np.asarray(y, np.float64)
    return np.abs(y - Y_ref) <= tolerance(A)


# ---------------------------------------------------------------------------
# SwiGLU of a gate/up pair (the genie-ai-runtime README, "At a glance": fused
# RMSNorm + RoPE + SwiGLU kernels; the pages do not define the function, and
# the reading taken is Qwen3's MLP activation, h = silu(g) * u with
# silu(z) = z * sigmoid(z), on the outputs g = X.Wg^T and u = X.Wu^T).

SILU_LIPSCHITZ = 1.0999  # max |silu'(z)| = 1.0998... (near z = 2.40)


def silu(z):
    """silu(z) = z / (1 + exp(-z)) in fp64 (exp(-z) may overflow to inf for
    very negative z, giving the correct limit -0)."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gemm_swiglu(Wg, Wu, X_bf16, N: int, K: int):
    """H = silu(X.Wg^T) * (X.Wu^T) in fp64, from two oracle contractions.
    Returns (H, G, U, Ag, Au): the fp64 gate and up outputs and their
    sum |w*x| are what the bound of swiglu_tolerance needs."""
    G, Ag = gemm(Wg, X_bf16, N, K)
    U, Au = gemm(Wu, X_bf16, N, K)
    return silu(G) * U, G, U, Ag, Au


def swiglu_tolerance(G, U, Ag, Au):
    """Per-element bound on |h_gpu - h_ref| for h = silu(g) * u, derived from
    the matmul bound tau = 2e-3 * A + 1e-5 on g and on u:
      |silu(g)u - silu(g*)u*| <= L tau_g (|u*| + tau_u) + |silu(g*)| tau_u,
    L = max |silu'|, plus 1e-6 |h*| for the fp32 evaluation of silu and the
    product on the GPU (a few rounding steps of 2^-24)."""
    tg, tu = tolerance(Ag), tolerance(Au)
    sg = np.abs(silu(G))
    return SILU_LIPSCHITZ * tg * (np.abs(U) + tu) + sg * tu + 1e-6 * sg * np.abs(U)


# ---------------------------------------------------------------------------
# RMSNorm of the activations ahead of a projection (the genie-ai-runtime
# README, "At a glance": fused RMSNorm + RoPE + SwiGLU kernels; the pages do
# not define it, and the reading taken is Qwen3's: x_hat = x / sqrt(mean(x^2)
# + eps) * gamma over the K inputs, stored as bf16 before the matmul, as an
# engine that keeps activations in bf16 would).

def bf16_to_f64(b):
    """bf16 bit patterns -> fp64 (exact): the 16 bits are the top half of a
    binary32."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rmsnorm_f64(X_bf16, gamma_bf16, eps: float):
    """x / sqrt(mean(x^2) + eps) * gamma per row, fp64 (rows of X)."""
    X = bf16_to_f64(X_bf16)
    g = bf16_to_f64(gamma_bf16)
    if X.ndim == 1:
        X = X.reshape(1, -1)
    r = 1.0 / np.sqrt(np.mean(X * X, axis=1, keepdims=True) + eps)
    return X * r * g


def rmsnorm_bf16(X_bf16, gamma_bf16, eps: float):
    """The normalised activations as bf16 bits: the fp64 value rounded to
    fp32, then to bf16 (round to nearest even)."""
    Xh = rmsnorm_f64(X_bf16, gamma_bf16, eps).astype(np.float32)
    return float_to_bf16_rne(Xh).reshape(Xh.shape)


def gemm_rmsnorm(W, X_bf16, gamma_bf16, eps: float, N: int, K: int):
    """Y = rmsnorm(X).W^T: the oracle contraction of the bf16 normalised
    activations; returns (Y, A, X_hat_bf16)."""
    Xh = rmsnorm_bf16(X_bf16, gamma_bf16, eps)
    Y, A = gemm(W, Xh, N, K)
    return Y, A, Xh


# ---------------------------------------------------------------------------
# FP16 <-> INT8 KV-cache convert (kv_oracle.c; genie-ai-runtime README,
# "Project layout" and "At a glance": INT8 KV cache with FP16-ULP-bounded
# drift).  One fp32 scale per KV vector (a token's head), s = max|v| / 127,
# codes rint(v / s), dequantised values fp16(fp32(q * s)).

KV_QMAX = 127


def float_to_half_rne(x: float) -> int:
    return int(lib().oracle_float_to_half_rne(float(x)))


def half_to_float(h: int) -> float:
    return float(lib().oracle_half_to_float(int(h)))


def kv_quant(v16):
    """v16: uint16 binary16 patterns, shape (nvec, dim).  Returns the int8
    codes (same shape) and the fp32 scale of every vector."""
    v16 = np.ascontiguousarray(v16, dtype=np.uint16)
    nvec, dim = v16.shape
    q = np.empty((nvec, dim), np.int8)
    s = np.empty(nvec, np.float32)
    lib().oracle_kv_quant(_ptr(v16, ctypes.c_uint16), nvec, dim, _ptr(q, ctypes.c_int8),
                          _ptr(s, ctypes.c_float))
    return q, s


def kv_dequant(q, s):
    """Codes (nvec, dim) int8 and scales (nvec,) fp32 -> binary16 patterns."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    nvec, dim = q.shape
    v = np.empty((nvec, dim), np.uint16)
    lib().oracle_kv_dequant(_ptr(q, ctypes.c_int8), _ptr(s, ctypes.c_float), nvec, dim,
                            _ptr(v, ctypes.c_uint16))
    return v
