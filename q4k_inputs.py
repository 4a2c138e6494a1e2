"""Seeded synthetic inputs for the Q4_K weight-only matmul.

This module is shared by the tests, the smoke check and the benchmark, and it
holds none of the method's arithmetic: it draws raw block bytes and bf16
activation bit patterns, nothing else.

Weights.  Each 144-byte Q4_K block gets
  * d and dmin: binary16 of |z| * 2e-3, z ~ N(0, 1) drawn in fp64 (numpy's
    correctly rounded fp64 -> fp16 conversion);
  * the 12 scale bytes and the 128 quant bytes: independent uniform bytes.
The packing of sixteen 6-bit fields into 12 bytes and of 256 nibbles into 128
bytes maps every field bit to exactly one byte bit, so uniform random bytes
are the same distribution as independent uniform sc, m in 0..63 and q in
0..15 -- the value distributions of the Qwen3-4B-shaped workloads.

Activations.  x = bf16(z), z ~ N(0, 1) drawn in fp32, rounded to nearest even.

Workloads (shapes of Qwen3-4B, whose CLI banner in the genie-ai-runtime README
reports 36 layers, 2560 hidden): projections q 4096x2560, k 1024x2560,
v 1024x2560, o 2560x4096, gate 9728x2560, up 9728x2560, down 2560x9728 (N x K),
and a Q4_K LM head 151936x2560.

KV cache.  FP16 KV vectors of 128 values (one token's head; the README's CLI
banner gives 8 KV heads, and Qwen3-4B's head size is 128), for 36 layers x
K and V x 8 heads x 1024 tokens (the README's KV pool is sized at 1024
context): 589,824 vectors.  Values are binary16 of s_v * z, z ~ N(0, 1), with
one magnitude s_v per vector drawn log-uniform in [2^-4, 2^4], and a few
outlier values per vector times 8 (attention activations have a heavy tail).
"""
import numpy as np

BLOCK_BYTES = 144
QK = 256

# (name, N, K) in layer order; the index is the projection id used in seeds.
PROJECTIONS = [
    ("q", 4096, 2560),
    ("k", 1024, 2560),
    ("v", 1024, 2560),
    ("o", 2560, 4096),
    ("gate", 9728, 2560),
    ("up", 9728, 2560),
    ("down", 2560, 9728),
]
N_LAYERS = 36
LM_HEAD = ("lm_head", 151936, 2560)


def rng(seed):
    return np.random.default_rng(seed)


def weight_bytes(g, N, K):
    """uint8 array (N, K/256*144): N rows of K/256 Q4_K blocks."""
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    nb = K // QK
    dz = np.abs(g.standard_normal((N, nb, 2))) * 2e-3
    hdr = dz.astype(np.float16).view(np.uint16)          # (N, nb, 2)
    body = g.integers(0, 256, size=(N, nb, 140), dtype=np.uint8)
    out = np.empty((N, nb, BLOCK_BYTES), np.uint8)
    out[:, :, 0:4] = hdr.view(np.uint8).reshape(N, nb, 4)  # little-endian d, dmin
    out[:, :, 4:] = body
    return out.reshape(N, nb * BLOCK_BYTES)


def f32_to_bf16_bits(x):
    """Round binary32 values to bf16 (nearest, ties to even); finite inputs."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def activations(g, M, K):
    """uint16 array (M, K) of bf16 patterns of N(0,1) samples."""
    return f32_to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))


def bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------- workloads

def single_gemv(seed=0):
    """2560 x 2560 Q4_K GEMV at M=1, seed 0."""
    g = rng(seed)
    W = weight_bytes(g, 2560, 2560)
    X = activations(g, 1, 2560)
    return W, X


def decode_layer(seed=1, layer=0, M=1):
    """One Qwen3-4B layer's seven projections at M tokens: list of
    (name, N, K, W, X); child seeds [seed, layer, projection]."""
    out = []
    for p, (name, N, K) in enumerate(PROJECTIONS):
        g = rng([seed, layer, p])
        W = weight_bytes(g, N, K)
        X = activations(g, M, K)
        out.append((name, N, K, W, X))
    return out


def prefill_projection(seed, layer, p, M):
    """One projection of the M-token prefill workloads (seed 2: M=33 over 36
    layers; seed 3: M=2048, layer 0)."""
    name, N, K = PROJECTIONS[p]
    g = rng([seed, layer, p])
    return name, N, K, weight_bytes(g, N, K), activations(g, M, K)


def lm_head(seed=4, M=512):
    """151936 x 2560 Q4_K LM head; X512 drawn after W, X1 = X512[0]."""
    _, N, K = LM_HEAD
    g = rng(seed)
    W = weight_bytes(g, N, K)
    X = activations(g, M, K)
    return W, X


# ---------------------------------------------------------------------------
# KV cache vectors

KV_DIM = 128
KV_HEADS = 8
KV_CTX = 1024


def kv_vectors(g, nvec, dim=KV_DIM):
    """(nvec, dim) binary16 bit patterns (uint16): per-vector magnitude
    log-uniform in [2^-4, 2^4], two outliers per vector scaled by 8."""
    mag = np.exp2(g.uniform(-4.0, 4.0, size=(nvec, 1)))
    z = g.standard_normal((nvec, dim)) * mag
    cols = g.integers(0, dim, size=(nvec, 2))
    rows = np.arange(nvec)[:, None]
    z[rows, cols] *= 8.0
    return z.astype(np.float16).view(np.uint16)


def kv_cache(seed=5, ctx=KV_CTX):
    """The whole cache of the workload: 36 layers x (K, V) x ctx tokens x 8
    heads vectors of 128 values, as (nvec, 128) binary16 bit patterns."""
    return kv_vectors(rng(seed), N_LAYERS * 2 * ctx * KV_HEADS)
