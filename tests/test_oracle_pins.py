"""Pins of the CPU oracle against things other than itself.

Every pin is checked against a fixed point outside the oracle's own code:
hand-derived blocks, an independent encoder, exact rational arithmetic,
library routines (numpy's binary16 conversion and matmul, torch's bfloat16
rounding), closed forms, and planted mistakes that must break the tolerance.
The block format and dequantisation rule are GGUF's Q4_K, the format of the
Qwen3-4B-Q4_K_M model in the genie-ai-runtime README ("At a glance").
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import q4k_inputs as qi
from oracle import q4k_pack as pk
from tests import golden_blocks

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def random_fields(g, nb, constrain=False):
    """Random fields for nb blocks (d, dmin positive binary16 of moderate size)."""
    d = pk.half_bits(np.abs(g.standard_normal(nb)) * 2e-3 + 1e-5)
    dmin = pk.half_bits(np.abs(g.standard_normal(nb)) * 2e-3 + 1e-5)
    sc = g.integers(0, 64, (nb, 8))
    m = g.integers(0, 64, (nb, 8))
    q = g.integers(0, 16, (nb, 256))
    if constrain:
        sc = g.integers(1, 64, (nb, 8))
        rows = np.arange(nb)
        sc[rows, g.integers(0, 8, nb)] = 63
        m[rows, g.integers(0, 8, nb)] = 63
        qv = q.reshape(nb, 8, 32)
        qv[:, :, 0] = 0
        qv[:, :, 1] = 15
        q = qv.reshape(nb, 256)
    return d, dmin, sc, m, q


def fields_to_w32(d, dmin, sc, m, q):
    """fp32 weights from fields via numpy fp64 (exact for these magnitudes)."""
    dv = pk.half_value(d)[:, None, None]
    dm = pk.half_value(dmin)[:, None, None]
    qv = q.reshape(-1, 8, 32).astype(np.float64)
    w = dv * sc[:, :, None] * qv - dm * m[:, :, None]
    return w.reshape(-1, 256).astype(np.float32)


# --------------------------------------------------------------- scalars

def test_half_decode_matches_numpy_for_every_pattern():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(v)) for v in h])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_bf16_rne_matches_torch_rounding():
    g = np.random.default_rng(7)
    u = g.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    # exact ties (dropped half == 0x8000) on both parities, and near-ties
    hi = g.integers(0, 2**16, 4000, dtype=np.uint64).astype(np.uint32) << 16
    special = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001,
                              np.array([0x7F7FFFFF, 0x7F7F8000, 0xFF7FFFFF, 0x00000001,
                                        0x80008000, 0x7F800000, 0xFF800000, 0],
                                       np.uint32)]).astype(np.uint32)
    u = np.concatenate([u, special])
    f = u.view(np.float32)
    got = oracle.float_to_bf16_rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    gotf = (got.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(gotf[nan]))


def test_bf16_widening_is_exact():
    for b in (0x0000, 0x3F80, 0xBF80, 0x4049, 0x7F7F, 0x0001):
        assert np.float32(oracle.bf16_to_float(b)).view(np.uint32) == (b << 16)


# --------------------------------------------------------- format / fields

def test_scale_bit_table_covers_every_bit_once():
    seen = {}
    fields = set()
    for kind, j, fb, byte, bb in pk.scale_bit_table():
        assert 0 <= byte < 12 and 0 <= bb < 8 and 0 <= fb < 6
        assert (byte, bb) not in seen
        seen[(byte, bb)] = (kind, j, fb)
        fields.add((kind, j, fb))
    assert len(seen) == 96 and len(fields) == 96


def test_golden_blocks_unpack_and_dequant():
    for blk in golden_blocks.load():
        q, sc, m, d, dm = oracle.unpack_fields(blk["bytes"])
        assert d[0] == blk["d"] and dm[0] == blk["dmin"], blk["name"]
        assert list(sc[0]) == blk["sc"], blk["name"]
        assert list(m[0]) == blk["m"], blk["name"]
        for i, v in blk["q"].items():
            assert q[0, i] == v, (blk["name"], i)
        w = oracle.dequant_f32(blk["bytes"])
        for i, v in blk["w"].items():
            assert w[i] == np.float32(v), (blk["name"], i, w[i], v)
        for i, bits in blk["wbits"].items():
            assert w[i:i + 1].view(np.uint32)[0] == bits, (blk["name"], i)


def test_golden_blocks_encode_back():
    """The independent encoder writes the hand-derived fields to the same bytes."""
    for blk in golden_blocks.load():
        q, sc, m, d, dm = oracle.unpack_fields(blk["bytes"])
        again = pk.pack_blocks(d, dm, sc, m, q)
        assert np.array_equal(again[0], blk["bytes"]), blk["name"]


def test_every_scale_field_value_round_trips():
    """Each of the 16 six-bit fields swept over 0..63, the rest random."""
    g = np.random.default_rng(11)
    for kind in ("sc", "m"):
        for j in range(8):
            d, dmin, sc, m, q = random_fields(g, 64)
            (sc if kind == "sc" else m)[:, j] = np.arange(64)
            blocks = pk.pack_blocks(d, dmin, sc, m, q)
            q2, sc2, m2, d2, dm2 = oracle.unpack_fields(blocks)
            assert np.array_equal(sc2, sc) and np.array_equal(m2, m), (kind, j)
            assert np.array_equal(q2, q)
            assert np.array_equal(d2, d) and np.array_equal(dm2, dmin)


def test_every_nibble_position_round_trips():
    """Each of the 256 quant positions swept over 0..15, the rest random."""
    g = np.random.default_rng(12)
    nb = 256 * 16
    d, dmin, sc, m, q = random_fields(g, nb)
    pos = np.repeat(np.arange(256), 16)
    val = np.tile(np.arange(16), 256)
    q[np.arange(nb), pos] = val
    blocks = pk.pack_blocks(d, dmin, sc, m, q)
    q2, sc2, m2, _, _ = oracle.unpack_fields(blocks)
    assert np.array_equal(q2, q)
    assert np.array_equal(sc2, sc) and np.array_equal(m2, m)


def test_random_bytes_decode_encode_bijection():
    g = np.random.default_rng(13)
    blocks = g.integers(0, 256, (3000, 144), dtype=np.uint8)
    q, sc, m, d, dm = oracle.unpack_fields(blocks)
    assert np.array_equal(pk.pack_blocks(d, dm, sc, m, q), blocks)


# ------------------------------------------------------------------ dequant

def _is_rne(exact: Fraction, w: np.float32) -> bool:
    lo = np.nextafter(w, np.float32(-np.inf))
    hi = np.nextafter(w, np.float32(np.inf))
    e = abs(exact - Fraction(float(w)))
    el = abs(exact - Fraction(float(lo)))
    eh = abs(exact - Fraction(float(hi)))
    if e > el or e > eh:
        return False
    if e == el or e == eh:          # tie: the chosen one has an even significand
        return int(np.array([w]).view(np.uint32)[0]) % 2 == 0
    return True


def test_dequant_is_the_correct_rounding_of_the_exact_value():
    g = np.random.default_rng(21)
    nb = 64
    # arbitrary finite binary16 d/dmin of both signs and all exponents
    d = g.integers(0, 0x7C00, nb).astype(np.uint16) | (g.integers(0, 2, nb) << 15).astype(np.uint16)
    dmin = g.integers(0, 0x7C00, nb).astype(np.uint16) | (g.integers(0, 2, nb) << 15).astype(np.uint16)
    sc = g.integers(0, 64, (nb, 8))
    m = g.integers(0, 64, (nb, 8))
    q = g.integers(0, 16, (nb, 256))
    blocks = pk.pack_blocks(d, dmin, sc, m, q)
    w = oracle.dequant_f32(blocks).reshape(nb, 256)
    for b in range(nb):
        for i in g.integers(0, 256, 24):
            s = i // 32
            exact = pk.exact_weight(d[b], dmin[b], sc[b, s], q[b, i], m[b, s])
            assert _is_rne(exact, w[b, i]), (b, i, exact, w[b, i])


def test_dequant_bf16_is_torch_rounding_of_dequant_f32():
    g = np.random.default_rng(22)
    blocks = qi.weight_bytes(g, 40, 2560)
    w32 = oracle.dequant_f32(blocks)
    w16 = oracle.dequant_bf16(blocks)
    ref = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(w16, ref)


def test_dequant_matches_fields_path():
    g = np.random.default_rng(23)
    fields = random_fields(g, 500)
    blocks = pk.pack_blocks(*fields[:2], fields[2], fields[3], fields[4])
    assert np.array_equal(oracle.dequant_f32(blocks).reshape(500, 256), fields_to_w32(*fields))


# ------------------------------------------------------------- contraction

def _rows(blocks_per_row, n_rows):
    return blocks_per_row.reshape(n_rows, -1)


def test_closed_form_constant_blocks():
    """q, sc, m constant: every w = -1/256, so x = 1 gives y = -K/256 exactly."""
    blk = [b for b in golden_blocks.load() if b["name"] == "closed_form"][0]["bytes"]
    N, K = 3, 2560
    W = np.tile(blk, (N, K // 256))
    X = np.full((2, K), 0x3F80, np.uint16)           # bf16 1.0
    Y, A = oracle.gemm(W, X, N, K)
    assert np.all(Y == -10.0) and np.all(A == 10.0)
    X2 = np.full((1, K), 0xC000, np.uint16)          # bf16 -2.0
    Y2, A2 = oracle.gemm(W, X2, N, K)
    assert np.all(Y2 == 20.0) and np.all(A2 == 20.0)


def test_closed_form_per_subblock_constants():
    """Constant q per sub-block: y = sum_s w_s * sum_{k in s} x_k (exact)."""
    g = np.random.default_rng(31)
    N, K = 4, 768
    nb = N * K // 256
    d, dmin, sc, m, _ = random_fields(g, nb)
    qsub = g.integers(0, 16, (nb, 8))
    q = np.repeat(qsub, 32, axis=1)
    W = pk.pack_blocks(d, dmin, sc, m, q).reshape(N, -1)
    X = qi.activations(g, 3, K)
    Y, A = oracle.gemm(W, X, N, K)
    w = oracle.dequant_f32(W).reshape(nb, 256)
    xf = qi.bf16_bits_to_f32(X).astype(np.float64)
    for mi in range(3):
        for n in range(N):
            exact = Fraction(0)
            for b in range(K // 256):
                gb = n * (K // 256) + b
                for s in range(8):
                    # every weight of the sub-block is the same fp32 value
                    assert np.all(w[gb, 32 * s:32 * s + 32] == w[gb, 32 * s])
                    w32 = Fraction(float(w[gb, 32 * s]))
                    xs = sum(Fraction(float(v)) for v in xf[mi, b * 256 + 32 * s: b * 256 + 32 * s + 32])
                    exact += w32 * xs
            assert abs(Fraction(Y[mi, n]) - exact) <= Fraction(K) * Fraction(2) ** -52 * Fraction(A[mi, n])


def test_identity_probe_isolates_every_weight():
    """X = I_K gives Y = Wdq^T exactly: each output picks one weight."""
    g = np.random.default_rng(32)
    N, K = 5, 512
    fields = random_fields(g, N * K // 256)
    W = pk.pack_blocks(*fields).reshape(N, -1)
    X = np.zeros((K, K), np.uint16)
    X[np.arange(K), np.arange(K)] = 0x3F80
    Y, _ = oracle.gemm(W, X, N, K)
    w32 = fields_to_w32(*fields).reshape(N, K)
    assert np.array_equal(Y, w32.T.astype(np.float64))


def test_matches_numpy_fp64_matmul_non_square():
    g = np.random.default_rng(33)
    N, K, M = 37, 768, 5
    fields = random_fields(g, N * K // 256)
    W = pk.pack_blocks(*fields).reshape(N, -1)
    X = qi.activations(g, M, K)
    Y, A = oracle.gemm(W, X, N, K)
    w = fields_to_w32(*fields).reshape(N, K).astype(np.float64)
    x = qi.bf16_bits_to_f32(X).astype(np.float64)
    Yn = x @ w.T
    An = np.abs(x) @ np.abs(w).T
    assert np.all(np.abs(Y - Yn) <= 1e-12 * An)
    assert np.allclose(A, An, rtol=1e-12, atol=0)
    assert np.all(A >= np.abs(Y))


def test_exact_rational_bruteforce_on_tiny_inputs():
    g = np.random.default_rng(34)
    for N, K, M in ((1, 256, 1), (3, 256, 2), (4, 512, 3), (2, 512, 1)):
        W = qi.weight_bytes(g, N, K)
        X = qi.activations(g, M, K)
        Y, A = oracle.gemm(W, X, N, K)
        w = oracle.dequant_f32(W).reshape(N, K)
        x = qi.bf16_bits_to_f32(X)
        for mi in range(M):
            for n in range(N):
                terms = [Fraction(float(w[n, k])) * Fraction(float(x[mi, k])) for k in range(K)]
                exact = sum(terms)
                abs_exact = sum(abs(t) for t in terms)
                bound = Fraction(K) * Fraction(2) ** -53 * abs_exact
                assert abs(Fraction(Y[mi, n]) - exact) <= bound
                assert abs(Fraction(A[mi, n]) - abs_exact) <= bound


def test_m_zero_and_shape_errors():
    g = np.random.default_rng(35)
    W = qi.weight_bytes(g, 3, 256)
    Y, A = oracle.gemm(W, np.zeros((0, 256), np.uint16), 3, 256)
    assert Y.shape == (0, 3)
    with pytest.raises(ValueError):
        oracle.gemm(W, np.zeros((1, 512), np.uint16), 3, 256)


# ------------------------------------------------------------ quantiser

def test_quantizer_round_trips_grid_values():
    """quantize(dequant(fields)) returns the same fields for grid blocks with
    every sc >= 1, some sc = 63 and m = 63, each sub-block's q spanning 0..15."""
    g = np.random.default_rng(41)
    nb = 2000
    fields = random_fields(g, nb, constrain=True)
    blocks = pk.pack_blocks(*fields)
    w = oracle.dequant_f32(blocks).reshape(nb, 256)
    d2, dm2, sc2, m2, q2 = pk.quantize_blocks(w)
    assert np.array_equal(d2, fields[0]) and np.array_equal(dm2, fields[1])
    assert np.array_equal(sc2, fields[2]) and np.array_equal(m2, fields[3])
    assert np.array_equal(q2, fields[4])
    again = oracle.dequant_f32(pk.pack_blocks(d2, dm2, sc2, m2, q2)).reshape(nb, 256)
    assert np.array_equal(again.view(np.uint32), w.view(np.uint32))


# ------------------------------------------ the tolerance is not vacuous

@pytest.fixture(scope="module")
def single_gemv_ref():
    W, X = qi.single_gemv(0)
    Y, A = oracle.gemm(W, X, 2560, 2560)
    return W, X, Y, A


def _fail_fraction(Wbad, X, Y, A):
    Yb, _ = oracle.gemm(Wbad, X, 2560, 2560)
    return 1.0 - oracle.within_tolerance(Yb, Y, A).mean()


def test_planted_nibble_swap_breaks_tolerance(single_gemv_ref):
    W, X, Y, A = single_gemv_ref
    Wb = W.reshape(-1, 144).copy()
    qs = Wb[:, 16:]
    Wb[:, 16:] = ((qs & 0x0F) << 4) | (qs >> 4)
    assert _fail_fraction(Wb.reshape(W.shape), X, Y, A) > 0.25


def test_planted_dropped_min_term_breaks_tolerance(single_gemv_ref):
    W, X, Y, A = single_gemv_ref
    Wb = W.reshape(-1, 144).copy()
    Wb[:, 2:4] = 0                                   # dmin = 0
    assert _fail_fraction(Wb.reshape(W.shape), X, Y, A) > 0.25


def test_planted_wrong_subblock_scales_break_tolerance(single_gemv_ref):
    W, X, Y, A = single_gemv_ref
    Wb = W.reshape(-1, 144).copy()
    Wb[:, 4:16] = np.roll(Wb[:, 4:16], 1, axis=1)    # fields read from the wrong bytes
    assert _fail_fraction(Wb.reshape(W.shape), X, Y, A) > 0.25


def test_planted_sign_flip_breaks_tolerance(single_gemv_ref):
    W, X, Y, A = single_gemv_ref
    Wb = W.reshape(-1, 144).copy()
    Wb[:, 1] ^= 0x80                                 # d -> -d
    assert _fail_fraction(Wb.reshape(W.shape), X, Y, A) > 0.25


def test_planted_transposed_x_breaks_tolerance(single_gemv_ref):
    W, X, Y, A = single_gemv_ref
    Yb, _ = oracle.gemm(W, X[:, ::-1].copy(), 2560, 2560)
    assert 1.0 - oracle.within_tolerance(Yb, Y, A).mean() > 0.25


# ---------------------------------------------------------------------------
# SwiGLU epilogue (h = silu(g) * u)

def test_silu_closed_forms_and_library():
    import torch
    z = np.concatenate([np.linspace(-60, 60, 2001), [0.0, 1e-300, -1e-300, 700.0, -700.0]])
    s = oracle.silu(z)
    assert s[np.where(z == 0.0)[0][0]] == 0.0
    # silu(z) - silu(-z) = z, since sigmoid(z) + sigmoid(-z) = 1
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-14, atol=1e-300)
    # silu(z) -> z for large z, -> 0 for very negative z
    assert oracle.silu(np.array([700.0]))[0] == 700.0
    assert 0.0 > oracle.silu(np.array([-700.0]))[0] > -1e-300     # -700 e^-700
    assert oracle.silu(np.array([-800.0]))[0] == 0.0               # e^800 overflows
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    assert np.allclose(s, ref, rtol=1e-13, atol=1e-300)


def test_silu_lipschitz_constant():
    z = np.linspace(-20, 20, 400001)
    sig = 1.0 / (1.0 + np.exp(-z))
    d = sig * (1.0 + z * (1.0 - sig))          # silu'(z)
    assert np.max(np.abs(d)) <= oracle.SILU_LIPSCHITZ
    assert np.max(np.abs(d)) > oracle.SILU_LIPSCHITZ - 1e-3


def _swiglu_case(seed, N=48, K=512, M=3):
    g = np.random.default_rng(seed)
    Wg = qi.weight_bytes(g, N, K)
    Wu = qi.weight_bytes(g, N, K)
    X = qi.activations(g, M, K)
    return Wg, Wu, X, N, K


def test_swiglu_is_silu_of_gate_times_up():
    Wg, Wu, X, N, K = _swiglu_case(200)
    H, G, U, Ag, Au = oracle.gemm_swiglu(Wg, Wu, X, N, K)
    Gs, _ = oracle.gemm(Wg, X, N, K)
    Us, _ = oracle.gemm(Wu, X, N, K)
    assert np.array_equal(G, Gs) and np.array_equal(U, Us)
    sig = 1.0 / (1.0 + np.exp(-Gs))
    assert np.allclose(H, Gs * sig * Us, rtol=1e-13, atol=0)


def test_swiglu_bound_holds_for_perturbed_inputs_and_rejects_mistakes():
    """The bound admits any g, u within the matmul bound (worst-case signs),
    and planted mistakes in the epilogue fail it on most outputs."""
    Wg, Wu, X, N, K = _swiglu_case(201)
    H, G, U, Ag, Au = oracle.gemm_swiglu(Wg, Wu, X, N, K)
    tol = oracle.swiglu_tolerance(G, U, Ag, Au)
    tg, tu = oracle.tolerance(Ag), oracle.tolerance(Au)
    for sg in (-1, 1):
        for su in (-1, 1):
            h = oracle.silu(G + sg * tg) * (U + su * tu)
            assert np.all(np.abs(h - H) <= tol)
    sig = 1.0 / (1.0 + np.exp(-G))
    for wrong in (sig * U,                       # sigmoid instead of silu
                  oracle.silu(U) * G,            # gate and up swapped
                  G * U,                         # no activation
                  oracle.silu(np.roll(G, 1, axis=1)) * U):   # gate of the neighbouring row
        bad = np.abs(wrong - H) > tol
        assert bad.mean() > 0.25, bad.mean()


# ---------------------------------------------------------------------------
# RMSNorm ahead of a projection

def test_rmsnorm_library_and_invariants():
    import torch
    g = np.random.default_rng(400)
    K = 2560
    X = qi.activations(g, 3, K)
    gamma = qi.f32_to_bf16_bits((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
    eps = 1e-6
    ref = torch.nn.functional.rms_norm(torch.from_numpy(oracle.bf16_to_f64(X)), (K,),
                                       weight=torch.from_numpy(oracle.bf16_to_f64(gamma)),
                                       eps=eps).numpy()
    assert np.allclose(oracle.rmsnorm_f64(X, gamma, eps), ref, rtol=1e-14, atol=0)
    # scale invariance (eps = 0): a power-of-two scaling of x cancels exactly
    X2 = qi.f32_to_bf16_bits((qi.bf16_bits_to_f32(X) * 4.0).astype(np.float32))
    assert np.array_equal(oracle.rmsnorm_f64(X2, gamma, 0.0), oracle.rmsnorm_f64(X, gamma, 0.0))
    # constant row c: x_hat = gamma * c / sqrt(c^2 + eps)
    c = np.full((1, K), qi.f32_to_bf16_bits(np.float32(-0.75)), dtype=np.uint16)
    want = oracle.bf16_to_f64(gamma) * (-0.75 / np.sqrt(0.5625 + eps))
    assert np.allclose(oracle.rmsnorm_f64(c, gamma, eps)[0], want, rtol=1e-15, atol=0)


def test_rmsnorm_bf16_rounding_and_contraction():
    g = np.random.default_rng(401)
    N, K = 24, 512
    W = qi.weight_bytes(g, N, K)
    X = qi.activations(g, 2, K)
    gamma = qi.f32_to_bf16_bits((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
    Y, A, Xh = oracle.gemm_rmsnorm(W, X, gamma, 1e-6, N, K)
    f = oracle.rmsnorm_f64(X, gamma, 1e-6)
    # x_hat is the nearest bf16 to the fp32 rounding of the exact value
    back = oracle.bf16_to_f64(Xh)
    assert np.all(np.abs(back - f) <= np.abs(f) * 2.0 ** -8 + 1e-300)
    Y2, A2 = oracle.gemm(W, Xh, N, K)
    assert np.array_equal(Y, Y2) and np.array_equal(A, A2)


# ---------------------------------------------------------------------------
# FP16 <-> INT8 KV-cache convert (oracle/kv_oracle.c)

def test_kv_half_to_float_exhaustive():
    """Every binary16 pattern decodes as numpy's float16 -> float32 (a
    library routine)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.half_to_float(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_kv_float_to_half_rne_matches_numpy():
    """fp32 -> binary16 round-to-nearest-even against numpy's conversion, on
    every binary16 value, every midpoint between neighbours (the ties), points
    just beside them, subnormals, the overflow edge and random floats."""
    pos = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2                          # exact in fp32
    pts = np.concatenate([pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                          np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                          [65504.0, 65519.99, 65520.0, 70000.0, 2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26]])
    g = np.random.default_rng(7)
    pts = np.concatenate([pts, np.exp2(g.uniform(-30, 17, 20000)) * g.choice([-1, 1], 20000)])
    x = np.concatenate([pts, -pts]).astype(np.float32)
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half_rne(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


def test_kv_quant_closed_form():
    """A vector whose largest magnitude is 127 * 2^k has the exact scale 2^k
    and codes rint(v / 2^k): ties go to even (2.5 -> 2, 3.5 -> 4, -2.5 -> -2),
    and dequantisation returns the values exactly."""
    base = np.array([127, -127, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 0.0, -0.0, 126.5, 0.25,
                     64, -1, 100, 7], np.float64)
    codes = np.array([127, -127, 2, 4, -2, -4, 0, 2, 0, 0, 126, 0, 64, -1, 100, 7], np.int8)
    for k in (0, -6, 3):
        v = (base * 2.0 ** k).astype(np.float16).view(np.uint16)[None, :]
        q, s = oracle.kv_quant(v)
        assert s[0] == np.float32(2.0 ** k)
        assert np.array_equal(q[0], codes)
        back = oracle.kv_dequant(q, s).view(np.float16).astype(np.float64)[0]
        assert np.array_equal(back, codes.astype(np.float64) * 2.0 ** k)


def test_kv_quant_zero_vector_and_sign():
    v = np.zeros((2, 8), np.float16)
    v[1] = [-1, 1, -0.5, 0.5, -127, 127, 0, -0.0]
    q, s = oracle.kv_quant(v.view(np.uint16))
    assert s[0] == 0 and not q[0].any()
    assert np.array_equal(oracle.kv_dequant(q, s)[0], np.zeros(8, np.uint16))
    assert s[1] == 1.0 and list(q[1]) == [-1, 1, 0, 0, -127, 127, 0, 0]


def test_kv_dequant_rounding_matches_numpy():
    """v' = fp16(fp32(q * s)): numpy's fp32 product, then its fp16
    conversion, agrees bit for bit (this also fixes the two-step rounding)."""
    g = np.random.default_rng(11)
    q = g.integers(-127, 128, size=(4000, 16)).astype(np.int8)
    s = (np.exp2(g.uniform(-20, 8, 4000)) * g.uniform(1, 2, 4000)).astype(np.float32)
    ref = (q.astype(np.float32) * s[:, None]).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.kv_dequant(q, s), ref)


def test_kv_round_trip_contract():
    """On the workload's vectors: |q| <= 127 with 127 reached; the round trip
    stays within s/2 (plus half a binary16 ulp of v' and the fp32 rounding
    of s and of v/s); quantising v' again gives the same codes and the
    values move by at most one binary16 ulp (no drift beyond the first round
    trip)."""
    v = qi.kv_vectors(qi.rng(12), 3000, 128)
    q, s = oracle.kv_quant(v)
    assert np.abs(q.astype(int)).max(axis=1).tolist() == [127] * 3000
    x = v.view(np.float16).astype(np.float64)
    back = oracle.kv_dequant(q, s)
    xb = back.view(np.float16).astype(np.float64)
    ulp16 = np.spacing(np.abs(back.view(np.float16))).astype(np.float64)
    bound = s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -16) + ulp16 / 2
    assert np.all(np.abs(xb - x) <= bound)
    q2, s2 = oracle.kv_quant(back)
    assert np.array_equal(q2, q)
    back2 = oracle.kv_dequant(q2, s2).view(np.float16).astype(np.float64)
    assert np.all(np.abs(back2 - xb) <= ulp16)
