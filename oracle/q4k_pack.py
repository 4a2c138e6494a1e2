"""Independent encoder for Q4_K blocks, and the min/max quantiser.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The encoder is a bit-writer driven by a declarative table: every bit of every
6-bit field is given its byte and bit position.  It is written apart from the
decoder in ``q4k_oracle.c`` (which reads fields with masks and shifts), so that
the two can pin each other: a transposed index on either side breaks the
round trip.  The layout is GGUF's Q4_K (the format of the Qwen3-4B-Q4_K_M
model named in the genie-ai-runtime README, "At a glance").
"""
from fractions import Fraction

import numpy as np

BLOCK_BYTES = 144
QK = 256


def scale_bit_table():
    """(kind, j, field_bit, byte, byte_bit) for all 96 bits of the 12 scale
    bytes; kind is 'sc' or 'm', j the sub-block 0..7.

    Sub-blocks 0..3: all six bits of sc_j in byte j, of m_j in byte j+4.
    Sub-blocks 4..7: bits 0..3 of sc_j in the low nibble of byte j+4 and bits
    0..3 of m_j in its high nibble; bits 4..5 of sc_j in bits 6..7 of byte j-4
    and bits 4..5 of m_j in bits 6..7 of byte j.
    """
    table = []
    for j in range(4):
        for b in range(6):
            table.append(("sc", j, b, j, b))
            table.append(("m", j, b, j + 4, b))
    for j in range(4, 8):
        for b in range(4):
            table.append(("sc", j, b, j + 4, b))
            table.append(("m", j, b, j + 4, 4 + b))
        for b in (4, 5):
            table.append(("sc", j, b, j - 4, 2 + b))
            table.append(("m", j, b, j, 2 + b))
    return table


def quant_position(i):
    """(byte index within qs, bit shift) of weight i's 4-bit quant."""
    return 32 * (i // 64) + (i % 32), 4 * ((i // 32) % 2)


def pack_blocks(d_bits, dmin_bits, sc, m, q):
    """Fields -> uint8 array (nblocks, 144).

    d_bits, dmin_bits: uint16 (nblocks,) binary16 patterns;
    sc, m: (nblocks, 8) ints 0..63; q: (nblocks, 256) ints 0..15.
    """
    d_bits = np.asarray(d_bits, np.uint16).reshape(-1)
    nb = d_bits.size
    dmin_bits = np.asarray(dmin_bits, np.uint16).reshape(nb)
    sc = np.asarray(sc, np.int64).reshape(nb, 8)
    m = np.asarray(m, np.int64).reshape(nb, 8)
    q = np.asarray(q, np.int64).reshape(nb, QK)
    if sc.min(initial=0) < 0 or sc.max(initial=0) > 63 or m.min(initial=0) < 0 \
            or m.max(initial=0) > 63:
        raise ValueError("6-bit field out of range")
    if q.min(initial=0) < 0 or q.max(initial=0) > 15:
        raise ValueError("4-bit quant out of range")
    out = np.zeros((nb, BLOCK_BYTES), np.uint8)
    out[:, 0] = d_bits & 0xFF
    out[:, 1] = d_bits >> 8
    out[:, 2] = dmin_bits & 0xFF
    out[:, 3] = dmin_bits >> 8
    scales = np.zeros((nb, 12), np.int64)
    for kind, j, fb, byte, bb in scale_bit_table():
        src = sc if kind == "sc" else m
        scales[:, byte] |= ((src[:, j] >> fb) & 1) << bb
    out[:, 4:16] = scales.astype(np.uint8)
    qs = np.zeros((nb, 128), np.int64)
    for i in range(QK):
        byte, shift = quant_position(i)
        qs[:, byte] |= q[:, i] << shift
    out[:, 16:] = qs.astype(np.uint8)
    return out


def half_bits(x):
    """Nearest binary16 (numpy's IEEE conversion) as bit patterns."""
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def half_value(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def exact_weight(d_bits, dmin_bits, sc, q, m):
    """Exact rational value of one weight, from its fields."""
    d = Fraction(float(half_value(d_bits)))
    dmin = Fraction(float(half_value(dmin_bits)))
    return d * int(sc) * int(q) - dmin * int(m)


def _rn(x):
    """Round half to even (numpy's rint)."""
    return np.rint(x)


def quantize_blocks(w):
    """Plain min/max affine quantiser: fp32 weights (nblocks, 256) -> fields.

    Per sub-block s: mn_s = -min(0, min w), a_s = (max w + mn_s) / 15.
    Per block: d = fp16(max a_s / 63), dmin = fp16(max mn_s / 63).
    Then sc_s = RN(a_s / d), m_s = RN(mn_s / dmin) clamped to 0..63, and
    q = RN((w + dmin*m_s) / (d*sc_s)) clamped to 0..15.  Arithmetic in fp64.
    Returns (d_bits, dmin_bits, sc, m, q).
    """
    w = np.asarray(w, np.float64).reshape(-1, 8, 32)
    nb = w.shape[0]
    mn = -np.minimum(0.0, w.min(axis=2))
    a = (w.max(axis=2) + mn) / 15.0
    d_bits = half_bits(a.max(axis=1) / 63.0)
    dmin_bits = half_bits(mn.max(axis=1) / 63.0)
    d = half_value(d_bits)[:, None]
    dmin = half_value(dmin_bits)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d > 0, np.clip(_rn(a / d), 0, 63), 0).astype(np.int64)
        m = np.where(dmin > 0, np.clip(_rn(mn / dmin), 0, 63), 0).astype(np.int64)
        step = (d * sc)[:, :, None]
        q = np.where(step > 0,
                     np.clip(_rn((w + (dmin * m)[:, :, None]) / step), 0, 15), 0)
    return d_bits, dmin_bits, sc, m, q.astype(np.int64).reshape(nb, QK)
