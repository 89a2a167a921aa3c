"""OCP E2M1 (FP4) encode / decode and K32 power-of-two block dequantisation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

sglang-glm53-flash-sm120 PR #13 (description) runs an MoE whose expert
weights are E2M1 values with one scale per 32 elements along K ("E2M1-K32"),
applying those weight scales in FP32 against FP8 activations.  E2M1: sign
bit, two exponent bits (bias 1), one mantissa bit, no infinities or NaN; the
eight magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  The pages leave the scale
format open; reading taken: each K32 scale is a power of two stored as its
biased exponent byte (UE8M0, value 2^(byte - 127)), the microscaling form
the gfx950 scaled MFMA consumes.  Two codes per byte, the even K index in
the low nibble.
"""

import numpy as np

E2M1_MAX = 6.0
_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """uint8 codes 0..15 -> float64 values (bit 3 = sign)."""
    c = np.asarray(codes, dtype=np.uint8)
    v = _MAG[c & 7]
    return np.where(c & 8, -v, v)


def e2m1_encode(v):
    """float -> E2M1 code, round to nearest, ties to the even code (mantissa
    bit 0), saturating at +-6; the sign of zero is kept."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    d = np.abs(a[..., None] - _MAG)                       # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                      # one or two nearest magnitudes
    codes = np.arange(8)
    # among the nearest, the even code (codes 0, 2, 4, 6 have mantissa 0)
    score = np.where(cand, np.where(codes % 2 == 0, 0, 1), 2)
    m = np.argmin(score, axis=-1).astype(np.uint8)
    return np.where(np.signbit(v), m | 8, m).astype(np.uint8)


def unpack_e2m1(packed, cols):
    """uint8 [..., cols/2] (low nibble = even column) -> codes uint8 [..., cols]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (cols,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def dequant_k32(packed, scale_bytes):
    """Packed E2M1 [rows, cols/2] with UE8M0 scale bytes [rows, cols/32] ->
    float64 [rows, cols]."""
    rows, half = packed.shape
    cols = 2 * half
    v = e2m1_decode(unpack_e2m1(packed, cols)).reshape(rows, cols // 32, 32)
    s = np.ldexp(1.0, np.asarray(scale_bytes, dtype=np.int64) - 127)
    return (v * s[:, :, None]).reshape(rows, cols)
