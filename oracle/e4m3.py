"""OCP E4M3FN codec and BF16 rounding, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The FP8 format is the one FlashInfer PR #4287 (PR summary; "Public contract
and review fixes") and sglang-glm53-flash-sm120 PR #13 (description) call
"FP8": E4M3 with the OCP "FN" encoding -- 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits, no infinities, NaN only at S.1111.111, largest
finite magnitude 1.75 * 2^8 = 448.  PR #13's validation paragraph speaks of
adjacent-code rounding ties, i.e. round-to-nearest with ties broken to the
even code; values at or beyond 448 saturate to 448 (the reading taken for the
quantisers of this path, whose scaled inputs never exceed 448 by more than an
FP32 rounding).

Encoding (value v, a = |v|):
  * sign bit = sign of v (so -0 encodes as 0x80);
  * a >= 448                -> 448 (code 0x7E);
  * a <  2^-6 (subnormal)   -> mantissa m = rne(a * 2^9), code = m
                               (m = 8 lands on 0x08 = 2^-6, the least normal);
  * otherwise e = floor(log2 a), m = rne(a * 2^(3-e)) in [8, 16]; a carry
    (m = 16) moves to e + 1, m = 8; code = (e + 7) << 3 | (m - 8).
All scalings are by powers of two, so the only rounding is the rne().
"""

import numpy as np

E4M3_MAX = 448.0
#: Smallest positive normal FP32 number; the quantisers floor their scale
#: here so an all-zero group never inverts a zero scale (FlashInfer PR #4287,
#: review of the zero-activation scale, and its public-contract section).
FLT_MIN = np.float32(2.0 ** -126)


def e4m3_decode_table():
    """float64 value of each byte 0..255 (NaN for 0x7F and 0xFF)."""
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        sgn = -1.0 if (c & 0x80) else 1.0
        ex = (c >> 3) & 0xF
        man = c & 0x7
        if ex == 0xF and man == 0x7:
            t[c] = np.nan
        elif ex == 0:
            t[c] = sgn * man * 2.0 ** -9          # (man/8) * 2^(1-7)
        else:
            t[c] = sgn * (1.0 + man / 8.0) * 2.0 ** (ex - 7)
    return t


_TABLE = e4m3_decode_table()


def e4m3_decode(codes):
    """Decode uint8 codes to float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v):
    """Encode values (any float dtype; taken exactly) to uint8 E4M3FN codes.

    Round to nearest, ties to even; saturate at +-448.  NaN inputs are not
    part of the domain and are not handled.
    """
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.abs(v)

    # subnormal range: unit 2^-9
    m_sub = np.rint(np.minimum(a, 2.0 ** -6) * 512.0)

    # normal range
    with np.errstate(divide="ignore", invalid="ignore"):
        f, x = np.frexp(a)                 # a = f * 2^x, f in [0.5, 1)
    e = x.astype(np.int64) - 1             # floor(log2 a) for a > 0
    m = np.rint(np.ldexp(a, (3 - e).astype(np.int32)))  # in [8, 16]
    carry = m >= 16.0
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8.0, m)
    code_norm = ((e + 7) << 3) | (m.astype(np.int64) - 8)

    code = np.where(a < 2.0 ** -6, m_sub.astype(np.int64), code_norm)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def bf16_round_f32(x):
    """Round float32 values to the nearest BF16 (ties to even); float32 out."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_round_f64(x):
    """Round float64 values to the nearest BF16 (single rounding, ties to
    even); float64 out.  Normal range only (|x| >= 2^-126 or 0), which covers
    every output this path produces."""
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)                     # x = f * 2^e, |f| in [0.5, 1)
    q = np.rint(np.ldexp(f, 8))            # 8 significant bits
    return np.ldexp(q, e - 8)
