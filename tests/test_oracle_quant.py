"""Pins for the oracle's 1x128 group quantisation (CPU only).

Checked against:
  * closed forms: a group built from known E4M3 values times 2^k whose
    largest magnitude is 448 * 2^k has scale exactly 2^k and quantises back to
    exactly those codes (FP32 and UE8M0 modes);
  * invariants: every non-zero FP32-mode group holds a +-448 code at its
    largest element, the dequantised value is within half an E4M3 step (plus
    one FP32 rounding) of the input, all-zero groups give codes 0 and the
    FLT_MIN scale (the zero-scale floor);
  * the UE8M0 exponent against a brute-force scan over exponents.
"""

import numpy as np
import pytest

from oracle import (FLT_MIN, e4m3_decode, e4m3_decode_table, e4m3_encode,
                    quant_act_ref, quant_groups_ref, ue8m0_exponent)
from oracle.quant import SCALE_FP32, SCALE_UE8M0


@pytest.mark.parametrize("mode", [SCALE_FP32, SCALE_UE8M0])
@pytest.mark.parametrize("k", [-20, -3, 0, 5, 30])
def test_known_codes_roundtrip(mode, k):
    rng = np.random.default_rng(k + 100)
    codes = rng.integers(0, 256, size=(6, 256)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    codes[:, 5] = 0x7E                     # group 0's amax = 448 * 2^k
    codes[:, 200] = 0xFE                   # group 1's amax = 448 * 2^k
    v = (e4m3_decode(codes) * 2.0 ** k).astype(np.float32)
    q, s = quant_groups_ref(v, mode)
    assert np.all(s == np.float32(2.0 ** k))
    # -0 and +0 are the same value; compare by value, then the nonzero codes exactly
    assert np.array_equal(e4m3_decode(q), e4m3_decode(codes))
    nz = e4m3_decode(codes) != 0
    assert np.array_equal(q[nz], codes[nz])


def test_fp32_mode_invariants():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((64, 1024)) * rng.uniform(1e-3, 1e3, (64, 1))).astype(np.float32)
    x[3, 128:256] = 0.0
    q, s = quant_act_ref(x, SCALE_FP32)
    assert q.dtype == np.uint8 and s.shape == (64, 8) and s.dtype == np.float32
    g = x.reshape(64, 8, 128)
    amax = np.abs(g).max(-1)
    nz = amax > 0
    # the largest element of a non-zero group maps to +-448
    qg = q.reshape(64, 8, 128)
    imax = np.abs(g).argmax(-1)
    top = np.take_along_axis(qg, imax[..., None], -1)[..., 0]
    assert np.all((top[nz] & 0x7F) == 0x7E)
    # zero group: codes zero, scale floored at FLT_MIN
    assert np.all(qg[3, 1] & 0x7F == 0) and s[3, 1] == FLT_MIN
    # scale formula: amax / 448 in FP32, floored
    assert np.all(s[nz] == (amax[nz] / np.float32(448)).astype(np.float32))
    # error bound: |deq - x| <= (half E4M3 step at |x/s| + fp32 slack) * s
    d = e4m3_decode(q).reshape(64, 8, 128) * s[..., None].astype(np.float64)
    t = e4m3_decode_table()[:0x7F]
    y = np.abs(g / s[..., None].astype(np.float64))
    idx = np.clip(np.searchsorted(t, y), 1, 126)
    step = t[idx] - t[idx - 1]
    bound = (0.5 * step + 448 * 2.0 ** -22) * s[..., None]
    assert np.all(np.abs(d - g) <= bound)


def test_ue8m0_exponent_brute_force():
    rng = np.random.default_rng(1)
    a = np.concatenate([np.abs(rng.standard_normal(2000)) * 10.0 ** rng.uniform(-30, 30, 2000),
                        448.0 * 2.0 ** np.arange(-40, 40, dtype=np.float64),
                        np.nextafter(448.0 * 2.0 ** np.arange(-40, 40, dtype=np.float64), np.inf),
                        np.nextafter(448.0 * 2.0 ** np.arange(-40, 40, dtype=np.float64), 0),
                        [0.0, 1e-45, 2.0 ** -140]]).astype(np.float32).astype(np.float64)
    got = ue8m0_exponent(a)
    for ai, gi in zip(a, got):
        want = next(e for e in range(-126, 200) if 448.0 * 2.0 ** e >= ai)
        assert gi == want, (ai, gi, want)


def test_ue8m0_mode_is_exact_power_of_two_scaling():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((16, 512)) * 3).astype(np.float32)
    q, s = quant_act_ref(x, SCALE_UE8M0)
    m, e = np.frexp(s)
    assert np.all(m == 0.5)                                   # powers of two
    amax = np.abs(x.reshape(16, 4, 128)).max(-1)
    assert np.all(448.0 * s >= amax) and np.all(224.0 * s < amax)  # least exponent
    want = e4m3_encode(x.reshape(16, 4, 128).astype(np.float64) / s[..., None])
    assert np.array_equal(q, want.reshape(16, 512))
