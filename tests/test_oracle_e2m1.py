"""Pins for the oracle's E2M1 codec, K32 dequantisation and W4A8 expert
path (CPU only).

Checked against things other than the code under test:
  * the E2M1 closed form (sign, two exponent bits with bias 1, one mantissa
    bit; exponent field 0 is subnormal) for all 16 codes;
  * a brute-force nearest-value search over the 16 codes with ties broken to
    the even code, plus hand-listed midpoints and saturation;
  * a pure-Python element-by-element unpack and dequantisation (nibble k % 2
    of byte k // 2, low nibble first; scale 2^(byte - 127) of group k // 32);
  * the W8A8 expert path (pinned on its own) on the same weights written as
    E4M3 codes with unit block scales -- exact, since every E2M1 value times
    2^j, |j| <= 3, is an E4M3 value -- which must agree bit for bit (catches
    a swapped nibble order, a wrong scale index or a transposed operand);
  * one-hot weights placing one activation element through each layout.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (dequant_k32, e2m1_decode, e2m1_encode, e4m3_decode, experts_ref,
                    experts_w4a8_ref, plan_ref, quant_act_ref, unpack_e2m1)
from moe_workloads import make_case


def _closed_form(c):
    s = -1.0 if c & 8 else 1.0
    e, m = (c >> 1) & 3, c & 1
    return s * (0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m))


def test_decode_closed_form_all_codes():
    for c in range(16):
        v = e2m1_decode(np.array([c], np.uint8))[0]
        assert v == _closed_form(c) and math.copysign(1, v) == math.copysign(1, _closed_form(c)) \
            or (v == 0 and _closed_form(c) == 0), c


def test_encode_roundtrip_and_sign_of_zero():
    for c in range(16):
        v = _closed_form(c)
        if c == 8:
            v = -0.0
        assert int(e2m1_encode(np.array([v]))[0]) == c


@pytest.mark.parametrize("mid,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4),
                                      (3.5, 6), (5.0, 6), (7.0, 7), (1e30, 7), (6.0, 7)])
def test_encode_ties_to_even_and_saturation(mid, code):
    assert int(e2m1_encode(np.array([mid]))[0]) == code
    assert int(e2m1_encode(np.array([-mid]))[0]) == code | 8


def test_encode_brute_force_nearest():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-7, 7, 4000), rng.normal(0, 1, 2000),
                        np.arange(-6.5, 6.51, 0.125)])
    got = e2m1_encode(v)
    vals = np.array([_closed_form(c) for c in range(16)])
    for x, c in zip(v, got):
        a = min(abs(x), 6.0)
        d = [abs(a - abs(vals[k])) for k in range(8)]
        best = min(d)
        cand = [k for k in range(8) if d[k] == best]
        want = [k for k in cand if k % 2 == 0] or cand
        assert int(c) & 7 == want[0], (x, c)
        assert bool(int(c) & 8) == (math.copysign(1, x) < 0)


def test_unpack_and_dequant_elementwise():
    rng = np.random.default_rng(6)
    rows, cols = 5, 96
    packed = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    sb = rng.integers(100, 150, (rows, cols // 32), dtype=np.uint8)
    codes = unpack_e2m1(packed, cols)
    deq = dequant_k32(packed, sb)
    for r in range(rows):
        for k in range(cols):
            byte = int(packed[r, k // 2])
            nib = (byte >> 4) if k % 2 else (byte & 15)
            assert codes[r, k] == nib
            want = _closed_form(nib) * 2.0 ** (int(sb[r, k // 32]) - 127)
            assert deq[r, k] == want


def _as_w8a8(w4, w4e):
    """E2M1 weights [E, rows, cols/2] with exponent bytes as E4M3 codes with
    unit 128x128 block scales, decoded element by element here (the closed
    form, not the oracle's table); codes from torch's float8 cast."""
    E, rows, half = w4.shape
    cols = 2 * half
    vals = np.empty((E, rows, cols))
    tab = np.array([_closed_form(c) for c in range(16)])
    lo, hi = tab[w4 & 15], tab[w4 >> 4]
    vals[..., 0::2], vals[..., 1::2] = lo, hi
    vals *= np.repeat(2.0 ** (w4e.astype(np.int64) - 127), 32, axis=-1)
    codes = torch.from_numpy(vals).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(e4m3_decode(codes.numpy()), vals), "not E4M3-representable"
    return codes.numpy(), np.ones((E, rows // 128, cols // 128), np.float32)


def test_w4a8_equals_w8a8_on_shared_values():
    c = make_case("tiny", fmt="w4a8")
    rng = np.random.default_rng(7)
    w13, w2 = c.w13.numpy(), c.w2.numpy()
    # exponents 124..130 (scales 2^-3 .. 2^3) varied per row and K32 group
    w13e = rng.integers(124, 131, c.w13_s.shape, dtype=np.uint8)
    w2e = rng.integers(124, 131, c.w2_s.shape, dtype=np.uint8)
    c13, s13 = _as_w8a8(w13, w13e)
    c2, s2 = _as_w8a8(w2, w2e)
    xq, xs = quant_act_ref(c.x.float().numpy())
    ids, w = c.topk_ids.numpy(), c.topk_weights.numpy()
    srt, eid, P = plan_ref(ids, c.E, c.block_m)
    r4 = experts_w4a8_ref(xq, xs, w13, w13e, w2, w2e, w, srt, eid, P, c.top_k, c.block_m)
    r8 = experts_ref(xq, xs, c13, s13, c2, s2, w, srt, eid, P, c.top_k, c.block_m)
    assert np.array_equal(r4.h_q, r8.h_q) and np.array_equal(r4.h_s, r8.h_s)
    assert np.array_equal(r4.ref64, r8.ref64)
    assert np.abs(r4.ref64).max() > 0


def test_w4a8_one_hot_layout():
    """One nonzero E2M1 weight per matrix: g, h and out must pick single
    activation / intermediate elements at the right places."""
    M, E, K, I, top_k, bm = 1, 1, 256, 128, 1, 16
    x = np.zeros((M, K), np.float32)
    k0, n0, c0 = 161, 37, 200                      # K index, gate row, output column
    x[0, k0] = 3.0
    xq, xs = quant_act_ref(x)
    xval = e4m3_decode(xq[0, k0]) * xs[0, k0 // 128]
    w13 = np.zeros((E, 2 * I, K // 2), np.uint8)
    w13e = np.full((E, 2 * I, K // 32), 127, np.uint8)
    # gate row n0 and up row I + n0 both read K index k0 (odd: high nibble)
    w13[0, n0, k0 // 2] = 0x4 << 4                  # 2.0
    w13[0, I + n0, k0 // 2] = 0x2 << 4              # 1.0
    w13e[0, n0, k0 // 32] = 128                     # x2 -> gate weight 4.0
    w2 = np.zeros((E, K, I // 2), np.uint8)
    w2e = np.full((E, K, I // 32), 127, np.uint8)
    w2[0, c0, n0 // 2] = 0x2 << 4                   # n0 odd: high nibble, 1.0
    w2e[0, c0, n0 // 32] = 126                      # x0.5
    ids = np.zeros((M, top_k), np.int32)
    w = np.ones((M, top_k), np.float32)
    srt, eid, P = plan_ref(ids, E, bm)
    dbg = {}
    r = experts_w4a8_ref(xq, xs, w13, w13e, w2, w2e, w, srt, eid, P, top_k, bm, debug=dbg)
    g = dbg["g"][0]
    assert g[n0] == 4.0 * xval and g[I + n0] == 1.0 * xval
    assert np.count_nonzero(g) == 2
    hval = e4m3_decode(r.h_q[0, n0]) * r.h_s[0, n0 // 128]
    assert np.count_nonzero(r.ref64) == 1 and r.ref64[0, c0] == 0.5 * hval
    silu = 4.0 * xval / (1 + math.exp(-4.0 * xval)) * xval
    assert abs(hval - silu) <= 2 ** -3 * abs(silu)
