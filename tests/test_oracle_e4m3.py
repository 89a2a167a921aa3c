"""Pins for the oracle's E4M3FN codec and BF16 rounding (CPU only).

The codec is checked against things other than itself:
  * hand-derived textbook points in tests/golden/e4m3_points.txt;
  * a brute-force nearest-value search over the 127 non-negative finite
    E4M3 values with ties broken to the even code;
  * torch's float8_e4m3fn cast (a library routine) after a clamp to +-448;
  * structural facts of the format (253 distinct finite values, monotone
    positive half, NaN only at 0x7F / 0xFF).
BF16 rounding is checked against torch's bfloat16 cast and hand-made ties.
"""

import os

import numpy as np
import pytest
import torch

from oracle import (bf16_round_f32, bf16_round_f64, e4m3_decode, e4m3_decode_table,
                    e4m3_encode)

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden_points():
    pts = []
    with open(os.path.join(HERE, "golden", "e4m3_points.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v, c = line.split()[:2]
            pts.append((float(v), int(c, 16)))
    return pts


def test_decode_table_structure():
    t = e4m3_decode_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.count_nonzero(np.isnan(t)) == 2
    finite = t[~np.isnan(t)]
    assert len(np.unique(finite)) == 253            # +0 and -0 are one value
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                 # monotone
    assert t[0x7E] == 448.0 and t[0x38] == 1.0 and t[0x08] == 2.0 ** -6
    assert t[0x01] == 2.0 ** -9 and t[0x00] == 0.0
    assert np.signbit(t[0x80]) and t[0x80] == 0.0
    assert np.all(t[0x80:0xFF] == -t[0x00:0x7F])


def test_golden_points():
    pts = _golden_points()
    assert len(pts) >= 20
    v = np.array([p[0] for p in pts])
    want = np.array([p[1] for p in pts], dtype=np.uint8)
    got = e4m3_encode(v)
    for vi, gi, wi in zip(v, got, want):
        assert gi == wi, f"{vi}: got {gi:#04x} want {wi:#04x}"


def _brute_encode(vals):
    """Nearest of the non-negative finite values, ties to the even code,
    saturate at 448.  O(n * 127), independent of the closed-form encoder."""
    t = e4m3_decode_table()[:0x7F]                 # codes 0..0x7E
    out = np.empty(len(vals), dtype=np.uint8)
    for i, v in enumerate(vals):
        a = abs(float(v))
        if a >= 448.0:
            c = 0x7E
        else:
            d = np.abs(t - a)
            best = np.nonzero(d == d.min())[0]
            c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        if np.signbit(v):
            c |= 0x80
        out[i] = c
    return out


def test_encode_matches_brute_force_random():
    rng = np.random.default_rng(1234)
    v = np.concatenate([
        rng.standard_normal(3000) * 100,
        rng.standard_normal(3000) * 0.01,
        rng.uniform(-500, 500, 2000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 2000),
    ]).astype(np.float32)
    assert np.array_equal(e4m3_encode(v), _brute_encode(v))


def test_encode_matches_brute_force_all_midpoints():
    """Every midpoint between adjacent finite values, and one FP32 ulp on
    each side of it: the cases where a rounding slip shows."""
    t = e4m3_decode_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (t[:-1] + t[1:]) / 2)  # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    v = np.concatenate([mids, up, dn, -mids, -up, -dn, t.astype(np.float32)])
    assert np.array_equal(e4m3_encode(v), _brute_encode(v))


def test_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(99)
    v = np.concatenate([rng.standard_normal(200_000) * 150,
                        rng.standard_normal(200_000) * 1e-3]).astype(np.float32)
    ref = torch.from_numpy(v).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3_encode(v)
    # torch keeps -0 for tiny negative values that round to zero, as does the oracle
    assert np.array_equal(got, ref)


def test_bf16_round_f32_matches_torch():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(100_000) * 10,
                        rng.standard_normal(1000) * 1e-30]).astype(np.float32)
    # add exact ties: low 16 bits 0x8000
    bits = rng.integers(0, 2 ** 31, 1000, dtype=np.uint32) & np.uint32(0x7F7F0000)
    ties = (bits | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties, -ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_round_f32(v), ref)


def test_bf16_round_f64_single_rounding():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to even -> 1
    assert bf16_round_f64(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # just above the midpoint (not representable in fp32): rounds up; a
    # double rounding through fp32 would land on the tie and go to 1.0
    assert bf16_round_f64(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7
    assert bf16_round_f64(np.array([-(3.0 + 2.0 ** -7)]))[0] == -3.0     # tie, even mantissa
    assert bf16_round_f64(np.array([3.0 + 3 * 2.0 ** -7]))[0] == 3.0 + 2.0 ** -5  # tie, odd -> up
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(50_000) * 7).astype(np.float32)
    assert np.array_equal(bf16_round_f64(v.astype(np.float64)), bf16_round_f32(v).astype(np.float64))
    assert bf16_round_f64(np.array([0.0]))[0] == 0.0
