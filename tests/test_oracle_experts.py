"""Pins for the oracle's expert path (CPU only).

Checked against:
  * exact rational arithmetic (fractions.Fraction; every E4M3 value and FP32
    scale is a dyadic rational) for sampled gate/up sums g, down rows y and
    final outputs of the tiny workload;
  * one-hot weights, which must reproduce single activation elements and
    place them by the gate/up/down layout (catches transposed operands, a
    swapped gate/up half, wrong scale-block indices);
  * SwiGLU against scipy's logistic function (a library routine);
  * a dense special case (one expert, top-1, weight 1) against a plain FP64
    MLP written with matmuls;
  * invariants: linear in the route weights, token-permutation equivariant,
    expert-relabel invariant, a duplicated route equals one route carrying
    the summed weight, masked routes and zero-scale experts contribute exactly
    nothing, int32 and int64 ids agree, and the output accumulates.
"""

from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from oracle import (FLT_MIN, e4m3_decode, e4m3_decode_table, experts_ref, plan_ref,
                    quant_act_ref, quant_groups_ref)
from oracle.experts import silu_mul
from moe_workloads import make_case


def _np(case):
    return dict(
        x=case.x.float().numpy(), ids=case.topk_ids.numpy(), w=case.topk_weights.numpy(),
        w13=case.w13.numpy(), w13_s=case.w13_s.numpy(), w2=case.w2.numpy(), w2_s=case.w2_s.numpy())


def _run(d, E, top_k, bm, ids=None, w=None, out_init=None, debug=None, w13_s=None):
    ids = d["ids"] if ids is None else ids
    w = d["w"] if w is None else w
    xq, xs = quant_act_ref(d["x"])
    s, x, P = plan_ref(ids, E, bm)
    return experts_ref(xq, xs, d["w13"], d["w13_s"] if w13_s is None else w13_s, d["w2"], d["w2_s"],
                       w, s, x, P, top_k, bm, out_init=out_init, debug=debug), (xq, xs, s, x, P)


@pytest.fixture(scope="module")
def tiny():
    c = make_case("tiny")
    return c, _np(c)


_T = e4m3_decode_table()


def _F(v):
    return Fraction(float(v))


def test_exact_rational_sampled(tiny):
    c, d = tiny
    dbg = {}
    res, (xq, xs, s, x, P) = _run(d, c.E, c.top_k, c.block_m, debug=dbg)
    R = c.M * c.top_k
    rows = [p for p in range(P) if s[p] < R][:3]
    I, K = c.I, c.K
    for p in rows:
        e = int(x[p // c.block_m])
        t = int(s[p]) // c.top_k
        for n in [0, 5, 127, 128, 300, I, I + 77, 2 * I - 1]:
            ex = sum(_F(_T[xq[t, k]]) * _F(xs[t, k // 128]) * _F(_T[d["w13"][e, n, k]])
                     * _F(d["w13_s"][e, n // 128, k // 128]) for k in range(K))
            got = dbg["g"][p][n]
            assert abs(Fraction(got) - ex) <= abs(ex) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 200)
        for col in [0, 1, 130, K - 1]:
            ex = sum(_F(_T[res.h_q[p, j]]) * _F(res.h_s[p, j // 128]) * _F(_T[d["w2"][e, col, j]])
                     * _F(d["w2_s"][e, col // 128, j // 128]) for j in range(I))
            got = dbg["y"][p][col]
            assert abs(Fraction(got) - ex) <= abs(ex) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 200)
    # final reduction for a couple of outputs
    for t in range(c.M):
        for col in [3, 200]:
            ex = Fraction(0)
            for j in range(c.top_k):
                r = t * c.top_k + j
                p = int(np.nonzero(s[:P] == r)[0][0])
                ex += _F(np.float32(d["w"][t, j])) * Fraction(dbg["y"][p][col])
            assert abs(Fraction(res.ref64[t, col]) - ex) <= abs(ex) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 200)


def test_silu_matches_scipy():
    rng = np.random.default_rng(0)
    g = rng.standard_normal(10000) * 20
    u = rng.standard_normal(10000)
    assert np.allclose(silu_mul(g, u), g * scipy.special.expit(g) * u, rtol=1e-14, atol=0)
    assert silu_mul(np.array([-1000.0]), np.array([3.0]))[0] == 0.0


def test_one_hot_layout():
    M, E, K, I, top_k, bm = 3, 2, 256, 256, 1, 16
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((M, K)) * 2).astype(np.float32)
    xq, xs = quant_act_ref(x)
    xd = e4m3_decode(xq) * np.repeat(xs.astype(np.float64), 128, axis=1)
    w13 = np.zeros((E, 2 * I, K), np.uint8)
    w13_s = np.ones((E, 2 * I // 128, K // 128), np.float32)
    w2 = np.zeros((E, K, I), np.uint8)
    w2_s = np.ones((E, K // 128, I // 128), np.float32)
    j0, k_gate, k_up, c0 = 131, 7, 200, 250
    e = 1
    w13[e, j0, k_gate] = 0x38                 # gate row j0 picks x[k_gate]
    w13[e, I + j0, k_up] = 0x38               # up row I + j0 picks x[k_up]
    w13_s[e, j0 // 128, k_gate // 128] = 2.0  # scale of the gate block doubles it
    w2[e, c0, j0] = 0x38                      # output column c0 picks h[j0]
    w2_s[e, c0 // 128, j0 // 128] = 0.5
    ids = np.array([[1], [0], [1]])
    w = np.array([[0.25], [1.0], [1.0]], np.float32)
    s, xe, P = plan_ref(ids, E, bm)
    dbg = {}
    res = experts_ref(xq, xs, w13, w13_s, w2, w2_s, w, s, xe, P, top_k, bm, debug=dbg)
    for t in (0, 2):
        p = int(np.nonzero(s[:P] == t)[0][0])
        g = dbg["g"][p]
        assert g[j0] == 2.0 * xd[t, k_gate] and g[I + j0] == xd[t, k_up]
        assert np.count_nonzero(g) == 2
        h = silu_mul(np.array([2.0 * xd[t, k_gate]]), np.array([xd[t, k_up]]))[0]
        hd = e4m3_decode(res.h_q[p]) * np.repeat(res.h_s[p].astype(np.float64), 128)
        assert np.count_nonzero(hd) == 1 and abs(hd[j0] - h) <= abs(h) * 2.0 ** -20
        out = res.ref64[t]
        assert np.count_nonzero(out) == 1
        assert out[c0] == float(w[t, 0]) * 0.5 * hd[j0]
    assert np.all(res.ref64[1] == 0.0)        # expert 0 has all-zero weights


def test_dense_special_case_is_plain_mlp():
    M, E, K, I = 5, 1, 384, 256
    rng = np.random.default_rng(8)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w13 = rng.integers(0, 0x7E, (1, 2 * I, K)).astype(np.uint8) | (rng.integers(0, 2, (1, 2 * I, K)) * 0x80).astype(np.uint8)
    w2 = rng.integers(0, 0x7E, (1, K, I)).astype(np.uint8)
    w13_s = rng.uniform(1e-4, 1e-3, (1, 2 * I // 128, K // 128)).astype(np.float32)
    w2_s = rng.uniform(1e-4, 1e-3, (1, K // 128, I // 128)).astype(np.float32)
    ids = np.zeros((M, 1), np.int64)
    w = np.ones((M, 1), np.float32)
    xq, xs = quant_act_ref(x)
    s, xe, P = plan_ref(ids, E, 16)
    res = experts_ref(xq, xs, w13, w13_s, w2, w2_s, w, s, xe, P, 1, 16)
    # textbook: h = silu(X W1^T) * (X W3^T), out = Q(h) W2^T
    X = e4m3_decode(xq) * np.repeat(xs.astype(np.float64), 128, axis=1)
    Wg = e4m3_decode(w13[0, :I]) * np.kron(w13_s[0, :I // 128].astype(np.float64), np.ones((128, 128)))
    Wu = e4m3_decode(w13[0, I:]) * np.kron(w13_s[0, I // 128:].astype(np.float64), np.ones((128, 128)))
    W2 = e4m3_decode(w2[0]) * np.kron(w2_s[0].astype(np.float64), np.ones((128, 128)))
    a = X @ Wg.T
    h = (a * scipy.special.expit(a) * (X @ Wu.T)).astype(np.float32)
    hq, hs = quant_groups_ref(h)
    H = e4m3_decode(hq) * np.repeat(hs.astype(np.float64), 128, axis=1)
    out = H @ W2.T
    assert np.allclose(res.ref64, out, rtol=1e-12, atol=1e-300)


def test_linear_in_route_weights(tiny):
    c, d = tiny
    a, _ = _run(d, c.E, c.top_k, c.block_m)
    b, _ = _run(d, c.E, c.top_k, c.block_m, w=(d["w"] * 2).astype(np.float32))
    assert np.array_equal(b.ref64, 2 * a.ref64)


def test_token_permutation_equivariant():
    c = make_case("tiny", M=16)
    d = _np(c)
    a, _ = _run(d, c.E, c.top_k, c.block_m)
    perm = np.random.default_rng(1).permutation(c.M)
    d2 = dict(d, x=d["x"][perm], ids=d["ids"][perm], w=d["w"][perm])
    b, _ = _run(d2, c.E, c.top_k, c.block_m)
    assert np.allclose(b.ref64, a.ref64[perm], rtol=1e-13, atol=1e-300)


def test_expert_relabel_invariant():
    c = make_case("tiny", M=16)
    d = _np(c)
    a, _ = _run(d, c.E, c.top_k, c.block_m)
    pi = np.random.default_rng(2).permutation(c.E)          # new id of old expert e is pi[e]
    inv = np.argsort(pi)
    d2 = dict(d, ids=pi[d["ids"]], w13=d["w13"][inv], w13_s=d["w13_s"][inv],
              w2=d["w2"][inv], w2_s=d["w2_s"][inv])
    b, _ = _run(d2, c.E, c.top_k, c.block_m)
    assert np.allclose(b.ref64, a.ref64, rtol=1e-12, atol=1e-300)


def test_duplicate_route_equals_summed_weight(tiny):
    c, d = tiny
    ids = d["ids"].copy()
    w = d["w"].copy()
    ids[:, 1] = ids[:, 0]
    a, _ = _run(d, c.E, c.top_k, c.block_m, ids=ids, w=w)
    ids2 = ids.copy()
    ids2[:, 1] = -1
    w2 = w.copy()
    w2[:, 0] = w[:, 0] + w[:, 1]
    b, _ = _run(d, c.E, c.top_k, c.block_m, ids=ids2, w=w2.astype(np.float32))
    assert np.allclose(a.ref64, b.ref64, rtol=1e-6, atol=1e-300)   # w0 + w1 rounds in fp32


def test_masked_route_and_zero_scale_expert(tiny):
    c, d = tiny
    ids = d["ids"].copy()
    ids[1, 0] = -1
    a, _ = _run(d, c.E, c.top_k, c.block_m, ids=ids)
    w = d["w"].copy()
    w[1, 0] = 0.0
    b, _ = _run(d, c.E, c.top_k, c.block_m, w=w)
    # BLAS may block a different number of rows differently: last-bit FP64 slack
    assert np.allclose(a.ref64, b.ref64, rtol=1e-12, atol=1e-300)
    # zero block scales on one expert == masking its routes
    e = int(d["ids"][0, 0])
    zs = d["w13_s"].copy()
    zs[e] = 0.0
    z, _ = _run(d, c.E, c.top_k, c.block_m, w13_s=zs)
    ids3 = d["ids"].copy()
    ids3[ids3 == e] = -1
    m, _ = _run(d, c.E, c.top_k, c.block_m, ids=ids3)
    assert np.allclose(z.ref64, m.ref64, rtol=1e-12, atol=1e-300)
    assert np.all(np.isfinite(z.ref64))
    # its rows requantise an all-zero h: codes 0 and the floored scale
    s, xe, P = plan_ref(d["ids"], c.E, c.block_m)
    rows = [p for p in range(P) if xe[p // c.block_m] == e and s[p] < c.M * c.top_k]
    assert np.all(z.h_q[rows] & 0x7F == 0) and np.all(z.h_s[rows] == FLT_MIN)


def test_int32_int64_ids_identical(tiny):
    c, d = tiny
    a, _ = _run(d, c.E, c.top_k, c.block_m, ids=d["ids"].astype(np.int32))
    b, _ = _run(d, c.E, c.top_k, c.block_m, ids=d["ids"].astype(np.int64))
    assert np.array_equal(a.ref64, b.ref64) and np.array_equal(a.h_q, b.h_q)


def test_output_accumulates(tiny):
    c, d = tiny
    a, _ = _run(d, c.E, c.top_k, c.block_m)
    init = np.random.default_rng(5).standard_normal((c.M, c.K)).astype(np.float32)
    b, _ = _run(d, c.E, c.top_k, c.block_m, out_init=init)
    assert np.allclose(b.ref64 - init, a.ref64, rtol=1e-12, atol=1e-12 * np.abs(init).max())


@pytest.mark.parametrize("geom", ["tiny", "page1_small"])
def test_token_sampling_equals_full_evaluation(geom):
    """experts_ref(tokens=S) -- the mode every full-size GPU parity case uses
    -- equals the full evaluation restricted to S: the intermediate codes and
    scales of S's plan rows bit for bit, S's output rows to FP64 rounding, and
    every other output row left at out_init with zero codes and the floored
    scale in the rows it skipped.  Checked on the tiny workload and on a
    page-1-like geometry (E=16, K=512, I=256, top-8, block_m=64, M=96) with a
    prefilled output."""
    if geom == "tiny":
        c = make_case("tiny")
        S = [1, 3]
    else:
        from moe_workloads import CONFIGS
        cfg = dict(CONFIGS["page1"], M=96, E=16, K=512, I=256, seed=31)
        c = make_case("page1_small", config=cfg)
        S = [0, 7, 8, 50, 95]
    d = _np(c)
    rng = np.random.default_rng(3)
    init = (rng.standard_normal((c.M, c.K)) * 0.1).astype(np.float32)
    xq, xs = quant_act_ref(d["x"])
    s, x, P = plan_ref(d["ids"], c.E, c.block_m)
    args = (xq, xs, d["w13"], d["w13_s"], d["w2"], d["w2_s"], d["w"], s, x, P, c.top_k, c.block_m)
    full = experts_ref(*args, out_init=init)
    part = experts_ref(*args, out_init=init, tokens=S)
    R = c.M * c.top_k
    tok_of_row = np.where(s < R, s // c.top_k, -1)
    in_S = np.isin(tok_of_row, S) & full.row_valid
    assert in_S.any()
    assert np.array_equal(part.h_q[in_S], full.h_q[in_S])
    assert np.array_equal(part.h_s[in_S], full.h_s[in_S])
    skipped = full.row_valid & ~in_S
    assert skipped.any()
    assert np.all(part.h_q[skipped] == 0) and np.all(part.h_s[skipped] == FLT_MIN)
    np.testing.assert_allclose(part.ref64[S], full.ref64[S], rtol=1e-12, atol=1e-14)
    others = np.setdiff1d(np.arange(c.M), S)
    assert np.array_equal(part.ref64[others], init[others].astype(np.float64))
    assert np.array_equal(np.nonzero(part.computed_tokens)[0], np.asarray(sorted(S)))
    # and the sampled rows really differ from out_init (the routes were added)
    assert not np.allclose(part.ref64[S], init[S].astype(np.float64))
