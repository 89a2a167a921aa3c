"""Pins for the oracle's router (CPU only).

Checked against:
  * brute force on small expert counts: the chosen set is the unique k-subset
    whose every member beats every non-member under (larger logit, then
    lower index), found by enumerating all k-subsets, and the listed order is
    that same ranking;
  * torch's softmax + topk (library routines) on continuous logits, where
    ties have probability zero: same experts, same order, and weights within
    FP32 rounding of torch's renormalised probabilities;
  * closed forms: with top_k = E the weights are the full softmax (scipy's)
    times the scaling; with top_k = 1 the weight is the scaling itself;
    weight ratios are exp(l_i - l_j);
  * invariants: adding a constant to a token's logits changes nothing; the
    routed weights sum to the scaling factor; relabelling experts relabels
    the choice; the shared expert is slot top_k with weight 1.
"""

import itertools

import numpy as np
import pytest
import scipy.special
import torch

from oracle import router_ref


def _rank_key(l, i):
    return (-float(l[i]), i)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("E,k", [(5, 1), (6, 3), (7, 7), (8, 4)])
def test_brute_force_selection_with_ties(seed, E, k):
    rng = np.random.default_rng(seed * 100 + E * 10 + k)
    # few distinct values: many exact ties
    logits = rng.integers(-2, 3, size=(12, E)).astype(np.float32)
    ids, _ = router_ref(logits, k)
    for t in range(logits.shape[0]):
        l = logits[t]
        best = None
        for S in itertools.combinations(range(E), k):
            rest = [j for j in range(E) if j not in S]
            if all(_rank_key(l, i) < _rank_key(l, j) for i in S for j in rest):
                assert best is None, "two subsets satisfy the ranking"
                best = S
        assert best is not None
        assert sorted(ids[t].tolist()) == sorted(best)
        listed = ids[t].tolist()
        assert listed == sorted(listed, key=lambda i: _rank_key(l, i))


def test_matches_torch_softmax_topk():
    g = torch.Generator().manual_seed(7)
    logits = torch.randn((300, 288), generator=g)
    probs = torch.softmax(logits, dim=-1)
    tw, tids = torch.topk(probs, 8, dim=-1)
    tw = tw / tw.sum(dim=-1, keepdim=True)
    ids, w = router_ref(logits.numpy(), 8)
    assert np.array_equal(ids, tids.numpy().astype(np.int32))
    np.testing.assert_allclose(w, tw.double().numpy(), rtol=2e-6)


def test_closed_forms():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((20, 9)).astype(np.float32)
    ids, w = router_ref(logits, 9, routed_scaling=2.5)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids, 1) * 2.5, rtol=1e-12)
    ids1, w1 = router_ref(logits, 1, routed_scaling=2.5)
    assert np.array_equal(ids1[:, 0], np.argmax(logits, axis=1)) and np.all(w1 == 2.5)
    ids3, w3 = router_ref(logits, 3)
    l = np.take_along_axis(logits, ids3, 1).astype(np.float64)
    np.testing.assert_allclose(w3[:, 0] / w3[:, 1], np.exp(l[:, 0] - l[:, 1]), rtol=1e-12)


def test_invariants_and_shared_expert():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((50, 256)).astype(np.float32)
    ids, w = router_ref(logits, 8, n_shared=1, routed_scaling=2.5)
    assert ids.shape == (50, 9) and np.all(ids[:, 8] == 256) and np.all(w[:, 8] == 1.0)
    np.testing.assert_allclose(w[:, :8].sum(1), 2.5, rtol=1e-12)
    # shift by a constant that is exact in FP32 (a power of two, values stay exact)
    ids2, w2 = router_ref(logits + np.float32(4.0), 8, n_shared=1, routed_scaling=2.5)
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-6)
    perm = rng.permutation(256)
    ids3, w3 = router_ref(logits[:, perm], 8)
    assert np.array_equal(perm[ids3], ids[:, :8])
    np.testing.assert_allclose(w3, w[:, :8] / 2.5, rtol=1e-12)


def test_signed_zeros_are_one_value():
    logits = np.array([[0.0, -0.0, -1.0, 0.0], [-0.0, 0.0, 0.0, -0.0]], dtype=np.float32)
    ids, w = router_ref(logits, 3)
    assert ids.tolist() == [[0, 1, 3], [0, 1, 2]]
    np.testing.assert_allclose(w, 1.0 / 3.0, rtol=1e-15)
