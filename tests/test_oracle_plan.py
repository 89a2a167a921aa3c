"""Pins for the oracle's routing plan (CPU only).

Checked against:
  * a brute-force construction (scan every expert, then every route in
    order) written directly from the plan's definition;
  * the special case block_m = 1, which is a stable argsort of the valid ids
    (numpy's library routine);
  * invariants: each valid route appears exactly once, each expert's segment
    is padded to the block_m round-up, #sentinels = P - R_valid, expert ids
    are non-decreasing, P never exceeds the worst-case capacity;
  * the worst case that makes the capacity bound tight.
"""

import numpy as np
import pytest
import torch

from oracle import plan_capacity, plan_ref
from moe_workloads import make_routing


def _brute_plan(ids, E, bm):
    ids = [int(i) for i in np.asarray(ids).reshape(-1)]
    R = len(ids)
    sorted_ids, expert_ids = [], []
    for e in range(E):
        mine = [r for r in range(R) if ids[r] == e]
        if not mine:
            continue
        nblk = (len(mine) + bm - 1) // bm
        sorted_ids += mine + [R] * (nblk * bm - len(mine))
        expert_ids += [e] * nblk
    return np.array(sorted_ids, np.int32), np.array(expert_ids, np.int32), len(sorted_ids)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("bm", [1, 4, 16, 64])
def test_plan_matches_brute_force(seed, bm):
    rng = np.random.default_rng(seed)
    M, top_k, E = int(rng.integers(1, 40)), int(rng.integers(1, 6)), int(rng.integers(1, 20))
    ids = rng.integers(-2, E + 2, size=(M, top_k))          # includes masked / out-of-range
    s, x, P = plan_ref(ids, E, bm)
    bs, bx, bP = _brute_plan(ids, E, bm)
    assert P == bP
    assert np.array_equal(s, bs) and np.array_equal(x, bx)


def test_plan_int32_int64_identical():
    rng = np.random.default_rng(5)
    ids = rng.integers(-1, 33, size=(50, 4))
    a = plan_ref(ids.astype(np.int32), 33, 16)
    b = plan_ref(ids.astype(np.int64), 33, 16)
    assert a[2] == b[2] and np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_plan_block_m_1_is_stable_argsort():
    rng = np.random.default_rng(11)
    ids = rng.integers(-1, 50, size=(300, 7)).reshape(-1)
    s, x, P = plan_ref(ids, 50, 1)
    valid = np.nonzero((ids >= 0) & (ids < 50))[0]
    order = valid[np.argsort(ids[valid], kind="stable")]
    assert P == valid.size
    assert np.array_equal(s, order)
    assert np.array_equal(x, ids[order])


def _check_invariants(ids, E, bm):
    ids = np.asarray(ids).reshape(-1)
    R = ids.size
    s, x, P = plan_ref(ids, E, bm)
    valid = (ids >= 0) & (ids < E)
    cap, bcap = plan_capacity(R, 1, E, bm)
    assert P <= cap and P % bm == 0 and len(x) == P // bm
    real = s[s < R]
    assert np.array_equal(np.sort(real), np.nonzero(valid)[0])     # each valid route once
    assert np.count_nonzero(s == R) == P - valid.sum()
    assert np.all(np.diff(x) > 0) if len(x) > 1 and bm == 1 else np.all(np.diff(x) >= 0)
    for e in np.unique(x):
        blocks = np.nonzero(x == e)[0]
        assert np.array_equal(blocks, np.arange(blocks[0], blocks[-1] + 1))
        seg = s[blocks[0] * bm:(blocks[-1] + 1) * bm]
        c = int(np.count_nonzero(ids == e))
        assert len(seg) == -(-c // bm) * bm                        # padding = round-up
        assert np.all(ids[seg[:c]] == e) and np.all(np.diff(seg[:c]) > 0)
        assert np.all(seg[c:] == R)


@pytest.mark.parametrize("kind,M,E,top_k,bm", [
    ("softmax", 4, 8, 2, 16),
    ("softmax", 1, 257, 9, 16),
    ("softmax", 256, 288, 8, 64),
    ("skew", 128, 512, 10, 64),
    ("zipf", 256, 288, 8, 128),
])
def test_plan_invariants_on_workload_routing(kind, M, E, top_k, bm):
    ids, _ = make_routing(kind, M, E, top_k, seed=3, device="cpu")
    _check_invariants(ids.numpy(), E, bm)


def test_plan_all_masked():
    ids = -np.ones((10, 3), np.int64)
    s, x, P = plan_ref(ids, 4, 16)
    assert P == 0 and s.size == 0 and x.size == 0


def test_capacity_is_tight():
    # every route hits a different expert: each needs a whole block
    R, bm = 37, 16
    ids = np.arange(R)
    s, x, P = plan_ref(ids, 64, bm)
    cap, bcap = plan_capacity(R, 1, 64, bm)
    assert P == cap == R * bm and bcap == R
    # capacity formula at the workload sizes
    assert plan_capacity(4, 2, 8, 16) == (128, 8)
    assert plan_capacity(1, 9, 257, 16) == (144, 9)
    assert plan_capacity(4096, 8, 288, 64)[0] == 50944
    assert plan_capacity(2048, 10, 512, 64) == (52736, 824)
    assert plan_capacity(8192, 8, 288, 128) == (102144, 798)
