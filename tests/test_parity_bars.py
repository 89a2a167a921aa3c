"""The parity bars themselves (CPU only): the output comparison accepts the
oracle's own BF16-rounded output -- the bar must not reject the exact answer
rounded once to the output dtype -- and rejects an element moved by more than
2e-2 * rms beyond its rounding; the intermediate-code comparison accepts
one-step moves within the budget and rejects two-step moves or too many."""

import numpy as np
import pytest

from oracle import bf16_round_f64, e4m3_encode
from parity import compare_intermediate, compare_output


def _ref(seed, shape=(64, 512), outliers=True):
    rng = np.random.default_rng(seed)
    r = rng.standard_normal(shape)
    if outliers:                       # a few elements far out, as routed sums produce
        r.flat[rng.choice(r.size, 8, replace=False)] *= 9.0
    return r


@pytest.mark.parametrize("seed", range(4))
def test_oracle_bf16_output_passes(seed):
    r = _ref(seed)
    st = compare_output(bf16_round_f64(r), r)
    assert st["max_abs_over_rms"] > 0


def test_small_element_moved_beyond_bar_fails():
    r = _ref(7, outliers=False)
    rms = float(np.sqrt(np.mean(r * r)))
    g = bf16_round_f64(r).copy()
    i = int(np.argmin(np.abs(r)))          # tiny element: its rounding allowance is ~0
    g.flat[i] = r.flat[i] + 0.021 * rms
    with pytest.raises(AssertionError, match="exceed"):
        compare_output(g, r)
    g.flat[i] = r.flat[i] + 0.019 * rms
    compare_output(g, r)


def test_rel_l2_bar():
    r = _ref(8, outliers=False)
    g = r * (1 + 6e-3)
    with pytest.raises(AssertionError, match="relative L2"):
        compare_output(g, r)


def _codes(seed, P=64, I=256):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((P, I)).astype(np.float32) * 100
    q = e4m3_encode(h)
    s = np.ones((P, I // 128), np.float32)
    return q, s


def test_intermediate_one_step_within_budget_passes():
    q, s = _codes(1, P=160, I=512)
    g = q.copy()
    g.flat[5] = q.flat[5] + (1 if q.flat[5] & 0x7F < 0x7E else -1)   # one step, same sign
    rows = np.ones(q.shape[0], bool)
    st = compare_intermediate(g, s, q, s, rows, max_frac=1e-4)
    assert st["mismatched"] == 1


def test_intermediate_two_steps_fail():
    q, s = _codes(2, P=160, I=512)
    g = q.copy()
    flat = np.nonzero(((q & 0x7F) > 0x10) & ((q & 0x7F) < 0x70))
    i = (flat[0][0], flat[1][0])
    g[i] = q[i] + 2
    rows = np.ones(q.shape[0], bool)
    with pytest.raises(AssertionError, match="more than one step"):
        compare_intermediate(g, s, q, s, rows, max_frac=1e-4)


def test_intermediate_budget_exceeded_fails():
    q, s = _codes(3, P=16, I=256)      # 4096 codes: one move is 2.4e-4 > 1e-4
    g = q.copy()
    g[0, 3] = q[0, 3] + 1 if (q[0, 3] & 0x7F) < 0x7E else q[0, 3] - 1
    rows = np.ones(q.shape[0], bool)
    with pytest.raises(AssertionError, match="fraction"):
        compare_intermediate(g, s, q, s, rows)
