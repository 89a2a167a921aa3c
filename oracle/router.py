"""Router: softmax top-k with routed scaling and an optional shared expert,
written out from its definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

FlashInfer PR #4287 runs its expert kernel behind a fixed router (real-model
evaluation: the AlphaMoE router held fixed; its companion router PR is named
among the related PRs) and states the two geometries it routes for in its
retained-measurements notes: routed scaling 1.0 with no shared expert, and
routed scaling 2.5 with one shared expert (E=257, top-9 including the shared
one).  The workload descriptions route with softmax over the experts, top-k,
and weights renormalised over the chosen experts.

Readings taken where the pages are silent:
  * the k chosen experts are the k largest logits, compared exactly as FP32
    values (softmax is increasing, so this is the top-k of the
    probabilities without the ties that rounding exp could create); equal
    logits go to the lower expert index; they are listed in that order
    (largest first);
  * weight of a chosen expert i: exp(l_i) / sum over the chosen exp(l_j),
    times the routed scaling factor (the full softmax denominator cancels in
    the renormalisation), computed here in FP64;
  * a shared expert is expert E_routed, appended to every token as route
    slot top_k with weight 1 (the routed scaling applies to routed experts
    only);
  * logits are finite.
"""

import numpy as np


def router_ref(logits, top_k, n_shared=0, routed_scaling=1.0):
    """logits: float32 [M, E_routed].  Returns (ids int32 [M, top_k + n_shared],
    weights float64 [M, top_k + n_shared])."""
    logits = np.asarray(logits, dtype=np.float32)
    M, E = logits.shape
    assert 1 <= top_k <= E and n_shared in (0, 1)
    # descending by value, ascending index among equal values
    order = np.lexsort((np.broadcast_to(np.arange(E), (M, E)), -logits.astype(np.float64)), axis=1)
    ids = order[:, :top_k].astype(np.int32)
    chosen = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    e = np.exp(chosen - chosen[:, :1])
    w = e / e.sum(axis=1, keepdims=True) * float(np.float32(routed_scaling))
    if n_shared:
        ids = np.concatenate([ids, np.full((M, 1), E, dtype=np.int32)], axis=1)
        w = np.concatenate([w, np.ones((M, 1))], axis=1)
    return ids, w
