"""moe_align_block_size routing plan, written out from its definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

FlashInfer PR #4287 (PR summary) runs its expert kernel over "the standard
moe_align_block_size routing plan": routes grouped by expert, each expert's
group padded to a multiple of block_m, one expert id per block, and a
device-side count ``num_tokens_post_padded``; its public-contract section and
the review of the host checks require ``sorted_token_ids`` to hold at least
``len(expert_ids) * block_m`` entries.  sglang-glm53-flash-sm120 PR #13
(description, validation) adds masked routes (``topk_id = -1``) with int32 or
int64 ids.

The pages leave the order inside an expert, the padding sentinel and the
treatment of out-of-range ids open.  Readings taken here:
  * a flat route index is r = t * top_k + j; the sentinel is R = M * top_k;
  * every id outside [0, E) is a masked route and appears nowhere;
  * inside an expert, routes keep ascending r (a stable counting sort);
  * experts are laid out in ascending id order, empty experts take no block;
  * entries at or beyond P (and expert ids at or beyond P / block_m) are
    unspecified.
"""

import numpy as np


def plan_capacity(M, top_k, E, block_m):
    """Worst-case plan sizes (sorted_cap, blocks_cap) for any routing.

    Every non-empty expert holds at least one route, so at most min(E, R)
    experts each add at most block_m - 1 padding slots to the R routes.
    """
    R = M * top_k
    n = R + min(E, R) * (block_m - 1)
    sorted_cap = -(-n // block_m) * block_m
    return sorted_cap, sorted_cap // block_m


def plan_ref(topk_ids, E, block_m):
    """Return (sorted_token_ids int32 [P], expert_ids int32 [P/block_m], P)."""
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    R = ids.size
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E)[:E]
    padded = -(-counts // block_m) * block_m
    offsets = np.zeros(E, dtype=np.int64)
    if E > 1:
        offsets[1:] = np.cumsum(padded)[:-1]
    P = int(padded.sum())
    sorted_ids = np.full(P, R, dtype=np.int32)
    expert_ids = np.empty(P // block_m, dtype=np.int32)
    for e in range(E):
        if counts[e] == 0:
            continue
        routes = np.nonzero(ids == e)[0]          # ascending flat index
        o = int(offsets[e])
        sorted_ids[o:o + routes.size] = routes
        expert_ids[o // block_m:(o + int(padded[e])) // block_m] = e
    return sorted_ids, expert_ids, P
