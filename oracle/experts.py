"""Routed expert computation: gate/up GEMM, SwiGLU + requant, down GEMM,
route weighting and reduce-add.  Dot products in FP64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What FlashInfer PR #4287 computes over an aligned plan (PR summary, "Public
contract and review fixes", the retained-measurements fixture notes):
  for every plan row p holding a real route r (t = r // top_k, expert
  e = expert_ids[p // block_m]):
    g[p, n] = sum_k  xdq[t, k] * W13dq[e, n, k],        n < 2I
      with xdq    = code value * x_s[t, k // 128]          (1x128 groups)
           W13dq  = code value * w13_s[e, n // 128, k // 128] (128x128 blocks)
    h[p, j] = silu(g[p, j]) * g[p, I + j],               j < I
      (rows [0, I) of W13 are the gate projection, rows [I, 2I) the up
       projection -- the logical layout; the page's eight-row interleave is a
       private weight prepack and is not used here)
    h is requantised to E4M3 per row and 128-column group (FP32 mirror of the
    GPU rounding points: h is rounded to FP32 first, then scale, inverse and
    codes follow the activation rule)
    y[p, c] = sum_j hdq[p, j] * W2dq[e, c, j],           c < K
    out[t, c] += w[r] * y[p, c]
The caller's output is an accumulator (PR summary: a caller-owned BF16 output
that the kernel adds into).  The reduction here is exact FP64 over all routes
and one final BF16 rounding is reported separately.

Weights are dequantised one expert at a time, never all at once (a point the
PR's review raised for its own reference).
"""

from dataclasses import dataclass

import numpy as np

from .e2m1 import dequant_k32
from .e4m3 import bf16_round_f64, e4m3_decode
from .quant import SCALE_FP32, quant_groups_ref


@dataclass
class ExpertsResult:
    h_q: np.ndarray          # uint8 [P, I]   intermediate codes (plan-row indexed)
    h_s: np.ndarray          # float32 [P, I/128]
    row_valid: np.ndarray    # bool [P]       rows that hold a real route
    ref64: np.ndarray        # float64 [M, K] out_init + sum of routes
    out_bf16: np.ndarray     # float64 [M, K] ref64 rounded once to BF16
    computed_tokens: np.ndarray  # bool [M]   tokens whose routes were evaluated


def dequant_blocks(codes, s):
    """E4M3 codes [rows, cols] times their [rows/128, cols/128] block scales,
    as float64 [rows, cols]."""
    rows, cols = codes.shape
    v = e4m3_decode(codes).reshape(rows // 128, 128, cols // 128, 128)
    v *= s.astype(np.float64)[:, None, :, None]
    return v.reshape(rows, cols)


def silu_mul(gate, up):
    """silu(gate) * up with silu(v) = v / (1 + e^-v), in FP64."""
    with np.errstate(over="ignore"):
        return gate / (1.0 + np.exp(-gate)) * up


def experts_ref(x_q, x_s, w13, w13_s, w2, w2_s, topk_weights, sorted_ids,
                expert_ids, P, top_k, block_m, out_init=None,
                inter_mode=SCALE_FP32, tokens=None, debug=None):
    """Evaluate the expert path over a given plan (W8A8: E4M3 weights with
    128x128 FP32 block scales).

    tokens: optional iterable of token indices; when given, only routes of
    those tokens are evaluated (same arithmetic, used to sample very large
    cases); rows of other tokens stay at out_init.
    debug: optional dict; receives the FP64 gate/up sums ``g`` and the FP64
    down-projection rows ``y`` keyed by plan row.
    """
    E, twoI, K = w13.shape
    I = twoI // 2
    assert w2.shape == (E, K, I)
    return _experts_core(x_q, x_s, lambda e: dequant_blocks(w13[e], w13_s[e]),
                         lambda e: dequant_blocks(w2[e], w2_s[e]), E, I, topk_weights,
                         sorted_ids, expert_ids, P, top_k, block_m, out_init, inter_mode, tokens,
                         debug)


def experts_w4a8_ref(x_q, x_s, w13, w13_s, w2, w2_s, topk_weights, sorted_ids,
                     expert_ids, P, top_k, block_m, out_init=None,
                     inter_mode=SCALE_FP32, tokens=None, debug=None):
    """The same expert path with E2M1 weights and K32 power-of-two scales
    (sglang-glm53-flash-sm120 PR #13, description: FP8 activations against
    E2M1-K32 weights, the weight scales applied in FP32):
      w13 uint8 [E, 2I, K/2] packed E2M1 (even K in the low nibble),
      w13_s uint8 [E, 2I, K/32] UE8M0 scale bytes; w2 [E, K, I/2], w2_s
      [E, K, I/32] likewise.  Activations and the intermediate keep their
    1x128 FP8 quantisation, so only the weight dequantisation differs."""
    E, twoI, half = w13.shape
    K, I = 2 * half, twoI // 2
    assert w2.shape == (E, K, I // 2) and w13_s.shape == (E, twoI, K // 32)
    return _experts_core(x_q, x_s, lambda e: dequant_k32(w13[e], w13_s[e]),
                         lambda e: dequant_k32(w2[e], w2_s[e]), E, I, topk_weights, sorted_ids,
                         expert_ids, P, top_k, block_m, out_init, inter_mode, tokens, debug)


def _experts_core(x_q, x_s, deq13, deq2, E, I, topk_weights, sorted_ids, expert_ids, P, top_k,
                  block_m, out_init, inter_mode, tokens, debug):
    """The expert path with the weights of expert e given dequantised by
    deq13(e) -> FP64 [2I, K] and deq2(e) -> FP64 [K, I]."""
    x_q = np.asarray(x_q)
    M, K = x_q.shape
    assert I % 128 == 0 and K % 128 == 0
    R = M * top_k
    wflat = np.asarray(topk_weights, dtype=np.float32).reshape(-1).astype(np.float64)
    sorted_ids = np.asarray(sorted_ids, dtype=np.int64)[:P]
    nblk = P // block_m
    expert_ids = np.asarray(expert_ids, dtype=np.int64)[:nblk]

    if out_init is None:
        acc = np.zeros((M, K), dtype=np.float64)
    else:
        acc = np.asarray(out_init, dtype=np.float32).astype(np.float64).copy()

    take = np.ones(M, dtype=bool)
    if tokens is not None:
        take = np.zeros(M, dtype=bool)
        take[np.asarray(list(tokens), dtype=np.int64)] = True

    row_valid = (sorted_ids >= 0) & (sorted_ids < R)
    h_q = np.zeros((P, I), dtype=np.uint8)
    h_s = np.zeros((P, I // 128), dtype=np.float32)
    # Padding rows see an all-zero A row: codes 0 and the floored scale.
    zc, zs = quant_groups_ref(np.zeros((1, I), np.float32), inter_mode)
    h_s[:] = zs[0]

    row_expert = np.repeat(expert_ids, block_m)
    for e in np.unique(expert_ids):
        rows = np.nonzero((row_expert == e) & row_valid)[0]
        if rows.size == 0:
            continue
        r = sorted_ids[rows]
        t = r // top_k
        keep = take[t]
        rows, r, t = rows[keep], r[keep], t[keep]
        if rows.size == 0:
            continue
        # gathered activation rows, dequantised
        A = e4m3_decode(x_q[t]) * np.repeat(x_s[t].astype(np.float64), 128, axis=1)
        W13d = deq13(e)
        g = A @ W13d.T                                  # [n, 2I] FP64
        del W13d
        if debug is not None:
            debug.setdefault("g", {}).update({int(p): g[i] for i, p in enumerate(rows)})
        h64 = silu_mul(g[:, :I], g[:, I:])
        h32 = h64.astype(np.float32)
        codes, scales = quant_groups_ref(h32, inter_mode)
        h_q[rows] = codes
        h_s[rows] = scales
        Hd = e4m3_decode(codes) * np.repeat(scales.astype(np.float64), 128, axis=1)
        W2d = deq2(e)
        y = Hd @ W2d.T                                  # [n, K] FP64
        del W2d
        if debug is not None:
            debug.setdefault("y", {}).update({int(p): y[i] for i, p in enumerate(rows)})
        np.add.at(acc, t, wflat[r][:, None] * y)

    return ExpertsResult(h_q=h_q, h_s=h_s, row_valid=row_valid, ref64=acc,
                         out_bf16=bf16_round_f64(acc), computed_tokens=take)
