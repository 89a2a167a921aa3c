"""Seeded synthetic workloads for the routed FP8 MoE expert path.

This module only synthesises inputs: it holds none of the expert path's
arithmetic.  Both the CPU oracle and the HIP library receive the bytes it
produces.  Weight storage (E4M3 codes with one FP32 scale per 128x128 block)
uses torch's own ``float8_e4m3fn`` cast after a clamp to +-448, a library
routine that is neither the oracle's codec nor the GPU kernels' converter.

Workloads (the sizes the method's pages measure, plus a decode, a skewed and a
power-of-two-scale case):
  tiny    M=4,    E=8,   K=256,  I=256,  top_k=2,  block_m=16
  decode  M=1,    E=257, K=7168, I=256,  top_k=9,  block_m=16
  page1   M=4096, E=288, K=4096, I=1024, top_k=8,  block_m=64 (M sweep 1024..8192)
  skew    M=2048, E=512, K=2048, I=512,  top_k=10, block_m=64
  zipf    M=8192, E=288, K=4096, I=1024, top_k=8,  block_m=128, power-of-two scales

W4A8 variant (``make_case(..., fmt="w4a8")``): the same masters stored as
E2M1 codes, two per byte (even K index in the low nibble), with one
power-of-two scale per 32 consecutive K -- 2^e, e the least integer with
6 * 2^e >= amax of the 32 values, kept as its biased exponent byte e + 127.
Codes round to nearest with ties to the even code, by comparison against the
seven midpoints of the E2M1 grid.  For ``skew`` the zero-scale expert cannot
be expressed (a power-of-two scale is never zero): its codes are all zero.

Recipe (every random draw from one ``torch.Generator`` per tensor kind,
seeded from the workload seed):
  x        bf16(N(0, 1))                                        [M, K]
  weights  N(0, 0.02^2) FP32 masters, per expert; scale per 128x128 block
           s = amax / 448 (FP32) or, for ``zipf``, s = 2^e with e the least
           integer with 448 * 2^e >= amax; codes = e4m3fn(clamp(w / s, +-448))
  routing  tiny/decode/page1: logits N(0,1) [M, E] -> softmax -> top-k ->
           weights renormalised to sum 1 (FP32)
           skew: slots 0..4 of each token draw i.i.d. from the hot set
           {0, 170, 341, 511}, slots 5..9 i.i.d. uniform over E (so a token
           may repeat an expert); weights softmax(N(0,1)) over the 10 slots;
           exactly 1% of routes (205 of 20,480) set to -1; expert 170 has all
           W13 and W2 block scales zero
           zipf: Gumbel-top-k, logit = log p_e + Gumbel(0, 1) with
           p_e proportional to (pi(e) + 1)^-1.1 for a seeded permutation pi;
           weights = softmax over the chosen logits
"""

from dataclasses import dataclass, field
import math

import torch

CONFIGS = {
    "tiny":   dict(M=4,    E=8,   K=256,  I=256,  top_k=2,  block_m=16,  seed=0, routing="softmax", pow2=False),
    "decode": dict(M=1,    E=257, K=7168, I=256,  top_k=9,  block_m=16,  seed=1, routing="softmax", pow2=False),
    "page1":  dict(M=4096, E=288, K=4096, I=1024, top_k=8,  block_m=64,  seed=2, routing="softmax", pow2=False),
    "skew":   dict(M=2048, E=512, K=2048, I=512,  top_k=10, block_m=64,  seed=3, routing="skew",    pow2=False),
    "zipf":   dict(M=8192, E=288, K=4096, I=1024, top_k=8,  block_m=128, seed=4, routing="zipf",    pow2=True),
}

SKEW_HOT = (0, 170, 341, 511)
SKEW_ZERO_SCALE_EXPERT = 170
SKEW_MASK_FRACTION = 0.01


@dataclass
class Case:
    name: str
    M: int
    E: int
    K: int
    I: int
    top_k: int
    block_m: int
    pow2: bool
    x: torch.Tensor            # bf16 [M, K]
    topk_ids: torch.Tensor     # int32 or int64 [M, top_k]
    topk_weights: torch.Tensor # fp32 [M, top_k]
    w13: torch.Tensor          # uint8 [E, 2I, K]           (w4a8: [E, 2I, K/2])
    w13_s: torch.Tensor        # fp32 [E, 2I/128, K/128]   (w4a8: uint8 [E, 2I, K/32])
    w2: torch.Tensor           # uint8 [E, K, I]            (w4a8: [E, K, I/2])
    w2_s: torch.Tensor         # fp32 [E, K/128, I/128]    (w4a8: uint8 [E, K, I/32])
    meta: dict = field(default_factory=dict)


def _gen(device, seed, kind):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + kind)
    return g


def _block_quant(w, pow2):
    """Store FP32 masters [rows, cols] as E4M3 codes + one scale per block."""
    rows, cols = w.shape
    blk = w.reshape(rows // 128, 128, cols // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))                       # [rows/128, cols/128]
    if pow2:
        m, x = torch.frexp(amax)
        e = torch.where(m <= 0.875, x - 9, x - 8)
        e = torch.where(amax == 0, torch.full_like(e, -126), e).clamp_min(-126)
        s = torch.ldexp(torch.ones_like(amax), e)
    else:
        s = (amax / 448.0).clamp_min(2.0 ** -126)
    q = (blk / s[:, None, :, None]).clamp(-448.0, 448.0)
    codes = q.reshape(rows, cols).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, s.to(torch.float32)


# E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6: the midpoints between
# neighbours, and whether a value exactly on one goes to the upper neighbour
# (the neighbour with an even code wins a tie)
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_TIE_UP = (False, True, False, True, False, True, False)


def _k32_quant(w):
    """Store FP32 masters [rows, cols] as packed E2M1 [rows, cols/2] plus one
    biased-exponent byte per 32 columns [rows, cols/32]."""
    rows, cols = w.shape
    grp = w.reshape(rows, cols // 32, 32).to(torch.float64)
    amax = grp.abs().amax(dim=-1)
    e = torch.ceil(torch.log2(torch.where(amax > 0, amax / 6.0, torch.ones_like(amax))))
    e = torch.where(6.0 * torch.exp2(e) < amax, e + 1, e)          # guard log2 rounding
    e = torch.where(6.0 * torch.exp2(e - 1) >= amax, e - 1, e)
    e = torch.where(amax == 0, torch.full_like(e, -126.0), e).clamp(-126, 126)
    q = grp / torch.exp2(e)[..., None]
    a = q.abs().clamp_max(6.0)
    m = torch.zeros_like(a, dtype=torch.int64)
    for mid, up in zip(_E2M1_MID, _E2M1_TIE_UP):
        m += (a >= mid) if up else (a > mid)
    codes = (m | (torch.signbit(q).to(torch.int64) << 3)).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).to(torch.uint8)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


def make_weights_w4(E, K, I, seed, device, std=0.02):
    """The W4A8 variant's weights, from the same seeded masters as
    make_weights: (w13 [E, 2I, K/2], w13_e [E, 2I, K/32], w2 [E, K, I/2],
    w2_e [E, K, I/32]), all uint8."""
    g = _gen(device, seed, 1)
    w13 = torch.empty((E, 2 * I, K // 2), dtype=torch.uint8, device=device)
    w13_e = torch.empty((E, 2 * I, K // 32), dtype=torch.uint8, device=device)
    w2 = torch.empty((E, K, I // 2), dtype=torch.uint8, device=device)
    w2_e = torch.empty((E, K, I // 32), dtype=torch.uint8, device=device)
    for e in range(E):
        m13 = torch.randn((2 * I, K), generator=g, device=device, dtype=torch.float32) * std
        w13[e], w13_e[e] = _k32_quant(m13)
        m2 = torch.randn((K, I), generator=g, device=device, dtype=torch.float32) * std
        w2[e], w2_e[e] = _k32_quant(m2)
    return w13, w13_e, w2, w2_e


def make_weights(E, K, I, seed, pow2, device, std=0.02):
    g = _gen(device, seed, 1)
    w13 = torch.empty((E, 2 * I, K), dtype=torch.uint8, device=device)
    w13_s = torch.empty((E, 2 * I // 128, K // 128), dtype=torch.float32, device=device)
    w2 = torch.empty((E, K, I), dtype=torch.uint8, device=device)
    w2_s = torch.empty((E, K // 128, I // 128), dtype=torch.float32, device=device)
    for e in range(E):
        m13 = torch.randn((2 * I, K), generator=g, device=device, dtype=torch.float32) * std
        w13[e], w13_s[e] = _block_quant(m13, pow2)
        m2 = torch.randn((K, I), generator=g, device=device, dtype=torch.float32) * std
        w2[e], w2_s[e] = _block_quant(m2, pow2)
    return w13, w13_s, w2, w2_s


def make_routing(kind, M, E, top_k, seed, device):
    g = _gen(device, seed, 2 + 1000 * M)
    if kind == "softmax":
        logits = torch.randn((M, E), generator=g, device=device, dtype=torch.float32)
        probs = torch.softmax(logits, dim=-1)
        w, ids = torch.topk(probs, top_k, dim=-1)
        w = w / w.sum(dim=-1, keepdim=True)
    elif kind == "skew":
        assert top_k == 10 and E > max(SKEW_HOT)
        hot = torch.tensor(SKEW_HOT, device=device)
        hi = torch.randint(0, len(SKEW_HOT), (M, 5), generator=g, device=device)
        rest = torch.randint(0, E, (M, top_k - 5), generator=g, device=device)
        ids = torch.cat([hot[hi], rest], dim=1)
        w = torch.softmax(torch.randn((M, top_k), generator=g, device=device), dim=-1)
        n_mask = int(round(SKEW_MASK_FRACTION * M * top_k))
        perm = torch.randperm(M * top_k, generator=g, device=device)[:n_mask]
        ids = ids.reshape(-1)
        ids[perm] = -1
        ids = ids.reshape(M, top_k)
    elif kind == "zipf":
        perm = torch.randperm(E, generator=g, device=device)
        p = (perm.to(torch.float64) + 1.0) ** -1.1
        logp = torch.log(p / p.sum()).to(torch.float32)
        u = torch.rand((M, E), generator=g, device=device, dtype=torch.float32)
        u = u.clamp(1e-20, 1.0 - 1e-7)
        gumbel = -torch.log(-torch.log(u))
        logits = logp[None, :] + gumbel
        top, ids = torch.topk(logits, top_k, dim=-1)
        w = torch.softmax(top, dim=-1)
    else:
        raise ValueError(kind)
    return ids.to(torch.int64), w.to(torch.float32).contiguous()


def make_case(name, M=None, device="cpu", ids_dtype=torch.int32, weights=None, config=None,
              fmt="w8a8"):
    """Build a workload.  ``weights`` may pass a previously built
    (w13, w13_s, w2, w2_s) tuple of the same geometry and format (M sweeps
    reuse the parent's weights; routing and x are seeded by (seed, M)).
    ``config`` (same keys as a CONFIGS entry) builds an ad-hoc geometry under
    ``name``.  fmt "w4a8": E2M1 weights with K32 exponent bytes in the
    w13 / w13_s / w2 / w2_s fields (shapes in make_weights_w4)."""
    assert fmt in ("w8a8", "w4a8")
    c = dict(CONFIGS[name] if config is None else config)
    if M is not None:
        c["M"] = M
    M, E, K, I, top_k = c["M"], c["E"], c["K"], c["I"], c["top_k"]
    seed = c["seed"]
    if weights is None:
        weights = make_weights(E, K, I, seed, c["pow2"], device) if fmt == "w8a8" \
            else make_weights_w4(E, K, I, seed, device)
    w13, w13_s, w2, w2_s = weights
    if c["routing"] == "skew":
        if fmt == "w8a8":
            w13_s[SKEW_ZERO_SCALE_EXPERT].zero_()
            w2_s[SKEW_ZERO_SCALE_EXPERT].zero_()
        else:
            w13[SKEW_ZERO_SCALE_EXPERT].zero_()
            w2[SKEW_ZERO_SCALE_EXPERT].zero_()
    gx = _gen(device, seed, 3 + 1000 * M)
    x = torch.randn((M, K), generator=gx, device=device, dtype=torch.float32).to(torch.bfloat16)
    ids, w = make_routing(c["routing"], M, E, top_k, seed, device)
    return Case(name=name, M=M, E=E, K=K, I=I, top_k=top_k, block_m=c["block_m"],
                pow2=c["pow2"], x=x, topk_ids=ids.to(ids_dtype).contiguous(),
                topk_weights=w, w13=w13, w13_s=w13_s, w2=w2, w2_s=w2_s,
                meta=dict(seed=seed, routing=c["routing"], fmt=fmt))


def flops(case, n_valid_routes=None):
    """Algorithmic FLOPs of the three GEMM-bearing steps: 2 * R_valid * 3 * K * I."""
    if n_valid_routes is None:
        ids = case.topk_ids
        n_valid_routes = int(((ids >= 0) & (ids < case.E)).sum())
    return 2.0 * n_valid_routes * 3.0 * case.K * case.I
