"""GPU parity: the HIP path (through the C ABI binding) against the CPU oracle
on the same seeded inputs.

Plan and activation codes/scales must be bit-exact; intermediate FP8 codes
may differ in at most 1e-4 of valid-row codes and only by one value step;
outputs must reach relative L2 <= 5e-3 and max abs <= 2e-2 * rms (tests/
parity.py states the bars).  Small cases run the oracle on every token; the
full-size workloads (the configuration bench.py times included) compare
sampled tokens, which the oracle evaluates one route at a time.
"""

import numpy as np
import pytest
import torch

import fp8_block_scale_amd as moe
from moe_workloads import make_case, CONFIGS, SKEW_ZERO_SCALE_EXPERT
from oracle import e4m3_encode, experts_ref, plan_ref, quant_act_ref, FLT_MIN
from oracle.quant import SCALE_FP32, SCALE_UE8M0

from parity import (CODE_MISMATCH_MAX, check_plan, check_tail_untouched, compare_intermediate,
                    compare_output, host_inputs, log, run_gpu, run_oracle)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()


_WEIGHTS = {}


def case_of(name, M=None, ids_dtype=torch.int32, **override):
    """Workloads generated on the GPU; weights cached per geometry.  Keyword
    overrides of the workload's config that keep E, K and I (block_m, seed
    of the routing) reuse its weights."""
    c = dict(CONFIGS[name], **override)
    key = (name, c["E"], c["K"], c["I"], c["pow2"])
    w = _WEIGHTS.get(key)
    cs = make_case(name, M=M, device=DEV, ids_dtype=ids_dtype, weights=w,
                   config=c if override else None)
    _WEIGHTS[key] = (cs.w13, cs.w13_s, cs.w2, cs.w2_s)
    return cs


def inter_mode_of(flags):
    return SCALE_UE8M0 if flags & moe.MOE_F_INTER_UE8M0 else SCALE_FP32


def full_parity(cs, flags=0, act_mode=SCALE_FP32, out_init=None, tokens=None, label=""):
    log(f"[parity] {label} {cs.name} M={cs.M} E={cs.E} K={cs.K} I={cs.I} top_k={cs.top_k} "
        f"bm={cs.block_m} flags={flags:#x} tokens={'all' if tokens is None else len(tokens)}")
    g = run_gpu(cs, out_init=out_init, flags=flags, act_mode=act_mode)
    h = host_inputs(cs)
    o = run_oracle(cs, h=h, out_init=out_init, act_mode=act_mode, inter_mode=inter_mode_of(flags),
                   tokens=tokens)
    check_plan(g, o)
    check_tail_untouched(g, o, cs.block_m)
    assert np.array_equal(g.x_q, o.x_q), "activation codes differ"
    assert np.array_equal(g.x_s, o.x_s), "activation scales differ"
    rows = o.res.row_valid.copy()
    if tokens is not None:
        t_of_row = np.where(rows, o.sorted[:o.P] // cs.top_k, -1)
        rows &= np.isin(t_of_row, np.asarray(tokens))
    ic = compare_intermediate(g.h_q[:o.P], g.h_s[:o.P], o.res.h_q, o.res.h_s, rows)
    trows = np.nonzero(o.res.computed_tokens)[0]
    oc = compare_output(g.out[trows], o.res.ref64[trows])
    log(f"[parity]   ok: P={o.P} inter={ic} out={oc} oracle_s={o.seconds:.2f}")
    return g, o, ic


# ------------------------------------------------------------ primitives

def test_device_e4m3_encoder_matches_oracle():
    # every sign/exponent/top-11-mantissa pattern with rounding-relevant low bits
    hi = np.arange(1 << 20, dtype=np.uint64) << np.uint64(12)
    lows = np.array([0, 1, 0x7FF, 0x800, 0x801, 0xFFF], dtype=np.uint64)
    bits = (hi[:, None] | lows[None, :]).reshape(-1).astype(np.uint32)
    rng = np.random.default_rng(0)
    bits = np.concatenate([bits, rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32)])
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    log(f"[e4m3] {v.size} values")
    inp = torch.from_numpy(v).to(DEV)
    out = torch.empty(v.size, dtype=torch.uint8, device=DEV)
    moe.moe_debug_e4m3_encode(inp, out)
    got = out.cpu().numpy()
    want = e4m3_encode(v)
    bad = got != want
    assert not bad.any(), f"{bad.sum()} mismatches, e.g. {v[bad][:5]} -> {got[bad][:5]} vs {want[bad][:5]}"


# ------------------------------------------------------------------ plan

PLAN_CASES = [
    ("tiny", None, torch.int32), ("tiny", None, torch.int64), ("decode", None, torch.int32),
    ("decode", 16, torch.int64), ("page1", 1024, torch.int32), ("page1", 4096, torch.int32),
    ("page1", 8192, torch.int64), ("skew", None, torch.int32), ("skew", None, torch.int64),
    ("zipf", None, torch.int32),
]


def _plan_ws(M, top_k, E, bm, multi):
    """The multi-workgroup build's workspace, or None for the one-workgroup kernel."""
    n = moe.moe_plan_workspace_size(M, top_k, E, bm) if multi else 0
    return torch.empty(n, dtype=torch.uint8, device=DEV) if n else None


@pytest.mark.parametrize("multi", [False, True])
@pytest.mark.parametrize("name,M,dt", PLAN_CASES)
def test_plan_bit_exact(name, M, dt, multi):
    c = CONFIGS[name]
    M = M or c["M"]
    from moe_workloads import make_routing
    ids, _ = make_routing(c["routing"], M, c["E"], c["top_k"], c["seed"], DEV)
    ids = ids.to(dt).contiguous()
    log(f"[plan] {name} M={M} {dt} multi={multi}")
    sc, bc = moe.moe_plan_capacity(M, c["top_k"], c["E"], c["block_m"])
    s = torch.full((sc,), 0x7F7F7F7F, dtype=torch.int32, device=DEV)
    x = torch.full((bc,), 0x7F7F7F7F, dtype=torch.int32, device=DEV)
    p = torch.empty(1, dtype=torch.int32, device=DEV)
    moe.moe_plan(ids, c["E"], c["block_m"], s, x, p,
                 _plan_ws(M, c["top_k"], c["E"], c["block_m"], multi))
    torch.cuda.synchronize()
    rs, rx, rP = plan_ref(ids.cpu().numpy(), c["E"], c["block_m"])
    P = int(p.item())
    assert P == rP
    s, x = s.cpu().numpy(), x.cpu().numpy()
    assert np.array_equal(s[:P], rs) and np.array_equal(x[:P // c["block_m"]], rx)
    assert np.all(s[P:] == 0x7F7F7F7F) and np.all(x[P // c["block_m"]:] == 0x7F7F7F7F)


@pytest.mark.parametrize("multi", [False, True])
@pytest.mark.parametrize("M,top_k,E,bm", [(1, 1, 1, 16), (3, 5, 7, 16), (1000, 3, 1, 128),
                                          (777, 7, 1024, 32), (5000, 13, 64, 64), (64, 1, 3, 256),
                                          (4096, 1, 257, 16), (100000, 2, 3, 128),
                                          (4099, 8, 1024, 16), (4100, 1, 5, 16), (2051, 2, 300, 32)])
def test_plan_edge_shapes(M, top_k, E, bm, multi):
    """Ragged and extreme shapes; 4100 and 4102 routes give the multi-group
    build 16 groups of 512 routes, the last seven of them empty."""
    g = torch.Generator(device=DEV)
    g.manual_seed(M * 31 + E)
    ids = torch.randint(-2, E + 2, (M, top_k), generator=g, device=DEV, dtype=torch.int32)
    sc, bc = moe.moe_plan_capacity(M, top_k, E, bm)
    s = torch.full((sc,), -7, dtype=torch.int32, device=DEV)
    x = torch.full((bc,), -7, dtype=torch.int32, device=DEV)
    p = torch.empty(1, dtype=torch.int32, device=DEV)
    log(f"[plan edge] M={M} top_k={top_k} E={E} bm={bm} multi={multi}")
    moe.moe_plan(ids, E, bm, s, x, p, _plan_ws(M, top_k, E, bm, multi))
    torch.cuda.synchronize()
    rs, rx, rP = plan_ref(ids.cpu().numpy(), E, bm)
    P = int(p.item())
    assert P == rP and np.array_equal(s.cpu().numpy()[:P], rs)
    assert np.array_equal(x.cpu().numpy()[:P // bm], rx)


def test_plan_all_masked_and_empty():
    ids = torch.full((10, 4), -1, dtype=torch.int64, device=DEV)
    sc, bc = moe.moe_plan_capacity(10, 4, 8, 16)
    s = torch.empty(sc, dtype=torch.int32, device=DEV)
    x = torch.empty(bc, dtype=torch.int32, device=DEV)
    p = torch.full((1,), 99, dtype=torch.int32, device=DEV)
    moe.moe_plan(ids, 8, 16, s, x, p)
    torch.cuda.synchronize()
    assert int(p.item()) == 0
    ids0 = torch.empty((0, 4), dtype=torch.int32, device=DEV)
    p.fill_(99)
    moe.moe_plan(ids0, 8, 16, s, x, p)
    torch.cuda.synchronize()
    assert int(p.item()) == 0


# ----------------------------------------------------------------- quant

@pytest.mark.parametrize("mode", [SCALE_FP32, SCALE_UE8M0])
@pytest.mark.parametrize("M,K,ld", [(1, 7168, 7168), (37, 256, 256), (300, 4096, 4104), (2048, 2048, 2048)])
def test_quant_bit_exact(mode, M, K, ld):
    g = torch.Generator(device=DEV)
    g.manual_seed(M + K)
    base = torch.randn((M, ld), generator=g, device=DEV) * torch.exp(
        torch.randn((M, 1), generator=g, device=DEV) * 3)
    x = base.to(torch.bfloat16)
    if M > 3:
        x[0, :128] = 0.0                                    # all-zero group
        x[1, :128] = 1e-40                                  # subnormal group
        x[2, 128:256] = torch.tensor(3.0e38).to(torch.bfloat16)  # huge values
        x[3, :] = -x[3, :]
    xv = x[:, :K]
    log(f"[quant] M={M} K={K} ld={ld} mode={mode}")
    xq = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    xs = torch.empty((M, K // 128), dtype=torch.float32, device=DEV)
    moe.moe_quant_act(xv, xq, xs, mode)
    torch.cuda.synchronize()
    rq, rs = quant_act_ref(xv.float().cpu().numpy(), mode)
    assert np.array_equal(xs.cpu().numpy(), rs)
    assert np.array_equal(xq.cpu().numpy(), rq)


@pytest.mark.parametrize("multi", [False, True])
@pytest.mark.parametrize("name,M,dt,mode,pad", [
    ("tiny", None, torch.int32, SCALE_FP32, 0), ("decode", None, torch.int64, SCALE_FP32, 0),
    ("decode", 16, torch.int32, SCALE_UE8M0, 64), ("page1", 4096, torch.int32, SCALE_FP32, 0),
    ("zipf", 1024, torch.int64, SCALE_UE8M0, 8), ("skew", 333, torch.int32, SCALE_FP32, 0)])
def test_plan_quant_matches_separate_calls(name, M, dt, mode, pad, multi):
    """moe_plan_quant (one launch fewer) writes exactly what moe_plan then
    moe_quant_act write: the whole plan buffers and the codes and scales."""
    c = CONFIGS[name]
    M = M or c["M"]
    E, k, bm, K = c["E"], c["top_k"], c["block_m"], c["K"]
    from moe_workloads import make_routing
    ids, _ = make_routing(c["routing"], M, E, k, c["seed"], DEV)
    ids = ids.to(dt).contiguous()
    g = torch.Generator(device=DEV)
    g.manual_seed(M + K)
    x = torch.randn((M, K + pad), generator=g, device=DEV).to(torch.bfloat16)[:, :K]
    log(f"[plan_quant] {name} M={M} {dt} mode={mode} ld={K + pad} multi={multi}")
    sc, bc = moe.moe_plan_capacity(M, k, E, bm)
    outs = []
    for fused in (False, True):
        s = torch.full((sc,), 0x7F7F7F7F, dtype=torch.int32, device=DEV)
        e = torch.full((bc,), 0x7F7F7F7F, dtype=torch.int32, device=DEV)
        p = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        q = torch.full((M, K), 0x5A, dtype=torch.uint8, device=DEV)
        qs = torch.full((M, K // 128), -1.0, dtype=torch.float32, device=DEV)
        ws = _plan_ws(M, k, E, bm, multi)
        if fused:
            moe.moe_plan_quant(ids, E, bm, s, e, p, x, q, qs, mode, ws)
        else:
            moe.moe_plan(ids, E, bm, s, e, p, ws)
            moe.moe_quant_act(x, q, qs, mode)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (s, e, p, q, qs)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    rq, rs = quant_act_ref(x.float().cpu().numpy(), mode)      # and both are the oracle's
    assert np.array_equal(outs[1][3].numpy(), rq) and np.array_equal(outs[1][4].numpy(), rs)


# --------------------------------------------------------- whole path

def test_tiny_full():
    full_parity(case_of("tiny"), label="auto-split")


def test_tiny_no_split():
    full_parity(case_of("tiny"), flags=1 << moe.MOE_F_SPLITK_SHIFT, label="split=1")


def test_tiny_accumulates_into_prefilled_output():
    cs = case_of("tiny")
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    init = (torch.randn((cs.M, cs.K), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    full_parity(cs, out_init=init, label="prefilled out")


FUSE_ON = moe.MOE_FUSE_ON << moe.MOE_F_FUSE_SHIFT
FUSE_OFF = moe.MOE_FUSE_OFF << moe.MOE_F_FUSE_SHIFT


@pytest.mark.parametrize("flags", [0, 1 << moe.MOE_F_SPLITK_SHIFT, 7 << moe.MOE_F_SPLITK_SHIFT,
                                   FUSE_OFF, FUSE_OFF | (7 << moe.MOE_F_SPLITK_SHIFT)])
def test_decode_full(flags):
    full_parity(case_of("decode"), flags=flags, label="decode")


@pytest.mark.parametrize("M", [2, 4, 8, 16])
def test_decode_sweep_full(M):
    full_parity(case_of("decode", M=M), label="decode sweep")


def test_page1_small_full():
    full_parity(case_of("page1", M=24), label="page1 small")


def test_skew_small_full():
    full_parity(case_of("skew", M=48), label="skew small")


E8 = moe.MOE_F_INTER_UE8M0 | moe.MOE_F_MMA_E8M0


@pytest.mark.parametrize("flags", [moe.MOE_F_INTER_UE8M0, E8])
def test_zipf_small_full(flags):
    full_parity(case_of("zipf", M=40), flags=flags, act_mode=SCALE_UE8M0, label="zipf small")


@pytest.mark.parametrize("bm", [8, 64, 128])
def test_small_grid_long_intermediate_rows(bm):
    """Small grid with I = 2048: the down stage's rows (16 K-blocks) are too
    long for the stream kernel's LDS tile, so its fallback kernel runs."""
    cfg = dict(CONFIGS["tiny"], M=24, E=8, K=512, I=2048, top_k=2, block_m=bm, seed=7)
    cs = make_case("long_rows", device=DEV, config=cfg)
    full_parity(cs, label="small grid, long intermediate rows")


PERSIST = ((moe.MOE_PATH_PERSISTENT << moe.MOE_F_GATEUP_PATH_SHIFT)
           | (moe.MOE_PATH_PERSISTENT << moe.MOE_F_DOWN_PATH_SHIFT))


@pytest.mark.parametrize("name,M,flags", [("tiny", None, 0), ("decode", None, 0),
                                          ("decode", 16, FUSE_ON), ("page1", 512, 0),
                                          ("page1", 512, PERSIST)])
def test_graph_replay_matches_eager(name, M, flags):
    """The whole layer captured in a HIP graph (the column-slice gate/up and
    the column-split down for tiny, the split-K gate/up and the column-split
    down for decode, steps 3-5 as one launch at decode M=16; at M=512 the
    per-block gate/up with the persistent down, then both persistent
    kernels): every replay, with eager work and synchronisations between
    replays, gives the eager output bit for bit."""
    cs = case_of(name, M=M)
    log(f"[graph] {name} M={cs.M} flags={flags:#x}")
    b = moe.MoeLayerBuffers(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, flags, DEV)
    args = (cs.x, cs.topk_ids, cs.topk_weights, cs.w13, cs.w13_s, cs.w2, cs.w2_s)
    ref = torch.zeros((cs.M, cs.K), dtype=torch.bfloat16, device=DEV)
    moe.moe_layer(b, *args, ref, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    out = torch.zeros_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer(b, *args, out, stream=torch.cuda.current_stream())
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager layer"
        # eager work between replays: the layer itself into a scratch output
        scratch = torch.zeros_like(ref)
        moe.moe_layer(b, *args, scratch, stream=torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(scratch, ref)


@pytest.mark.parametrize("bm", [16, 32])
def test_persistent_kernels_small_block_m(bm):
    """The persistent gate/up and down kernels with block_m 16 and 32: row
    tiles of 8 and 4 plan blocks."""
    cs = case_of("page1", M=512, block_m=bm)
    full_parity(cs, flags=PERSIST, tokens=_sample_tokens(cs.M, 12, 20 + bm),
                label=f"persistent bm={bm}")


def test_persistent_long_k_wide_i():
    """Persistent path at K=7168 (56 K-blocks per item) and I=2048 (16
    128-deep steps per down item, 16 j-tiles), E=32, top-8."""
    cfg = dict(CONFIGS["page1"], M=256, E=32, K=7168, I=2048, top_k=8, block_m=64, seed=11)
    cs = make_case("long_k", device=DEV, config=cfg)
    full_parity(cs, flags=PERSIST, tokens=_sample_tokens(cs.M, 6, 21),
                label="persistent K=7168 I=2048")


@pytest.mark.parametrize("K", [128, 640, 768, 896])
def test_persistent_ragged_scale_groups(K):
    """The persistent gate/up loads activation scales four K-blocks at a time
    into two alternating slots: K = 128 / 640 / 768 / 896 gives 1 / 5 / 6 / 7
    K-blocks, so the last group is short (1-3 K-blocks, its loads clamped to
    the last K-block) or the only one."""
    cfg = dict(CONFIGS["page1"], M=192, E=16, K=K, I=512, top_k=4, block_m=32, seed=17)
    cs = make_case("ragged_k", device=DEV, config=cfg)
    full_parity(cs, flags=PERSIST, tokens=_sample_tokens(cs.M, 8, 50 + K // 128),
                label=f"persistent K={K}")


@pytest.mark.parametrize("flags", [0, PERSIST])
def test_max_k(flags):
    """K = 32768, the largest hidden size the persistent kernels accept
    (256 K-blocks of weight-block scales per column tile), on both kernel
    families: E=4, I=256, top-2, M=64."""
    cfg = dict(CONFIGS["tiny"], M=64, E=4, K=32768, I=256, top_k=2, block_m=16, seed=19)
    cs = make_case("max_k", device=DEV, config=cfg)
    full_parity(cs, flags=flags, tokens=_sample_tokens(cs.M, 6, 60 + flags % 7),
                label=f"K=32768 flags={flags:#x}")


@pytest.mark.parametrize("flags", [0, PERSIST])
def test_max_i_single_k_block(flags):
    """I = 32768, the largest intermediate size the persistent kernels accept
    (256 column tiles per row tile; 256 128-deep steps per down item), with
    K = 128 (one K-block): E=2, top-1, M=32."""
    cfg = dict(CONFIGS["tiny"], M=32, E=2, K=128, I=32768, top_k=1, block_m=16, seed=23)
    cs = make_case("max_i", device=DEV, config=cfg)
    full_parity(cs, flags=flags, tokens=_sample_tokens(cs.M, 4, 70 + flags % 5),
                label=f"I=32768 K=128 flags={flags:#x}")


@pytest.mark.parametrize("flags", [0, PERSIST])
def test_max_experts(flags):
    """E = 1024, the largest expert count the ABI accepts, on both kernel
    families: top-8, M=128, K=I=256."""
    cfg = dict(CONFIGS["tiny"], M=128, E=1024, K=256, I=256, top_k=8, block_m=16, seed=29)
    cs = make_case("max_e", device=DEV, config=cfg)
    full_parity(cs, flags=flags, label=f"E=1024 flags={flags:#x}")


@pytest.mark.parametrize("gu,dn", [(1, 1), (1, 2), (2, 1), (2, 2)])
def test_kernel_path_combinations(gu, dn):
    """Every pairing of the per-block (1) and persistent (2) kernel families
    of the two stages, as two launches, on one input: the down stage's row
    tiles come from the gate/up stage whichever kernel it runs."""
    cs = case_of("page1", M=256)
    flags = ((gu << moe.MOE_F_GATEUP_PATH_SHIFT) | (dn << moe.MOE_F_DOWN_PATH_SHIFT)
             | (moe.MOE_FUSE_OFF << moe.MOE_F_FUSE_SHIFT))
    cap = moe.moe_plan_capacity(cs.M, cs.top_k, cs.E, cs.block_m)[0]
    sched = moe.moe_fp8_experts_schedule(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, cap, flags)
    assert sched[0] == (gu == 2) and sched[1] == (dn == 2)
    full_parity(cs, flags=flags, tokens=_sample_tokens(cs.M, 8, 30 + 3 * gu + dn),
                label=f"paths gate/up {gu} down {dn}")


def test_debug_count_non_pow2():
    """The E8M0 precondition check against a count from the raw bits."""
    def expect(t):
        b = t.cpu().contiguous().view(torch.int32).numpy().astype(np.uint32)
        ex = (b >> 23) & 0xFF
        return int((((b & 0x807FFFFF) != 0) | (ex == 0) | (ex == 0xFF)).sum())
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    z = case_of("zipf", M=64)
    p = case_of("page1", M=64)
    odd = torch.tensor([1.0, 0.5, 2.0 ** -126, 2.0 ** 127, 0.0, -1.0, 3.0, float("inf"), float("nan"),
                        2.0 ** -127, 1.5 * 2 ** 60], dtype=torch.float32, device=DEV)
    for t, label in ((z.w13_s, "zipf w13_s"), (z.w2_s, "zipf w2_s"), (p.w13_s, "page1 w13_s"),
                     (odd, "edge values")):
        flat = t.reshape(-1).contiguous()
        moe.moe_debug_count_non_pow2(flat, cnt)
        torch.cuda.synchronize()
        assert int(cnt.item()) == expect(flat), label
    assert expect(z.w13_s.reshape(-1)) == 0 and expect(odd) == 7


def _sample_tokens(M, n, seed, extra=()):
    rng = np.random.default_rng(seed)
    t = set(rng.choice(M, size=min(n, M), replace=False).tolist()) | set(extra)
    t |= {0, M - 1}
    return sorted(t)



def _cover_tokens(cs, n, seed, extra=()):
    """n random tokens (plus `extra`, the first and the last), then, greedily,
    the token that routes to the most experts no chosen token reaches yet,
    until every expert the batch touches feeds at least one compared row --
    so every touched expert's W13/W2 tiles and block scales are checked."""
    ids = cs.topk_ids.cpu().numpy()
    valid = (ids >= 0) & (ids < cs.E)
    t = set(_sample_tokens(cs.M, n, seed, extra))
    covered = np.zeros(cs.E, dtype=bool)
    for tok in t:
        covered[ids[tok][valid[tok]]] = True
    touched = np.zeros(cs.E, dtype=bool)
    touched[ids[valid]] = True
    onehot = np.zeros((cs.M, cs.E), dtype=bool)
    rr, cc = np.nonzero(valid)
    onehot[rr, ids[rr, cc]] = True
    while (touched & ~covered).any():
        gain = onehot[:, ~covered].sum(1)
        best = int(np.argmax(gain))
        assert gain[best] > 0
        t.add(best)
        covered |= onehot[best]
    return sorted(t)


def test_page1_full_size_sampled():
    """The configuration bench.py times (E=288, K=4096, I=1024, top-8, M=4096);
    the sampled tokens reach every expert."""
    cs = case_of("page1")
    full_parity(cs, tokens=_cover_tokens(cs, 8, 1), label="page1 full size")


@pytest.mark.parametrize("M", [1024, 2048, 8192])
def test_page1_sweep_sampled(M):
    cs = case_of("page1", M=M)
    full_parity(cs, tokens=_cover_tokens(cs, 6, M), label="page1 sweep")


@pytest.mark.parametrize("dt", [torch.int32, torch.int64])
def test_skew_full_size_sampled(dt):
    cs = case_of("skew", ids_dtype=dt)
    ids = cs.topk_ids.cpu().numpy()
    masked_tok = int(np.nonzero((ids < 0).any(1))[0][0])
    zero_tok = int(np.nonzero((ids == SKEW_ZERO_SCALE_EXPERT).any(1))[0][0])
    full_parity(cs, tokens=_cover_tokens(cs, 8, 3, extra=(masked_tok, zero_tok)),
                label=f"skew full size {dt}")


@pytest.mark.parametrize("flags", [moe.MOE_F_INTER_UE8M0, E8])
def test_zipf_full_size_sampled(flags):
    cs = case_of("zipf")
    full_parity(cs, flags=flags, act_mode=SCALE_UE8M0, tokens=_cover_tokens(cs, 6, 4),
                label="zipf full size")


# ------------------------------------------------------------ block_m = 8
# Plan blocks of 8 rows: the per-block kernels run a 16-row MFMA tile whose
# last 8 rows are masked (they belong to the next block and are never read),
# the persistent kernels cut 16 blocks per 128-row tile.

# The persistent down stage behind the per-block gate/up works on row tiles of
# at most 32 rows (a deeper W2 ring); experts with many blocks span several
# such tiles (skew's hot experts, page-1 at M=256), masked routes and the
# zero-scale expert included; power-of-two scales through the E8M0 MFMA.
@pytest.mark.parametrize("name,M,bm,flags", [
    ("page1", 256, 16, 0), ("page1", 256, 32, 0), ("skew", 512, 32, 0),
    ("zipf", 256, 32, E8), ("decode", 16, 8, 0)])
def test_small_tile_down(name, M, bm, flags):
    cs = case_of(name, M=M, block_m=bm)
    fl = (flags | (moe.MOE_PATH_STREAM << moe.MOE_F_GATEUP_PATH_SHIFT)
          | (moe.MOE_PATH_PERSISTENT << moe.MOE_F_DOWN_PATH_SHIFT) | FUSE_OFF)
    act = SCALE_UE8M0 if flags & moe.MOE_F_INTER_UE8M0 else SCALE_FP32
    tokens = None if cs.M <= 16 else _cover_tokens(cs, 6, 60 + bm)
    full_parity(cs, flags=fl, act_mode=act, tokens=tokens, label=f"small-tile down bm={bm}")

@pytest.mark.parametrize("name,M,flags", [
    ("tiny", None, 0), ("decode", None, 0), ("decode", 4, 0), ("decode", 16, 0),
    ("decode", 16, 7 << moe.MOE_F_SPLITK_SHIFT), ("decode", 16, FUSE_ON),
    ("skew", 64, 0), ("skew", 64, FUSE_ON)])
def test_block_m_8(name, M, flags):
    full_parity(case_of(name, M=M, block_m=8), flags=flags, label="block_m=8")


@pytest.mark.parametrize("gu,dn", [(1, 1), (2, 2), (1, 2)])
def test_block_m_8_kernel_families(gu, dn):
    cs = case_of("page1", M=256, block_m=8)
    flags = ((gu << moe.MOE_F_GATEUP_PATH_SHIFT) | (dn << moe.MOE_F_DOWN_PATH_SHIFT) | FUSE_OFF)
    full_parity(cs, flags=flags, tokens=_cover_tokens(cs, 6, 80 + gu + dn),
                label=f"block_m=8 paths {gu}/{dn}")


# The down stage split over output columns with the route sum in the same
# launch (the default while every route's intermediate row fits in LDS:
# I = 256, block_m 8 or 16, at most 192 routes).  Forced on: the tiny and
# decode workloads at both block sizes up to 189 routes, power-of-two scales
# through the E8M0 MFMA, and a skew-like batch (hot experts with many
# blocks, duplicate experts within a token, 1% masked routes, a zero-scale
# expert) at I = 256.
COLS = (moe.MOE_PATH_COLUMNS << moe.MOE_F_DOWN_PATH_SHIFT) | FUSE_OFF


@pytest.mark.parametrize("name,M,bm", [("tiny", None, 16), ("tiny", None, 8), ("decode", 1, 16),
                                       ("decode", 2, 8), ("decode", 21, 8), ("decode", 12, 16)])
def test_column_down(name, M, bm):
    cs = case_of(name, M=M, block_m=bm)
    cap = moe.moe_plan_capacity(cs.M, cs.top_k, cs.E, cs.block_m)[0]
    assert moe.moe_fp8_experts_schedule(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, cap, COLS)[1] == 2
    full_parity(cs, flags=COLS, label=f"column down bm={bm}")


def test_column_down_e8m0():
    cfg = dict(CONFIGS["zipf"], M=24, E=16, K=1024, I=256, top_k=6, block_m=16, seed=43)
    cs = make_case("zipf-i256", device=DEV, config=cfg)
    full_parity(cs, flags=COLS | E8, act_mode=SCALE_UE8M0, label="column down e8m0")


@pytest.mark.parametrize("dt", [torch.int32, torch.int64])
def test_column_down_skew(dt):
    cfg = dict(CONFIGS["skew"], M=18, I=256, block_m=16, seed=44)
    cs = make_case("skew-i256", device=DEV, config=cfg, ids_dtype=dt)
    full_parity(cs, flags=COLS, label=f"column down skew {dt}")


# The gate/up split over 16-column slices of the intermediate (K split over
# the eight waves of a workgroup, FP32 SwiGLU rows out, no split-K counters
# and no clearing launch), whose rows the column-split down requantises as it
# loads them.  Same cases as above; the intermediate codes compared are the
# ones the down stage writes back.
SLICES = (moe.MOE_PATH_COLUMNS << moe.MOE_F_GATEUP_PATH_SHIFT) | COLS


@pytest.mark.parametrize("name,M,bm", [("tiny", None, 16), ("tiny", None, 8), ("decode", 1, 16),
                                       ("decode", 2, 8), ("decode", 4, 16), ("decode", 21, 8),
                                       ("decode", 12, 16)])
def test_column_gateup(name, M, bm):
    cs = case_of(name, M=M, block_m=bm)
    cap = moe.moe_plan_capacity(cs.M, cs.top_k, cs.E, cs.block_m)[0]
    assert moe.moe_fp8_experts_schedule(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, cap,
                                        SLICES)[:3] == (2, 2, 1)
    full_parity(cs, flags=SLICES, label=f"column gate/up bm={bm}")


def test_column_gateup_scales():
    """Power-of-two intermediate scales (the requantisation's other rule),
    then with them inside the down stage's MFMA."""
    cs = case_of("decode", M=3, block_m=16)
    full_parity(cs, flags=SLICES | moe.MOE_F_INTER_UE8M0, label="column gate/up ue8m0 rule")
    cfg = dict(CONFIGS["zipf"], M=24, E=16, K=1024, I=256, top_k=6, block_m=16, seed=45)
    cz = make_case("zipf-i256", device=DEV, config=cfg)
    full_parity(cz, flags=SLICES | E8, act_mode=SCALE_UE8M0, label="column gate/up e8m0")


@pytest.mark.parametrize("dt", [torch.int32, torch.int64])
def test_column_gateup_skew(dt):
    cfg = dict(CONFIGS["skew"], M=18, I=256, block_m=16, seed=46)
    cs = make_case("skew-i256", device=DEV, config=cfg, ids_dtype=dt)
    full_parity(cs, flags=SLICES, label=f"column gate/up skew {dt}")


def test_column_gateup_matches_stream():
    """Against the per-block gate/up on the same plan: the intermediate
    codes agree to the same bar as against the oracle (only the FP32
    summation order differs), and so do the outputs."""
    cs = case_of("decode", M=8, block_m=16)
    a = run_gpu(cs, flags=SLICES)
    b = run_gpu(cs, flags=COLS | (moe.MOE_PATH_STREAM << moe.MOE_F_GATEUP_PATH_SHIFT))
    assert a.P == b.P and np.array_equal(a.sorted[:a.P], b.sorted[:b.P])
    s = a.sorted[:a.P]
    rows = (s >= 0) & (s < cs.M * cs.top_k)
    compare_intermediate(a.h_q[:a.P], a.h_s[:a.P], b.h_q[:b.P], b.h_s[:b.P], rows)
    compare_output(a.out, b.out)


@pytest.mark.parametrize("flags", [
    SLICES, COLS | (moe.MOE_PATH_STREAM << moe.MOE_F_GATEUP_PATH_SHIFT),
    (moe.MOE_PATH_STREAM << moe.MOE_F_GATEUP_PATH_SHIFT) | (moe.MOE_PATH_STREAM << moe.MOE_F_DOWN_PATH_SHIFT),
    (moe.MOE_PATH_PERSISTENT << moe.MOE_F_GATEUP_PATH_SHIFT)
    | (moe.MOE_PATH_PERSISTENT << moe.MOE_F_DOWN_PATH_SHIFT)])
def test_block_with_out_of_range_expert_adds_nothing(flags):
    """A plan block whose expert id is out of range (a caller's plan, not
    one moe_plan builds) is skipped by every kernel family: its routes add
    nothing, the rest of the layer is as the oracle computes it with those
    routes masked."""
    cs = case_of("tiny")
    h = host_inputs(cs)
    sorted_ref, eids_ref, P = plan_ref(h["ids"], cs.E, cs.block_m)
    bad = 1                                              # a block that holds routes
    R = cs.M * cs.top_k
    assert P >= 2 * cs.block_m and np.any(sorted_ref[bad * cs.block_m:(bad + 1) * cs.block_m] < R)
    b = moe.MoeLayerBuffers(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, flags, DEV)
    b.workspace.fill_(0x5A)
    moe.moe_plan(cs.topk_ids, cs.E, cs.block_m, b.sorted_ids, b.expert_ids, b.ntp, b.plan_ws)
    moe.moe_quant_act(cs.x, b.x_q, b.x_s, SCALE_FP32)
    b.expert_ids[bad] = cs.E
    out = torch.zeros((cs.M, cs.K), dtype=torch.bfloat16, device=DEV)
    moe.moe_fp8_experts(b.x_q, b.x_s, cs.w13, cs.w13_s, cs.w2, cs.w2_s, cs.topk_weights,
                        b.sorted_ids, b.expert_ids, b.ntp, cs.top_k, cs.block_m, out, b.workspace,
                        flags)
    torch.cuda.synchronize()
    masked = sorted_ref.copy()
    masked[bad * cs.block_m:(bad + 1) * cs.block_m] = R
    x_q, x_s = quant_act_ref(h["x"], SCALE_FP32)
    res = experts_ref(x_q, x_s, h["w13"], h["w13_s"], h["w2"], h["w2_s"], h["w"], masked, eids_ref,
                      P, cs.top_k, cs.block_m)
    compare_output(out.float().cpu().numpy().astype(np.float64), res.ref64)


# ------------------------------------------------- steps 3-5 in one launch
# MOE_FUSE_ON: one launch runs the per-block gate/up items, the down items
# (which wait for their block's intermediate rows) and the route sum (by the
# item completing a (token, tile)).  Parity against the oracle on all five
# workloads, and the output bit-identical to the two-launch path.

@pytest.mark.parametrize("name,M,flags,cover", [
    ("tiny", None, 0, False), ("decode", None, 0, False), ("decode", 2, 0, False),
    ("decode", 16, 7 << moe.MOE_F_SPLITK_SHIFT, False), ("page1", 24, 0, False),
    ("page1", None, 0, True), ("skew", None, 0, True),
    ("zipf", None, moe.MOE_F_INTER_UE8M0, True), ("zipf", None, E8, True)])
def test_single_launch(name, M, flags, cover):
    cs = case_of(name, M=M)
    act = SCALE_UE8M0 if flags & moe.MOE_F_INTER_UE8M0 else SCALE_FP32
    cap = moe.moe_plan_capacity(cs.M, cs.top_k, cs.E, cs.block_m)[0]
    assert moe.moe_fp8_experts_schedule(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, cap,
                                        flags | FUSE_ON)[4]
    tokens = _cover_tokens(cs, 6, 40) if cover else None
    g, o, _ = full_parity(cs, flags=flags | FUSE_ON, act_mode=act, tokens=tokens,
                          label="single launch")
    # the two launches on the per-block down kernel: the single launch runs its
    # work item and its route sum (the column-split down, the default at
    # decode sizes, adds FP32 route terms instead of the FP16 route rows)
    two = run_gpu(cs, flags=flags | FUSE_OFF | (moe.MOE_PATH_STREAM << moe.MOE_F_DOWN_PATH_SHIFT),
                  act_mode=act)
    assert np.array_equal(g.out, two.out), "single launch differs from the two launches"
    rows = o.res.row_valid if tokens is None else (two.sorted[:two.P] < cs.M * cs.top_k)
    assert np.array_equal(g.h_q[:g.P][rows], two.h_q[:two.P][rows])


def test_single_launch_repeat_and_masked():
    """Bit-identical repeat runs of the single launch on the skew workload
    (masked routes, duplicate experts in a token, a zero-scale expert), and
    an all-masked batch leaving the output untouched."""
    cs = case_of("skew", M=96)
    a = run_gpu(cs, flags=FUSE_ON)
    b = run_gpu(cs, flags=FUSE_ON)
    assert np.array_equal(a.out, b.out)
    cs.topk_ids = torch.full_like(cs.topk_ids, -1)
    init = torch.randn((cs.M, cs.K), device=DEV).to(torch.bfloat16)
    g = run_gpu(cs, out_init=init, flags=FUSE_ON)
    assert g.P == 0 and np.array_equal(g.out, init.float().cpu().numpy())


# ------------------------------------------------ FP8-MFMA gate/up mode
# MOE_F_FP8_GATEUP is experimental: the FP8 MFMA sums each instruction's
# products in a window about 15 bits below the largest one, so the SwiGLU
# inputs differ from exact sums by ~1e-5 relative and ~1e-3 of the
# requantised codes move -- ten times the 1e-4 code budget.  It is held to
# no bar of its own; this test records the finding, measured with the same
# comparison the exact path must pass.

def test_fp8_mfma_gate_up_exceeds_the_code_budget():
    """Why the default gate/up widens the codes to FP16: on one input
    (page-1 shape, M=1024, 8 sampled tokens = 65536 intermediate codes) the
    FP8-MFMA gate/up, whose hardware adds the products of an instruction in
    a window below the largest one, moves more intermediate codes than the
    1e-4 budget allows; the exact path on the same input stays within it."""
    cs = case_of("page1", M=1024)
    tok = _sample_tokens(cs.M, 8, 5)
    _, _, exact = full_parity(cs, tokens=tok, label="exact gate/up")
    g = run_gpu(cs, flags=moe.MOE_F_FP8_GATEUP)
    o = run_oracle(cs, tokens=tok)
    t_of_row = np.where(o.res.row_valid, o.sorted[:o.P] // cs.top_k, -1)
    rows = o.res.row_valid & np.isin(t_of_row, np.asarray(tok))
    fp8 = compare_intermediate(g.h_q[:o.P], g.h_s[:o.P], o.res.h_q, o.res.h_s, rows,
                               max_frac=1.0, one_step=False)
    log(f"[fp8 gate/up] exact {exact} fp8 {fp8}")
    assert exact["frac"] <= CODE_MISMATCH_MAX < fp8["frac"], (exact, fp8)


# ------------------------------------------------------------ contracts

@pytest.mark.parametrize("flags", [E8, E8 | PERSIST | FUSE_OFF])
def test_e8m0_wide_scale_spread(flags):
    """Power-of-two scales folded into the gate/up widening on activations
    whose 128-column groups differ by up to 2^24 in magnitude within a row,
    so the folded ratios reach deep into the FP16 subnormal range: codes,
    scales and output still meet the bars against the oracle (both kernel
    families)."""
    cfg = dict(CONFIGS["zipf"], M=96, E=16, K=1024, I=256, top_k=4, block_m=32, seed=41)
    cs = make_case("spread", device=DEV, config=cfg)
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    k = torch.randint(-12, 13, (cs.M, cs.K // 128), generator=g, device=DEV).float()
    cs.x = (cs.x.float() * torch.repeat_interleave(torch.exp2(k), 128, dim=1)).to(torch.bfloat16)
    full_parity(cs, flags=flags, act_mode=SCALE_UE8M0, label=f"e8m0 spread {flags:#x}")


def test_e8m0_matches_fp32_scale_kernels():
    """Power-of-two scales: the E8M0-scaled kernels and the FP32-scale
    kernels see identical inputs and must agree to the parity bars."""
    cs = case_of("zipf", M=512)
    fl = moe.MOE_F_INTER_UE8M0
    a = run_gpu(cs, flags=fl, act_mode=SCALE_UE8M0)
    b = run_gpu(cs, flags=fl | moe.MOE_F_MMA_E8M0, act_mode=SCALE_UE8M0)
    assert a.P == b.P and np.array_equal(a.sorted[:a.P], b.sorted[:b.P])
    rows = (a.sorted[:a.P] < cs.M * cs.top_k)
    compare_intermediate(b.h_q[:a.P], b.h_s[:a.P], a.h_q[:a.P], a.h_s[:a.P], rows)
    compare_output(b.out, a.out)


def test_truncated_extent():
    """num_tokens_post_padded = block_m: only the first block is computed and
    every block past it exits untouched."""
    cs = case_of("tiny")
    g = run_gpu(cs, ntp_override=cs.block_m)
    o = run_oracle(cs, P_override=cs.block_m)
    check_plan(g, o)
    bm = cs.block_m
    assert o.res.h_q.shape[0] == bm
    compare_intermediate(g.h_q[:bm], g.h_s[:bm], o.res.h_q, o.res.h_s, o.res.row_valid)
    # rows beyond the truncated extent keep the workspace fill
    assert g.P > bm and np.all(g.h_q[bm:g.P] == 0x5A)
    compare_output(g.out, o.res.ref64)


def test_two_calls_accumulate():
    cs = case_of("decode", M=4)
    b = moe.MoeLayerBuffers(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, 0, DEV)
    out = torch.zeros((cs.M, cs.K), dtype=torch.bfloat16, device=DEV)
    for _ in range(2):
        moe.moe_layer(b, cs.x, cs.topk_ids, cs.topk_weights, cs.w13, cs.w13_s, cs.w2, cs.w2_s, out)
    torch.cuda.synchronize()
    o = run_oracle(cs)
    compare_output(out.float().cpu().numpy(), 2 * o.res.ref64)


def test_all_routes_masked_leaves_output_unchanged():
    cs = case_of("tiny")
    cs.topk_ids = torch.full_like(cs.topk_ids, -1)
    init = torch.randn((cs.M, cs.K), device=DEV).to(torch.bfloat16)
    g = run_gpu(cs, out_init=init)
    assert g.P == 0
    assert np.array_equal(g.out, init.float().cpu().numpy())


def test_zero_scale_expert_contributes_zero():
    cs = case_of("skew", M=64)
    ids = cs.topk_ids.clone()
    g = run_gpu(cs)
    masked = case_of("skew", M=64)
    mids = ids.clone()
    mids[mids == SKEW_ZERO_SCALE_EXPERT] = -1
    masked.topk_ids = mids
    gm = run_gpu(masked)
    compare_output(g.out, gm.out)
    # that expert's rows requantise an all-zero h: codes 0, scale FLT_MIN
    rows = [p for p in range(g.P) if g.expert_ids[p // cs.block_m] == SKEW_ZERO_SCALE_EXPERT
            and g.sorted[p] < cs.M * cs.top_k]
    assert rows
    assert np.all(g.h_q[rows] & 0x7F == 0) and np.all(g.h_s[rows] == FLT_MIN)
    assert np.all(np.isfinite(g.out))


def test_int32_int64_ids_agree():
    a = run_gpu(case_of("skew", M=256, ids_dtype=torch.int32))
    b = run_gpu(case_of("skew", M=256, ids_dtype=torch.int64))
    assert a.P == b.P and np.array_equal(a.sorted, b.sorted)
    assert np.array_equal(a.h_q, b.h_q) and np.array_equal(a.h_s, b.h_s)
    # the route sum is taken in route order: the outputs are bit-identical
    assert np.array_equal(a.out, b.out)


def test_repeat_runs_bit_identical():
    cs = case_of("page1", M=256)
    a = run_gpu(cs)
    b = run_gpu(cs)
    assert np.array_equal(a.sorted, b.sorted) and np.array_equal(a.x_q, b.x_q)
    rows = a.sorted[:a.P] < cs.M * cs.top_k
    assert np.array_equal(a.h_q[:a.P][rows], b.h_q[:b.P][rows])
    assert np.array_equal(a.out, b.out)


def test_m_zero_is_a_no_op():
    b = moe.MoeLayerBuffers(0, 256, 256, 8, 2, 16, 0, DEV)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    w = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    cs = case_of("tiny")
    out = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    moe.moe_layer(b, x, ids, w, cs.w13, cs.w13_s, cs.w2, cs.w2_s, out)
    torch.cuda.synchronize()
    assert int(b.ntp.item()) == 0


# ------------------------------------------------------- all five steps, one call

@pytest.mark.parametrize("name,M,flags", [("decode", 1, 0), ("decode", 4, 0), ("decode", 16, 0),
                                          ("tiny", None, 0), ("page1", 512, 0),
                                          ("decode", 2, moe.MOE_F_INTER_UE8M0)])
def test_layer_call_matches_two_calls(name, M, flags):
    """moe_fp8_layer against moe_plan_quant then moe_fp8_experts on the same
    inputs, workspaces filled with garbage: plan, activation codes, output and
    intermediate codes bit for bit -- at decode sizes the clearing launch is
    folded into the plan's, elsewhere the two calls run as they are."""
    cs = case_of(name, M=M)
    log(f"[layer] {name} M={cs.M} flags={flags:#x}")
    outs = []
    for one_call in (False, True):
        b = moe.MoeLayerBuffers(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, flags, DEV)
        b.workspace.fill_(0x5A)
        b.sorted_ids.fill_(0x7F7F7F7F)
        b.expert_ids.fill_(0x7F7F7F7F)
        out = torch.zeros((cs.M, cs.K), dtype=torch.bfloat16, device=DEV)
        if one_call:
            moe.moe_fp8_layer(cs.x, cs.topk_ids, cs.topk_weights, cs.w13, cs.w13_s, cs.w2, cs.w2_s,
                              cs.block_m, b.sorted_ids, b.expert_ids, b.ntp, b.x_q, b.x_s, out,
                              b.workspace, flags, SCALE_FP32, b.plan_ws)
        else:
            moe.moe_plan_quant(cs.topk_ids, cs.E, cs.block_m, b.sorted_ids, b.expert_ids, b.ntp,
                               cs.x, b.x_q, b.x_s, SCALE_FP32, b.plan_ws)
            moe.moe_fp8_experts(b.x_q, b.x_s, cs.w13, cs.w13_s, cs.w2, cs.w2_s, cs.topk_weights,
                                b.sorted_ids, b.expert_ids, b.ntp, cs.top_k, cs.block_m, out,
                                b.workspace, flags)
        torch.cuda.synchronize()
        hq, hs = b.intermediate()
        P = int(b.ntp.item())
        outs.append((P, b.sorted_ids.clone(), b.expert_ids.clone(), b.x_q.clone(), b.x_s.clone(),
                     out, hq[:P].clone(), hs[:P].clone()))
    (P0, *a), (P1, *c) = outs
    assert P0 == P1
    for u, v, what in zip(a, c, ("sorted", "expert_ids", "x_q", "x_s", "out", "h_q", "h_s")):
        assert torch.equal(u, v), f"{what} differs between the one call and the two"
