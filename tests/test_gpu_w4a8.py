"""GPU parity of the W4A8 variant (moe_w4a8_experts: FP8 activations, E2M1
weights with K32 exponent bytes) against the oracle's W4A8 path, on the
bars of the FP8 path (tests/parity.py): plan and activation codes
bit-exact, intermediate codes within 1e-4 and one value step, outputs at
relative L2 <= 5e-3 and max abs <= 2e-2 * rms.  Full-size workloads compare
sampled tokens that reach every expert the batch touches.
"""

import numpy as np
import pytest
import torch

import fp8_block_scale_amd as moe
from moe_workloads import CONFIGS, SKEW_ZERO_SCALE_EXPERT, make_case
from oracle.quant import SCALE_FP32, SCALE_UE8M0

from parity import (check_plan, check_tail_untouched, compare_intermediate, compare_output,
                    host_inputs, log, run_gpu, run_oracle)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()


_WEIGHTS = {}


def case_of(name, M=None, ids_dtype=torch.int32, **override):
    c = dict(CONFIGS[name], **override)
    key = (name, c["E"], c["K"], c["I"], c["seed"])
    cs = make_case(name, M=M, device=DEV, ids_dtype=ids_dtype, weights=_WEIGHTS.get(key),
                   config=c if override else None, fmt="w4a8")
    _WEIGHTS[key] = (cs.w13, cs.w13_s, cs.w2, cs.w2_s)
    return cs


def parity(cs, flags=0, out_init=None, tokens=None, label=""):
    log(f"[w4a8] {label} {cs.name} M={cs.M} E={cs.E} K={cs.K} I={cs.I} top_k={cs.top_k} "
        f"bm={cs.block_m} flags={flags:#x} tokens={'all' if tokens is None else len(tokens)}")
    g = run_gpu(cs, out_init=out_init, flags=flags)
    inter = SCALE_UE8M0 if flags & moe.MOE_F_INTER_UE8M0 else SCALE_FP32
    o = run_oracle(cs, h=host_inputs(cs), out_init=out_init, inter_mode=inter, tokens=tokens)
    check_plan(g, o)
    check_tail_untouched(g, o, cs.block_m)
    assert np.array_equal(g.x_q, o.x_q) and np.array_equal(g.x_s, o.x_s)
    rows = o.res.row_valid.copy()
    if tokens is not None:
        t_of_row = np.where(rows, o.sorted[:o.P] // cs.top_k, -1)
        rows &= np.isin(t_of_row, np.asarray(tokens))
    ic = compare_intermediate(g.h_q[:o.P], g.h_s[:o.P], o.res.h_q, o.res.h_s, rows)
    trows = np.nonzero(o.res.computed_tokens)[0]
    oc = compare_output(g.out[trows], o.res.ref64[trows])
    log(f"[w4a8]   ok: P={o.P} inter={ic} out={oc} oracle_s={o.seconds:.2f}")
    return g, o


def cover_tokens(cs, n, seed, extra=()):
    """n random tokens plus the first, the last and `extra`, then greedily
    tokens that reach experts not yet reached, until every expert the batch
    touches feeds a compared row."""
    rng = np.random.default_rng(seed)
    t = set(rng.choice(cs.M, size=min(n, cs.M), replace=False).tolist()) | set(extra)
    t |= {0, cs.M - 1}
    ids = cs.topk_ids.cpu().numpy()
    valid = (ids >= 0) & (ids < cs.E)
    onehot = np.zeros((cs.M, cs.E), dtype=bool)
    rr, cc = np.nonzero(valid)
    onehot[rr, ids[rr, cc]] = True
    covered = onehot[sorted(t)].any(0)
    touched = onehot.any(0)
    while (touched & ~covered).any():
        best = int(np.argmax(onehot[:, ~covered].sum(1)))
        t.add(best)
        covered |= onehot[best]
    return sorted(t)


SPLIT1 = 1 << moe.MOE_F_SPLITK_SHIFT


@pytest.mark.parametrize("flags", [0, SPLIT1, moe.MOE_F_INTER_UE8M0])
def test_tiny(flags):
    parity(case_of("tiny"), flags=flags, label="tiny")


@pytest.mark.parametrize("bm", [8, 32, 64, 128])
def test_tiny_block_m(bm):
    parity(case_of("tiny", M=24, block_m=bm), label="tiny block_m")


def test_accumulates_into_prefilled_output():
    cs = case_of("tiny")
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    init = (torch.randn((cs.M, cs.K), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    parity(cs, out_init=init, label="prefilled")


def test_scale_spread_within_k_blocks():
    """K32 exponents spread over 23 binades inside each 128-wide K-block (the
    exactness limit of the gate/up widening) and over the rows; the weights
    keep their codes."""
    cs = case_of("tiny", M=16)
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    w13e = torch.randint(104, 128, cs.w13_s.shape, generator=g, device=DEV, dtype=torch.int32)
    w2e = torch.randint(110, 134, cs.w2_s.shape, generator=g, device=DEV, dtype=torch.int32)
    cs.w13_s = w13e.to(torch.uint8)
    cs.w2_s = w2e.to(torch.uint8)
    parity(cs, label="scale spread")


@pytest.mark.parametrize("M,flags", [(1, 0), (1, SPLIT1), (1, 7 << moe.MOE_F_SPLITK_SHIFT), (4, 0),
                                     (16, 0), (1, 1 << moe.MOE_F_DOWN_PATH_SHIFT),
                                     (16, 1 << moe.MOE_F_DOWN_PATH_SHIFT)])
def test_decode(M, flags):
    """The decode shape; by default its down stage is the column-split kernel
    (E2M1 weight slabs, the route sum in the same launch), forced here also
    onto the per-block down kernel with its finalize."""
    parity(case_of("decode", M=M), flags=flags, label="decode")


COLS = moe.MOE_PATH_COLUMNS << moe.MOE_F_DOWN_PATH_SHIFT


@pytest.mark.parametrize("name,M,bm", [("tiny", None, 8), ("decode", 2, 8), ("decode", 21, 8),
                                       ("decode", 12, 16)])
def test_column_down(name, M, bm):
    """The column-split down on E2M1 weights, forced: both block sizes, up
    to 189 routes."""
    cs = case_of(name, M=M, block_m=bm)
    parity(cs, flags=COLS, label=f"column down bm={bm}")


@pytest.mark.parametrize("dt", [torch.int32, torch.int64])
def test_column_down_skew(dt):
    """A skew-like batch at I = 256 on the column-split down: hot experts
    with several blocks, duplicate experts within a token, 1% masked routes,
    a zero-scale expert."""
    cfg = dict(CONFIGS["skew"], M=18, I=256, block_m=16, seed=47)
    cs = make_case("skew-i256", device=DEV, config=cfg, ids_dtype=dt, fmt="w4a8")
    parity(cs, flags=COLS, label=f"column down skew {dt}")


def test_page1_small():
    parity(case_of("page1", M=24), label="page1 small")


@pytest.mark.parametrize("M", [1024, 2048, 4096, 8192])
def test_page1_sampled(M):
    """Page 1's W4A8 workload (E=288, K=4096, I=1024, top-8) at its four
    token counts (the per-block gate/up at 1024, the persistent kernels above);
    the sampled tokens reach every expert."""
    cs = case_of("page1", M=M)
    parity(cs, tokens=cover_tokens(cs, 6, M), label="page1")


GU_PERSIST = moe.MOE_PATH_PERSISTENT << moe.MOE_F_GATEUP_PATH_SHIFT
GU_STREAM = moe.MOE_PATH_STREAM << moe.MOE_F_GATEUP_PATH_SHIFT
DN_PERSIST = moe.MOE_PATH_PERSISTENT << moe.MOE_F_DOWN_PATH_SHIFT
DN_STREAM = moe.MOE_PATH_STREAM << moe.MOE_F_DOWN_PATH_SHIFT


@pytest.mark.parametrize("gu,dn", [(GU_PERSIST, DN_STREAM), (GU_STREAM, DN_PERSIST),
                                   (GU_PERSIST, DN_PERSIST)])
@pytest.mark.parametrize("name,M,bm", [("tiny", 24, 8), ("tiny", 24, 16), ("tiny", 40, 128),
                                       ("page1", 300, 32), ("skew", 96, 64)])
def test_persistent_kernels(name, M, bm, gu, dn):
    """The W4A8 stages on the persistent kernels, forced (at these sizes the
    schedule would pick the per-block ones), every pairing, block_m 8..128."""
    cs = case_of(name, M=M, block_m=bm)
    parity(cs, flags=gu | dn, tokens=cover_tokens(cs, 6, M + bm) if cs.M > 64 else None,
           label="persistent")


def test_persistent_down_long_intermediate_rows():
    """I = 2048: rows too long for the per-block down kernel's LDS tile; the
    persistent down kernel takes them."""
    cfg = dict(CONFIGS["tiny"], M=24, E=8, K=512, I=2048, top_k=2, block_m=64, seed=7)
    cs = make_case("long_rows_w4", device=DEV, config=cfg, fmt="w4a8")
    parity(cs, flags=DN_PERSIST, label="persistent down, I=2048")


@pytest.mark.parametrize("K,I,M,E,top_k,bm,flags", [
    (384, 128, 37, 5, 3, 16, 0),                    # three K-blocks, one intermediate block
    (384, 128, 37, 5, 3, 16, GU_PERSIST | DN_PERSIST),
    (640, 384, 19, 7, 2, 8, 0),                     # five K-blocks, three intermediate blocks
    (640, 384, 19, 7, 2, 8, GU_PERSIST | DN_PERSIST),
    (128, 256, 64, 3, 3, 32, 3 << moe.MOE_F_SPLITK_SHIFT),   # one K-block (split 3 -> 1)
    # nine K-blocks in five splits (64 tokens: at 9 tokens the 1e-4 code
    # budget admits no rounding tie at all among 9216 codes)
    (1152, 256, 64, 4, 4, 16, 5 << moe.MOE_F_SPLITK_SHIFT),
])
def test_ragged_shapes(K, I, M, E, top_k, bm, flags):
    """Odd K-block counts, one- and three-block intermediate widths, ragged
    token counts, forced splits, both kernel families."""
    cfg = dict(CONFIGS["tiny"], M=M, E=E, K=K, I=I, top_k=top_k, block_m=bm, seed=K + I + M)
    cs = make_case("ragged_w4", device=DEV, config=cfg, fmt="w4a8")
    parity(cs, flags=flags, label="ragged")


def test_both_gate_up_families_agree_closely():
    """Same layer through both gate/up families: intermediates within the
    one-step budget of each other, outputs within the output bar."""
    cs = case_of("page1", M=512)
    g1 = run_gpu(cs, flags=GU_PERSIST)
    g2 = run_gpu(cs, flags=GU_STREAM)
    assert g1.P == g2.P
    rows = (g1.sorted[:g1.P] >= 0) & (g1.sorted[:g1.P] < cs.M * cs.top_k)
    compare_intermediate(g1.h_q[:g1.P], g1.h_s[:g1.P], g2.h_q[:g2.P], g2.h_s[:g2.P], rows)
    compare_output(g1.out, g2.out)


@pytest.mark.parametrize("dt", [torch.int32, torch.int64])
def test_skew_masked_routes_and_zero_expert(dt):
    """Masked routes (-1), int32 and int64 ids, an expert whose codes are all
    zero, hot experts with several plan blocks."""
    cs = case_of("skew", M=256, ids_dtype=dt)
    ids = cs.topk_ids.cpu().numpy()
    masked = int(np.nonzero((ids < 0).any(1))[0][0])
    zero = int(np.nonzero((ids == SKEW_ZERO_SCALE_EXPERT).any(1))[0][0])
    parity(cs, tokens=cover_tokens(cs, 8, 3, extra=(masked, zero)), label="skew")


def test_rejects_what_does_not_apply():
    cs = case_of("tiny")
    b = moe.MoeLayerBuffers(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, 0, DEV, w4a8=True)
    out = torch.zeros((cs.M, cs.K), dtype=torch.bfloat16, device=DEV)
    fuse_on = moe.MOE_FUSE_ON << moe.MOE_F_FUSE_SHIFT
    for fl in (moe.MOE_F_FP8_GATEUP, moe.MOE_F_INTER_UE8M0 | moe.MOE_F_MMA_E8M0, fuse_on,
               moe.MOE_F_W13_PACKED, moe.MOE_PATH_COLUMNS << moe.MOE_F_GATEUP_PATH_SHIFT):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_w4a8_experts(b.x_q, b.x_s, cs.w13, cs.w13_s, cs.w2, cs.w2_s, cs.topk_weights,
                                 b.sorted_ids, b.expert_ids, b.ntp, cs.top_k, cs.block_m, out,
                                 b.workspace, fl)
        assert ei.value.status == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("name,M,flags", [("decode", 16, 0), ("decode", 16, DN_STREAM),
                                          ("page1", 512, 0),
                                          ("page1", 512, GU_PERSIST | DN_PERSIST)])
def test_graph_replay_matches_eager(name, M, flags):
    """The W4A8 layer (plan + quantisation + moe_w4a8_experts, per-block and
    persistent kernels) captured in a HIP graph: every replay, with eager
    work and synchronisations between replays, gives the eager output bit
    for bit."""
    cs = case_of(name, M=M)
    log(f"[w4a8 graph] {name} M={cs.M} flags={flags:#x}")
    b = moe.MoeLayerBuffers(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, flags, DEV, w4a8=True)

    def layer(out, stream):
        moe.moe_plan_quant(cs.topk_ids, cs.E, cs.block_m, b.sorted_ids, b.expert_ids, b.ntp, cs.x,
                           b.x_q, b.x_s, moe.MOE_SCALE_FP32, b.plan_ws, stream)
        moe.moe_w4a8_experts(b.x_q, b.x_s, cs.w13, cs.w13_s, cs.w2, cs.w2_s, cs.topk_weights,
                             b.sorted_ids, b.expert_ids, b.ntp, cs.top_k, cs.block_m, out,
                             b.workspace, flags, stream)

    ref = torch.zeros((cs.M, cs.K), dtype=torch.bfloat16, device=DEV)
    layer(ref, torch.cuda.current_stream())
    torch.cuda.synchronize()
    out = torch.zeros_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(out, torch.cuda.current_stream())
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager layer"
        scratch = torch.zeros_like(ref)             # eager work between replays
        layer(scratch, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(scratch, ref)
