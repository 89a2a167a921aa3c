"""moe_fp8_experts_noalloc (the entry point for callers that cannot allocate:
its workspace is the library's static per-device scratch) against
moe_fp8_experts with a caller workspace, through the C ABI: two no-alloc
calls in a row -- the decode shape at M=16, then at M=4 with a forced split-K
factor, so the second call starts on the scratch contents the first left --
each bit-identical to the workspace entry point's output on the same inputs
(same kernels, deterministic reduction) and within the output bar of the
oracle's FP64 sum."""

import numpy as np
import pytest
import torch

import fp8_block_scale_amd as moe
from moe_workloads import make_case
from parity import compare_output, log, run_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _prepare(cs, flags):
    b = moe.MoeLayerBuffers(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, flags, DEV)
    moe.moe_plan_quant(cs.topk_ids, cs.E, cs.block_m, b.sorted_ids, b.expert_ids, b.ntp, cs.x,
                       b.x_q, b.x_s, moe.MOE_SCALE_FP32, b.plan_ws)
    return b


def _experts(cs, b, flags, noalloc):
    out = torch.zeros((cs.M, cs.K), dtype=torch.bfloat16, device=DEV)
    args = (b.x_q, b.x_s, cs.w13, cs.w13_s, cs.w2, cs.w2_s, cs.topk_weights, b.sorted_ids,
            b.expert_ids, b.ntp, cs.top_k, cs.block_m, out)
    if noalloc:
        moe.moe_fp8_experts_noalloc(*args, flags=flags)
    else:
        moe.moe_fp8_experts(*args, b.workspace, flags=flags)
    return out


def test_noalloc_matches_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    first = make_case("decode", M=16, device=DEV)
    w = (first.w13, first.w13_s, first.w2, first.w2_s)
    second = make_case("decode", M=4, device=DEV, weights=w)
    calls = [(first, 0), (second, 7 << moe.MOE_F_SPLITK_SHIFT)]
    bufs = [_prepare(cs, fl) for cs, fl in calls]
    refs = [_experts(cs, b, fl, noalloc=False) for (cs, fl), b in zip(calls, bufs)]
    torch.cuda.synchronize()
    got = []
    for (cs, fl), b in zip(calls, bufs):          # two no-alloc calls in a row
        log(f"[noalloc] decode M={cs.M} flags={fl:#x}")
        got.append(_experts(cs, b, fl, noalloc=True))
    torch.cuda.synchronize()
    for (cs, fl), r, g in zip(calls, refs, got):
        assert torch.equal(g, r), f"M={cs.M}: no-alloc output differs from the workspace call"
        o = run_oracle(cs)
        st = compare_output(g.float().cpu().numpy().astype(np.float64), o.res.ref64)
        log(f"[noalloc]   M={cs.M} ok: {st}")


def test_noalloc_column_slice_path():
    """The same through the column-slice gate/up and the column-split down
    (FP32 rows in the scratch, requantised by the down stage): decode M=2,
    then M=1 on what the first call left."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    flags = ((moe.MOE_PATH_COLUMNS << moe.MOE_F_GATEUP_PATH_SHIFT)
             | (moe.MOE_PATH_COLUMNS << moe.MOE_F_DOWN_PATH_SHIFT))
    first = make_case("decode", M=2, device=DEV)
    w = (first.w13, first.w13_s, first.w2, first.w2_s)
    second = make_case("decode", M=1, device=DEV, weights=w)
    calls = [(first, flags), (second, flags)]
    bufs = [_prepare(cs, fl) for cs, fl in calls]
    refs = [_experts(cs, b, fl, noalloc=False) for (cs, fl), b in zip(calls, bufs)]
    torch.cuda.synchronize()
    got = []
    for (cs, fl), b in zip(calls, bufs):
        log(f"[noalloc] column slices decode M={cs.M} flags={fl:#x}")
        got.append(_experts(cs, b, fl, noalloc=True))
    torch.cuda.synchronize()
    for (cs, fl), r, g in zip(calls, refs, got):
        assert torch.equal(g, r), f"M={cs.M}: no-alloc output differs from the workspace call"
        o = run_oracle(cs)
        st = compare_output(g.float().cpu().numpy().astype(np.float64), o.res.ref64)
        log(f"[noalloc]   M={cs.M} ok: {st}")
