"""The packed W13 layout (moe_prepack_w13, MOE_F_W13_PACKED): the prepack
writes exactly the documented layout (compared byte for byte with a numpy
construction of it from the header's definition), and every gate/up kernel
family computes bit-identical intermediates and outputs from packed weights
as from the plain layout (the same bytes reach the same LDS stage image)."""

import numpy as np
import pytest
import torch

import fp8_block_scale_amd as moe
from moe_workloads import CONFIGS, make_case

from parity import log

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()


def packed_reference(w13):
    """The layout as the header defines it, built with numpy fancy indexing."""
    E, twoI, K = w13.shape
    I, nkb, njt = twoI // 2, K // 128, twoI // 256
    r = np.arange(256)
    rows = np.where(r < 128, r, I + r - 128)                       # + jt * 128
    pos = np.arange(8)
    chunk = pos[None, :] ^ (r[:, None] & 7)                        # chunk stored at position pos
    out = np.empty((E, njt, nkb, 256, 8, 16), np.uint8)
    w = w13.reshape(E, twoI, nkb, 8, 16)
    for jt in range(njt):
        for kb in range(nkb):
            out[:, jt, kb] = w[:, (rows + jt * 128)[:, None], kb, chunk]
    return out.reshape(E, twoI, K)


@pytest.mark.parametrize("E,I,K", [(3, 256, 384), (2, 128, 128), (5, 384, 1024)])
def test_prepack_layout(E, I, K):
    g = torch.Generator(device=DEV)
    g.manual_seed(E * 1000 + I + K)
    w13 = torch.randint(0, 256, (E, 2 * I, K), generator=g, device=DEV, dtype=torch.int32)
    w13 = w13.to(torch.uint8)
    log(f"[prepack] E={E} I={I} K={K}")
    packed = moe.moe_prepack_w13(w13)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), packed_reference(w13.cpu().numpy()))


FUSE_ON = moe.MOE_FUSE_ON << moe.MOE_F_FUSE_SHIFT
PERSIST = ((moe.MOE_PATH_PERSISTENT << moe.MOE_F_GATEUP_PATH_SHIFT)
           | (moe.MOE_PATH_PERSISTENT << moe.MOE_F_DOWN_PATH_SHIFT))
STREAM = ((moe.MOE_PATH_STREAM << moe.MOE_F_GATEUP_PATH_SHIFT)
          | (moe.MOE_PATH_STREAM << moe.MOE_F_DOWN_PATH_SHIFT))
E8 = moe.MOE_F_INTER_UE8M0 | moe.MOE_F_MMA_E8M0


def _layer(cs, w13, flags, act_mode):
    b = moe.MoeLayerBuffers(cs.M, cs.K, cs.I, cs.E, cs.top_k, cs.block_m, flags, DEV)
    b.workspace.fill_(0x5A)
    out = torch.zeros((cs.M, cs.K), dtype=torch.bfloat16, device=DEV)
    moe.moe_plan_quant(cs.topk_ids, cs.E, cs.block_m, b.sorted_ids, b.expert_ids, b.ntp, cs.x,
                       b.x_q, b.x_s, act_mode, b.plan_ws)
    moe.moe_fp8_experts(b.x_q, b.x_s, w13, cs.w13_s, cs.w2, cs.w2_s, cs.topk_weights,
                        b.sorted_ids, b.expert_ids, b.ntp, cs.top_k, cs.block_m, out, b.workspace,
                        flags)
    torch.cuda.synchronize()
    P = int(b.ntp.item())
    hq, hs = b.intermediate()
    return out.cpu(), hq[:P].cpu(), hs[:P].cpu()


@pytest.mark.parametrize("name,M,flags", [
    ("tiny", None, 0), ("decode", 1, 0), ("decode", 16, 7 << moe.MOE_F_SPLITK_SHIFT),
    ("decode", 16, FUSE_ON), ("page1", 512, PERSIST), ("page1", 4096, 0), ("page1", 256, STREAM),
    ("zipf", 1024, E8), ("zipf", 64, E8 | STREAM),
    ("page1", 512, moe.MOE_F_FP8_GATEUP | PERSIST)])
def test_packed_weights_bit_identical(name, M, flags):
    cs = make_case(name, M=M, device=DEV)
    act = moe.MOE_SCALE_UE8M0 if cs.pow2 else moe.MOE_SCALE_FP32
    if cs.pow2:
        flags |= moe.MOE_F_INTER_UE8M0
    log(f"[packed] {name} M={cs.M} flags={flags:#x}")
    ref = _layer(cs, cs.w13, flags, act)
    packed = moe.moe_prepack_w13(cs.w13)
    got = _layer(cs, packed, flags | moe.MOE_F_W13_PACKED, act)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    assert ref[0].abs().max() > 0
