"""GPU parity of the router fused into the plan (moe_route_plan) against the
oracle: chosen experts and the whole plan bit-exact (the choice compares the
same FP32 logits on both sides), weights within FP32 rounding of the FP64
oracle, activation codes bit-exact when the quantisation rides along, and a
whole decode layer behind the router with a shared expert (the E=257,
top-9-including-shared geometry, routed scaling 2.5) to the output bar."""

import numpy as np
import pytest
import torch

import fp8_block_scale_amd as moe
from moe_workloads import make_case
from oracle import experts_ref, plan_ref, quant_act_ref, router_ref

from parity import compare_output, log

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()


def _logits(M, Er, seed, ties=False):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    if ties:       # few distinct values: exact ties everywhere, -0 and +0 among them
        v = torch.randint(-3, 4, (M, Er), generator=g, device=DEV).float()
        neg0 = torch.rand((M, Er), generator=g, device=DEV) < 0.5
        return torch.where((v == 0) & neg0, torch.tensor(-0.0, device=DEV), v)
    return torch.randn((M, Er), generator=g, device=DEV, dtype=torch.float32)


def _route(logits, k, ns, scale, bm, multi, x=None):
    M, Er = logits.shape
    E, kk = Er + ns, k + ns
    sc, bc = moe.moe_plan_capacity(M, kk, E, bm)
    ids = torch.full((M, kk), -7, dtype=torch.int32, device=DEV)
    w = torch.full((M, kk), -1.0, dtype=torch.float32, device=DEV)
    s = torch.full((sc,), 0x7F7F7F7F, dtype=torch.int32, device=DEV)
    e = torch.full((bc,), 0x7F7F7F7F, dtype=torch.int32, device=DEV)
    p = torch.empty(1, dtype=torch.int32, device=DEV)
    n = moe.moe_plan_workspace_size(M, kk, E, bm) if multi else 0
    ws = torch.empty(n, dtype=torch.uint8, device=DEV) if n else None
    q = qs = None
    if x is not None:
        q = torch.full(x.shape, 0x5A, dtype=torch.uint8, device=DEV)
        qs = torch.empty((M, x.shape[1] // 128), dtype=torch.float32, device=DEV)
    moe.moe_route_plan(logits, k, ns, scale, bm, ids, w, s, e, p, ws, x, q, qs)
    torch.cuda.synchronize()
    return ids, w, s, e, int(p.item()), q, qs


CASES = [  # M, E_routed, top_k, n_shared, scale, block_m, ties
    (1, 256, 8, 1, 2.5, 16, False), (16, 256, 8, 1, 2.5, 16, False),
    (4096, 288, 8, 0, 1.0, 64, False), (2048, 512, 10, 0, 1.0, 64, False),
    (200, 64, 8, 0, 1.0, 16, True), (5000, 64, 4, 1, 1.0, 128, True),
    (333, 1023, 32, 1, 0.75, 32, False), (3, 5, 5, 0, 1.0, 8, True),
]


@pytest.mark.parametrize("multi", [False, True])
@pytest.mark.parametrize("M,Er,k,ns,scale,bm,ties", CASES)
def test_route_plan_matches_oracle(M, Er, k, ns, scale, bm, ties, multi):
    kk = k + ns
    if not multi and moe.moe_plan_workspace_size(M, kk, Er + ns, bm) and M * kk > 30000:
        pytest.skip("too many routes for the one-workgroup build")
    log(f"[route] M={M} Er={Er} k={k} shared={ns} scale={scale} bm={bm} ties={ties} multi={multi}")
    logits = _logits(M, Er, M * 7 + Er, ties)
    ids, w, s, e, P, _, _ = _route(logits, k, ns, scale, bm, multi)
    rids, rw = router_ref(logits.cpu().numpy(), k, ns, scale)
    assert np.array_equal(ids.cpu().numpy(), rids), "chosen experts differ"
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), rw, rtol=2e-6, atol=1e-12)
    rs, rx, rP = plan_ref(rids, Er + ns, bm)
    s, e = s.cpu().numpy(), e.cpu().numpy()
    assert P == rP and np.array_equal(s[:P], rs) and np.array_equal(e[:P // bm], rx)
    assert np.all(s[P:] == 0x7F7F7F7F) and np.all(e[P // bm:] == 0x7F7F7F7F)


@pytest.mark.parametrize("M,multi", [(16, False), (600, True)])
def test_route_plan_with_quantisation(M, multi):
    logits = _logits(M, 256, 5 + M)
    g = torch.Generator(device=DEV)
    g.manual_seed(M)
    x = torch.randn((M, 7168), generator=g, device=DEV).to(torch.bfloat16)
    ids, w, s, e, P, q, qs = _route(logits, 8, 1, 2.5, 16, multi, x=x)
    rq, rs = quant_act_ref(x.float().cpu().numpy())
    assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(qs.cpu().numpy(), rs)
    rids, _ = router_ref(logits.cpu().numpy(), 8, 1, 2.5)
    assert np.array_equal(ids.cpu().numpy(), rids)


@pytest.mark.parametrize("M", [1, 16])
def test_decode_layer_behind_the_router(M):
    """256 routed experts + 1 shared (expert 256) of the decode geometry
    (K=7168, I=256), routed scaling 2.5, top-8 + shared: route + plan +
    quantisation in one call, then moe_fp8_experts; against router_ref ->
    plan_ref -> quant_act_ref -> experts_ref."""
    cs = make_case("decode", M=M, device=DEV)
    assert cs.E == 257
    logits = _logits(M, 256, 100 + M)
    kk = 9
    b = moe.MoeLayerBuffers(M, cs.K, cs.I, cs.E, kk, cs.block_m, 0, DEV)
    ids = torch.empty((M, kk), dtype=torch.int32, device=DEV)
    w = torch.empty((M, kk), dtype=torch.float32, device=DEV)
    moe.moe_route_plan(logits, 8, 1, 2.5, cs.block_m, ids, w, b.sorted_ids, b.expert_ids, b.ntp,
                       b.plan_ws, cs.x, b.x_q, b.x_s)
    out = torch.zeros((M, cs.K), dtype=torch.bfloat16, device=DEV)
    moe.moe_fp8_experts(b.x_q, b.x_s, cs.w13, cs.w13_s, cs.w2, cs.w2_s, w, b.sorted_ids,
                        b.expert_ids, b.ntp, kk, cs.block_m, out, b.workspace)
    torch.cuda.synchronize()
    rids, rw = router_ref(logits.cpu().numpy(), 8, 1, 2.5)
    rs, rx, rP = plan_ref(rids, 257, cs.block_m)
    xq, xs = quant_act_ref(cs.x.float().cpu().numpy())
    res = experts_ref(xq, xs, cs.w13.cpu().numpy(), cs.w13_s.cpu().numpy(), cs.w2.cpu().numpy(),
                      cs.w2_s.cpu().numpy(), rw.astype(np.float32), rs, rx, rP, kk, cs.block_m)
    st = compare_output(out.float().cpu().numpy().astype(np.float64), res.ref64)
    log(f"[router layer] M={M} {st}")


def test_graph_replay_matches_eager():
    """Routing + plan + quantisation (moe_route_plan, both builders) captured
    in a HIP graph: every replay writes the eager ids, weights, plan and codes
    bit for bit."""
    for M, multi in ((16, False), (4096, True)):
        logits = _logits(M, 256, 77 + M)
        g0 = torch.Generator(device=DEV)
        g0.manual_seed(M)
        x = torch.randn((M, 7168), generator=g0, device=DEV).to(torch.bfloat16)
        log(f"[router graph] M={M} multi={multi}")
        ref = _route(logits, 8, 1, 2.5, 16, multi, x)
        E, kk = 257, 9
        sc, bc = moe.moe_plan_capacity(M, kk, E, 16)
        ids = torch.empty((M, kk), dtype=torch.int32, device=DEV)
        w = torch.empty((M, kk), dtype=torch.float32, device=DEV)
        s = torch.empty(sc, dtype=torch.int32, device=DEV)
        e = torch.empty(bc, dtype=torch.int32, device=DEV)
        p = torch.empty(1, dtype=torch.int32, device=DEV)
        n = moe.moe_plan_workspace_size(M, kk, E, 16) if multi else 0
        ws = torch.empty(n, dtype=torch.uint8, device=DEV) if n else None
        q = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
        qs = torch.empty((M, x.shape[1] // 128), dtype=torch.float32, device=DEV)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            moe.moe_route_plan(logits, 8, 1, 2.5, 16, ids, w, s, e, p, ws, x, q, qs,
                               stream=torch.cuda.current_stream())
        for rep in range(3):
            for t in (ids, s, e, p):
                t.fill_(-3)
            graph.replay()
            torch.cuda.synchronize()
            P = int(p.item())
            assert P == ref[4], rep
            assert torch.equal(ids, ref[0]) and torch.equal(w, ref[1])
            assert torch.equal(s[:P], ref[2][:P]) and torch.equal(e[:P // 16], ref[3][:P // 16])
            assert torch.equal(q, ref[5]) and torch.equal(qs, ref[6])
