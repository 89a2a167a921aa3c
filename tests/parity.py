"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, and compare.

Bars (the stated parity tolerances):
  * plan (sorted ids, expert ids, padded length) and activation codes and
    scales: bit-exact;
  * intermediate FP8 codes: at most 1e-4 of the codes of valid rows may
    differ, and each differing code must be one value step from the oracle's
    (ranks of the 253 ordered E4M3 values; +0 and -0 are one value) -- or, in
    a group whose scale itself landed on the other side of a rounding
    boundary, within one value step after dequantisation;
  * output: relative L2 <= 5e-3 and, per element, |gpu - ref| <= 2e-2 *
    rms(ref) + half a BF16 ulp of ref, with the FP64 oracle sum (before its
    BF16 rounding) as ref: the 2e-2 * rms bound covers the arithmetic up to
    the FP32 sum, and the BF16 output then adds its one rounding (the
    oracle's own BF16-rounded output needs the same allowance: above ~6 rms
    half an ulp alone can exceed 2e-2 * rms).  Elements that used the
    rounding allowance are counted.
"""

import sys
import time

import numpy as np
import torch

import fp8_block_scale_amd as moe
from oracle import (e4m3_decode, e4m3_decode_table, experts_ref, experts_w4a8_ref, plan_ref,
                    quant_act_ref)
from oracle.quant import SCALE_FP32, SCALE_UE8M0

REL_L2_MAX = 5e-3
MAX_ABS_RMS = 2e-2
CODE_MISMATCH_MAX = 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def code_rank(c):
    c = np.asarray(c, dtype=np.int64)
    m = c & 0x7F
    return np.where(c & 0x80, -m, m)


def compare_intermediate(gq, gs, rq, rs, rows, max_frac=CODE_MISMATCH_MAX, one_step=True):
    """gq/rq uint8 [P, I], gs/rs fp32 [P, I/128]; rows: bool mask of valid rows.
    one_step=False drops the one-value-step rule (only the fraction is bounded)."""
    gq, rq = gq[rows], rq[rows]
    gs, rs = gs[rows], rs[rows]
    n = gq.size
    diff = gq != rq
    # +0 / -0 are the same value
    diff &= ~((gq & 0x7F == 0) & (rq & 0x7F == 0))
    nd = int(diff.sum())
    if nd == 0:
        return dict(n=n, mismatched=0, frac=0.0, scale_groups=0)
    adj = np.abs(code_rank(gq) - code_rank(rq)) <= 1
    P, I = gq.shape
    grp_scale_differs = np.repeat(gs != rs, 128, axis=1)
    bad = diff & ~adj
    n_far = int(bad.sum())
    if bad.any() and one_step:
        # a group whose scale landed on the other side of a rounding boundary:
        # both dequantised values must lie within half a step of the same h
        sg = np.repeat(gs.astype(np.float64), 128, axis=1)
        sr = np.repeat(rs.astype(np.float64), 128, axis=1)
        gv, rv = e4m3_decode(gq) * sg, e4m3_decode(rq) * sr
        bound = 0.5 * (e4m3_step(gq) * sg + e4m3_step(rq) * sr) * (1 + 1e-6)
        ok = grp_scale_differs & (np.abs(gv - rv) <= bound)
        still = bad & ~ok
        assert not still.any(), (
            f"{int(still.sum())} intermediate codes differ by more than one step, "
            f"e.g. gpu={gq[still][:8]} ref={rq[still][:8]}")
    frac = nd / n
    assert frac <= max_frac, f"intermediate code mismatch fraction {frac:.3g} > {max_frac:g}"
    return dict(n=n, mismatched=nd, frac=frac, beyond_one_step=n_far,
                scale_groups=int((gs != rs).sum()))


def e4m3_step(c):
    """Spacing of the E4M3 grid at each code's magnitude (2^-9 below 2^-6)."""
    m = e4m3_decode(np.asarray(c, dtype=np.uint8) & 0x7F)
    e = np.floor(np.log2(np.maximum(m, 2.0 ** -6)))
    return 2.0 ** (e - 3)


def bf16_ulp(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def compare_output(gpu, ref64, rows=None):
    """gpu: float64 values of the BF16 output; ref64: FP64 oracle sum."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref64, dtype=np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    err = g - r
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    rel_l2 = float(np.linalg.norm(err) / max(np.linalg.norm(r), 1e-300))
    bound = MAX_ABS_RMS * rms + 0.5 * bf16_ulp(r)
    viol = np.abs(err) > bound
    n_floor = int(((np.abs(err) > MAX_ABS_RMS * rms) & ~viol).sum())
    max_abs_rms = float(np.abs(err).max() / rms) if rms > 0 else 0.0
    assert rel_l2 <= REL_L2_MAX, f"relative L2 {rel_l2:.3g} > {REL_L2_MAX}"
    if viol.any():
        i = np.unravel_index(int(np.argmax(np.where(viol, np.abs(err), -1.0))), err.shape)
        raise AssertionError(
            f"{int(viol.sum())} outputs exceed 2e-2*rms + bf16 ulp/2; max |err|/rms = "
            f"{max_abs_rms:.3g}; worst at {tuple(int(v) for v in i)}: ref/rms {r[i] / rms:.4g}, "
            f"gpu/rms {g[i] / rms:.4g}, err/rms {err[i] / rms:.4g}, bf16 ulp/rms "
            f"{bf16_ulp(r[i]) / rms:.4g}, rms {rms:.4g}")
    return dict(rel_l2=rel_l2, max_abs_over_rms=max_abs_rms, rounding_allowance_used=n_floor,
                rms=rms)


# ------------------------------------------------------------------ runs

class GpuRun:
    pass


def run_gpu(case, out_init=None, flags=0, act_mode=moe.MOE_SCALE_FP32, ntp_override=None,
            garbage_plan=True, stream=None):
    """Whole path on the GPU through the C ABI binding."""
    dev = case.x.device
    assert dev.type == "cuda"
    w4 = is_w4a8(case)
    b = moe.MoeLayerBuffers(case.M, case.K, case.I, case.E, case.top_k, case.block_m, flags, dev,
                            w4a8=w4)
    if garbage_plan:
        b.sorted_ids.fill_(0x7F7F7F7F)
        b.expert_ids.fill_(0x7F7F7F7F)
        b.workspace.fill_(0x5A)
    out = torch.zeros((case.M, case.K), dtype=torch.bfloat16, device=dev) if out_init is None \
        else out_init.clone()
    moe.moe_plan(case.topk_ids, case.E, case.block_m, b.sorted_ids, b.expert_ids, b.ntp,
                 b.plan_ws, stream)
    moe.moe_quant_act(case.x, b.x_q, b.x_s, act_mode, stream)
    ntp = b.ntp
    if ntp_override is not None:
        ntp = torch.tensor([ntp_override], dtype=torch.int32, device=dev)
    experts = moe.moe_w4a8_experts if w4 else moe.moe_fp8_experts
    experts(b.x_q, b.x_s, case.w13, case.w13_s, case.w2, case.w2_s, case.topk_weights,
            b.sorted_ids, b.expert_ids, ntp, case.top_k, case.block_m, out, b.workspace, flags,
            stream)
    torch.cuda.synchronize()
    r = GpuRun()
    r.bufs = b
    r.P = int(b.ntp.item())
    r.sorted = b.sorted_ids.cpu().numpy()
    r.expert_ids = b.expert_ids.cpu().numpy()
    r.x_q = b.x_q.cpu().numpy()
    r.x_s = b.x_s.cpu().numpy()
    hq, hs = b.intermediate()
    r.h_q = hq.cpu().numpy()
    r.h_s = hs.cpu().numpy()
    r.out = out.float().cpu().numpy().astype(np.float64)
    return r


class OracleRun:
    pass


def is_w4a8(case):
    """Cases whose weights are E2M1 with K32 exponent bytes."""
    return case.meta.get("fmt") == "w4a8"


def host_inputs(case):
    """Copy a case's inputs to host numpy arrays (byte-identical)."""
    h = dict(x=case.x.float().cpu().numpy(), ids=case.topk_ids.cpu().numpy(),
             w=case.topk_weights.cpu().numpy(), w13=case.w13.cpu().numpy(),
             w13_s=case.w13_s.cpu().numpy(), w2=case.w2.cpu().numpy(), w2_s=case.w2_s.cpu().numpy())
    return h


def run_oracle(case, h=None, out_init=None, act_mode=SCALE_FP32, inter_mode=SCALE_FP32,
               tokens=None, P_override=None):
    h = host_inputs(case) if h is None else h
    o = OracleRun()
    o.sorted, o.expert_ids, o.P = plan_ref(h["ids"], case.E, case.block_m)
    o.x_q, o.x_s = quant_act_ref(h["x"], act_mode)
    P = o.P if P_override is None else min(P_override, o.P)
    init = None if out_init is None else out_init.float().cpu().numpy()
    t0 = time.time()
    ref = experts_w4a8_ref if is_w4a8(case) else experts_ref
    o.res = ref(o.x_q, o.x_s, h["w13"], h["w13_s"], h["w2"], h["w2_s"], h["w"], o.sorted,
                o.expert_ids, P, case.top_k, case.block_m, out_init=init, inter_mode=inter_mode,
                tokens=tokens)
    o.seconds = time.time() - t0
    return o


def check_plan(g, o):
    assert g.P == o.P, f"P gpu {g.P} oracle {o.P}"
    assert np.array_equal(g.sorted[:o.P], o.sorted), "sorted_token_ids differ"
    assert np.array_equal(g.expert_ids[:len(o.expert_ids)], o.expert_ids), "expert_ids differ"


def check_tail_untouched(g, o, bm):
    """Entries beyond P keep the garbage they were filled with."""
    assert np.all(g.sorted[o.P:] == 0x7F7F7F7F)
    assert np.all(g.expert_ids[o.P // bm:] == 0x7F7F7F7F)
