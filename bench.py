#!/usr/bin/env python3
"""Benchmark of the routed FP8 W8A8 block-scale MoE expert path on one MI355X.

One step = the whole hot path over one batch: routing plan, activation
quantisation, gate/up GEMM + SwiGLU + requantisation, down GEMM + weighted
reduce-add into the BF16 output -- all HIP kernels of libmoe_fp8 through its
C ABI, on one stream, with every input already resident in HBM.  The K timed
steps are captured in one HIP graph and replayed once (--eager: launched one
by one); stage times come from graphs of K launches of each stage.

Default workload: E=288 experts, hidden K=4096, intermediate I=1024, top-8,
M=4096 tokens, block_m=64 (synthetic, seeded; weights N(0, 0.02^2) stored as
E4M3 with 128x128 FP32 block scales).  Prints one JSON line:
  value        FP8-path TFLOP/s = 2 * valid_routes * 3 * K * I / step time
  ms_per_step  milliseconds per layer call (all five steps)
  roofline     the dominant kernel (gate/up) against whichever bound binds it
               -- HBM bytes at 8 TB/s or its MFMA's dense peak (FP16 for the
               exact path, whose FP8 codes are widened before the MFMA; FP8
               with --fp8-gateup) -- timed with HIP events on the launch
               stream inside the timed region; `traffic` is the HBM bytes per
               launch from rocprofv3 counters recorded in profiles/, reported
               only while the kernel sources still hash to the ones measured
  steps35      steps 3-5 (gate/up through the reduce, the basis of the HBM
               and MFMA targets) against the HBM peak and the dense FP8 peak
  cpu_baseline the CPU oracle on a bounded sample of the same batch (median
               of three runs, host CPU model, BLAS and thread count stated)

Runs on a single GPU only; --gpus N > 1 exits with a message.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms/layer + FP8 TFLOPS (HBM GB/s at small M), E288 H4096 I1024 top8"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
FP16_MFMA_PEAK = 2500.0         # TFLOP/s dense
FP8_MFMA_PEAK = 5000.0          # TFLOP/s dense


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="page1",
                    choices=["tiny", "decode", "page1", "skew", "zipf"])
    ap.add_argument("--M", type=int, default=None, help="override the token count")
    ap.add_argument("--block-m", type=int, default=None, help="override the plan block size")
    ap.add_argument("--fp8-gateup", action="store_true",
                    help="gate/up on the FP8 MFMA (MOE_F_FP8_GATEUP)")
    ap.add_argument("--e8m0", action="store_true",
                    help="power-of-two scales inside the FP8 MFMA (zipf workload)")
    ap.add_argument("--splitk", type=int, default=0,
                    help="force the small-grid gate/up split-K factor (1..255; 0 = automatic)")
    ap.add_argument("--gateup-path", choices=("auto", "stream", "persistent", "columns"), default="auto",
                    help="force the gate/up kernel family (tuning override)")
    ap.add_argument("--down-path", choices=("auto", "stream", "persistent", "columns"), default="auto",
                    help="force the down kernel family (tuning override)")
    ap.add_argument("--fuse", choices=("auto", "on", "off"), default="auto",
                    help="steps 3-5 as one launch (on), as two stages (off), or the library's "
                         "choice (auto)")
    ap.add_argument("--w4a8", action="store_true",
                    help="the W4A8 variant: E2M1 weights with K32 exponent bytes "
                         "(moe_w4a8_experts, per-block kernels)")
    ap.add_argument("--prepack", action="store_true",
                    help="W13 in the packed tile layout (moe_prepack_w13, done before timing)")
    ap.add_argument("--router", action="store_true",
                    help="route from FP32 logits inside the plan's launches (moe_route_plan): "
                         "softmax top-k, routed scaling; the decode workload's expert 256 as a "
                         "shared expert with routed scaling 2.5")
    ap.add_argument("--separate-plan-quant", action="store_true",
                    help="moe_plan then moe_quant_act instead of the fused moe_plan_quant")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of HIP graph replays (the default: one "
                         "graph of K steps and one of K launches per stage, each replayed once)")
    ap.add_argument("--weight-sets", type=int, default=0,
                    help="copies of the expert weights cycled through step by step, like "
                         "consecutive layers, so no step finds its weights in the 256 MB "
                         "Infinity Cache (0 = enough copies for >= 1 GiB of touched weights)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=96)
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB before warm-up (a known-size "
                         "kernel to scale HBM byte counters against)")
    return ap.parse_args()


def algorithmic_bytes(case, n_touched, R_valid, P, n_tok, w4a8=False):
    """Bytes each stage must move at least once (see the layout notes of the
    library): touched expert weights and scales, activations once per token,
    intermediate rows once per valid route, the plan, and the BF16 output
    read-modify-write.  W4A8 weights: half a byte per element plus one
    exponent byte per 32."""
    K, I, M = case.K, case.I, case.M
    if w4a8:
        w13 = n_touched * (I * K + 2 * I * (K // 32))
        w2 = n_touched * (K * I // 2 + K * (I // 32))
    else:
        w13 = n_touched * (2 * I * K + (2 * I // 128) * (K // 128) * 4)
        w2 = n_touched * (K * I + (K // 128) * (I // 128) * 4)
    xq = n_tok * (K + (K // 128) * 4)
    h = R_valid * (I + (I // 128) * 4)
    plan = P * 4 + (P // case.block_m) * 4
    gate_up = w13 + xq + h + plan
    down = w2 + h + plan + R_valid * 4 + 2 * M * K * 2
    layer = w13 + w2 + xq + R_valid * 4 + plan + 2 * M * K * 2
    return dict(gate_up=gate_up, down=down, layer=layer)


CSRC = os.path.join(ROOT, "fp8_block_scale_amd", "csrc")
KERNEL_SOURCES = {
    "gateup_pipe_kernel": ("gateup_pipe.hip", "common.h", "internal.h"),
    "gateup_stream_kernel": ("gateup.hip", "gateup_item.h", "common.h", "internal.h"),
    "fused_experts_kernel": ("fused.hip", "gateup_item.h", "down_item.h", "common.h", "internal.h"),
    "gateup_slices_kernel": ("gateup_slices.hip", "common.h", "internal.h"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def gateup_kernel_name(case, sorted_cap, flags):
    """The gate/up kernel the library picks for these sizes and flags."""
    import fp8_block_scale_amd as moe
    gu = moe.moe_fp8_experts_schedule(case.M, case.K, case.I, case.E, case.top_k,
                                      case.block_m, sorted_cap, flags)[0]
    return ("gateup_stream_kernel", "gateup_pipe_kernel", "gateup_slices_kernel")[gu]


def sources_sha(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, flags):
    """HBM bytes per launch of `kernel` on `workload`, from the counter table
    in profiles/ -- None unless an entry matches the kernel, the workload, the
    flags and the current hash of the kernel's sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    sha = sources_sha(kernel)
    for e in json.loads(m.group(1)):
        if (e["kernel"] == kernel and e["workload"] == workload and e["flags"] == flags
                and e["sources_sha"] == sha):
            return e["traffic_bytes"]
    return None


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, n_tokens, runs=3, w4a8=False):
    """The CPU oracle (plain numpy, FP64 dot products) on the first n_tokens
    tokens of the same batch, all five steps, timed `runs` times (median);
    reported in the metric's unit with the host CPU, BLAS and thread count."""
    import numpy as np
    from oracle import experts_ref, experts_w4a8_ref, plan_ref, quant_act_ref
    ref = experts_w4a8_ref if w4a8 else experts_ref
    blas, threads = "unknown", os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            threads = max(p.get("num_threads", 1) for p in info)
            blas = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in info)
    except Exception:  # pragma: no cover
        pass
    h = dict(x=case.x[:n_tokens].float().cpu().numpy(), ids=case.topk_ids.cpu().numpy(),
             w=case.topk_weights.cpu().numpy(), w13=case.w13.cpu().numpy(),
             w13_s=case.w13_s.cpu().numpy(), w2=case.w2.cpu().numpy(), w2_s=case.w2_s.cpu().numpy())
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        s, e, P = plan_ref(h["ids"], case.E, case.block_m)
        xq, xs = quant_act_ref(h["x"])
        xq_full = np.zeros((case.M, case.K), np.uint8)
        xs_full = np.zeros((case.M, case.K // 128), np.float32)
        xq_full[:n_tokens], xs_full[:n_tokens] = xq, xs
        ref(xq_full, xs_full, h["w13"], h["w13_s"], h["w2"], h["w2_s"], h["w"], s, e, P,
            case.top_k, case.block_m, tokens=range(n_tokens))
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    ids = h["ids"][:n_tokens]
    routes = int(((ids >= 0) & (ids < case.E)).sum())
    flops = 2.0 * routes * 3 * case.K * case.I
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_tokens} of {case.M} tokens ({routes} routes, all five steps), "
                      f"median of {runs} runs: {', '.join(f'{t:.2f}' for t in times)} s wall",
            "seconds": dt, "runs_s": [round(t, 3) for t in times], "host_cpus": os.cpu_count(),
            "cpu_model": host_cpu_model(), "blas": blas}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the expert path is benchmarked per GPU and its sharding is described, not run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_block_scale_amd as moe
    from moe_workloads import make_case

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.time()
    config = None
    if args.block_m is not None:
        from moe_workloads import CONFIGS
        config = dict(CONFIGS[args.workload], block_m=args.block_m)
    case = make_case(args.workload, M=args.M, device=dev, config=config,
                     fmt="w4a8" if args.w4a8 else "w8a8")
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    flags = 0
    act_mode = moe.MOE_SCALE_FP32
    if case.pow2:
        flags |= moe.MOE_F_INTER_UE8M0
        act_mode = moe.MOE_SCALE_UE8M0
        if args.e8m0:
            flags |= moe.MOE_F_MMA_E8M0
    if args.fp8_gateup:
        flags |= moe.MOE_F_FP8_GATEUP
    if args.splitk:
        flags |= (args.splitk & 0xFF) << moe.MOE_F_SPLITK_SHIFT
    paths = {"auto": moe.MOE_PATH_AUTO, "stream": moe.MOE_PATH_STREAM,
             "persistent": moe.MOE_PATH_PERSISTENT, "columns": moe.MOE_PATH_COLUMNS}
    flags |= paths[args.gateup_path] << moe.MOE_F_GATEUP_PATH_SHIFT
    flags |= paths[args.down_path] << moe.MOE_F_DOWN_PATH_SHIFT
    fuses = {"auto": moe.MOE_FUSE_AUTO, "on": moe.MOE_FUSE_ON, "off": moe.MOE_FUSE_OFF}
    flags |= fuses[args.fuse] << moe.MOE_F_FUSE_SHIFT

    # Weight copies: a step reads the touched experts' weights once; with
    # fewer than ~1 GiB of them per step, back-to-back steps would find them
    # in the last-level (Infinity) cache instead of HBM.
    ids = case.topk_ids
    valid = (ids >= 0) & (ids < case.E)
    n_touched = int(torch.unique(ids[valid]).numel())
    touched_w = n_touched * 3 * case.I * case.K // (2 if args.w4a8 else 1)
    nsets = args.weight_sets or max(1, min(64, -(-(1 << 30) // max(touched_w, 1))))
    if args.prepack:        # offline: not part of a step
        assert not args.w4a8, "the packed layout is for E4M3 W13"
        case.w13 = moe.moe_prepack_w13(case.w13)
        flags |= moe.MOE_F_W13_PACKED
    wsets = [(case.w13, case.w13_s, case.w2, case.w2_s)]
    for _ in range(nsets - 1):
        wsets.append(tuple(t.clone() for t in wsets[0]))

    b = moe.MoeLayerBuffers(case.M, case.K, case.I, case.E, case.top_k, case.block_m, flags, dev,
                            w4a8=args.w4a8)
    out = torch.zeros((case.M, case.K), dtype=torch.bfloat16, device=dev)
    if args.router:
        # the E=257 geometry: 256 routed experts + expert 256 shared, top-8 + shared
        n_shared = 1 if case.E == 257 else 0
        e_routed, k_routed = case.E - n_shared, case.top_k - n_shared
        scaling = 2.5 if n_shared else 1.0
        g = torch.Generator(device=dev)
        g.manual_seed(12345)
        logits = torch.randn((case.M, e_routed), generator=g, device=dev, dtype=torch.float32)
        case.topk_ids = torch.empty((case.M, case.top_k), dtype=torch.int32, device=dev)
        case.topk_weights = torch.empty((case.M, case.top_k), dtype=torch.float32, device=dev)

    def stage_plan_quant(stream, k):
        if args.router:
            moe.moe_route_plan(logits, k_routed, n_shared, scaling, case.block_m, case.topk_ids,
                               case.topk_weights, b.sorted_ids, b.expert_ids, b.ntp, b.plan_ws,
                               case.x, b.x_q, b.x_s, act_mode, stream)
        elif args.separate_plan_quant:
            moe.moe_plan(case.topk_ids, case.E, case.block_m, b.sorted_ids, b.expert_ids, b.ntp,
                         b.plan_ws, stream)
            moe.moe_quant_act(case.x, b.x_q, b.x_s, act_mode, stream)
        else:
            moe.moe_plan_quant(case.topk_ids, case.E, case.block_m, b.sorted_ids, b.expert_ids,
                               b.ntp, case.x, b.x_q, b.x_s, act_mode, b.plan_ws, stream)

    def stage_gate_up(stream, k):
        w13, w13_s = wsets[k % nsets][:2]
        moe.moe_fp8_gate_up(b.x_q, b.x_s, w13, w13_s, b.sorted_ids, b.expert_ids, b.ntp,
                            case.top_k, case.block_m, b.workspace, flags, stream)

    def stage_down(stream, k):
        w2, w2_s = wsets[k % nsets][2:]
        moe.moe_fp8_down_reduce(w2, w2_s, case.topk_weights, b.sorted_ids, b.expert_ids,
                                b.ntp, case.top_k, case.block_m, out, b.workspace, flags, stream)

    experts_fn = moe.moe_w4a8_experts if args.w4a8 else moe.moe_fp8_experts

    def stage_layer(stream, k):
        # all five steps in one call (moe_fp8_layer): the per-block gate/up's
        # clearing launch folds into the plan's at decode sizes
        w13, w13_s, w2, w2_s = wsets[k % nsets]
        moe.moe_fp8_layer(case.x, case.topk_ids, case.topk_weights, w13, w13_s, w2, w2_s,
                          case.block_m, b.sorted_ids, b.expert_ids, b.ntp, b.x_q, b.x_s, out,
                          b.workspace, flags, act_mode, b.plan_ws, stream)

    def stage_experts(stream, k):
        w13, w13_s, w2, w2_s = wsets[k % nsets]
        experts_fn(b.x_q, b.x_s, w13, w13_s, w2, w2_s, case.topk_weights, b.sorted_ids,
                   b.expert_ids, b.ntp, case.top_k, case.block_m, out, b.workspace, flags, stream)

    if args.w4a8:
        fused = False
    else:
        sched = moe.moe_fp8_experts_schedule(case.M, case.K, case.I, case.E, case.top_k,
                                             case.block_m, b.sorted_ids.numel(), flags)
        fused = sched[4]
    # one step: plan + quantisation, then steps 3-5 as the library schedules them
    stages = (stage_plan_quant, stage_experts)

    def step(k, ev=None):
        stream = torch.cuda.current_stream()
        for i, fn in enumerate(stages):
            if ev is not None:
                ev[i].record(stream)
            fn(stream, k)
        if ev is not None:
            ev[len(stages)].record(stream)

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    if args.router:     # the routes the router chose (same count, other experts)
        ids = case.topk_ids
        valid = (ids >= 0) & (ids < case.E)
        n_touched = int(torch.unique(ids[valid]).numel())

    stream = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    gate_up = down = None
    if args.eager:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(args.steps):
            step(i, evs[i])
        t_end.record(stream)
        torch.cuda.synchronize()
        ms = t_start.elapsed_time(t_end) / args.steps
        plan_quant = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
        experts = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    else:
        # One graph holding K steps, and one per stage holding K launches of
        # it, each replayed once between two events on the replay stream (a
        # graph launch per step would add its own overhead at decode sizes).
        def capture(fns):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for k in range(args.steps):
                    for fn in fns:
                        fn(torch.cuda.current_stream(), k)
            return g

        def replay_ms(g):
            g.replay()                               # warm
            torch.cuda.synchronize()
            t_start.record(stream)
            g.replay()
            t_end.record(stream)
            torch.cuda.synchronize()
            return t_start.elapsed_time(t_end) / args.steps

        one_call = not (args.router or args.w4a8 or args.separate_plan_quant)
        ms = replay_ms(capture([stage_layer] if one_call else stages))
        plan_quant, experts = (replay_ms(capture([fn])) for fn in stages)
        if not fused and not args.w4a8:   # the two stages of steps 3-5, each timed alone
            gate_up, down = (replay_ms(capture([fn])) for fn in (stage_gate_up, stage_down))

    R_valid = int(valid.sum())
    P = int(b.ntp.item())
    flops = 2.0 * R_valid * 3 * case.K * case.I
    nb = algorithmic_bytes(case, n_touched, R_valid, P, case.M, args.w4a8)
    tflops = flops / (ms * 1e-3) / 1e12

    if fused or gate_up is None:
        # the single launch (or eager timing without stage graphs): the
        # dominant kernel is steps 3-5 as a whole, HBM-bound at these sizes
        kname = "fused_experts_kernel" if fused else ("steps 3-5 (W4A8)" if args.w4a8
                                                       else "steps 3-5")
        t_hbm = nb["layer"] / (HBM_PEAK_GBS * 1e9)
        # gate/up (2/3 of the flops) on the FP16 MFMA, down on the FP8 one
        t_mfma = flops / (FP16_MFMA_PEAK * 1e12) * (2 / 3) + flops / (FP8_MFMA_PEAK * 1e12) / 3
        if t_mfma > t_hbm:
            peak = flops / t_mfma / 1e12            # the blend of the two dense peaks
            achieved = flops / (experts * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": round(peak, 1),
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "mfma": "blend: 2/3 of the flops at the fp16 and 1/3 at the fp8 dense peak",
                    "algorithmic_flops": flops}
        else:
            achieved = nb["layer"] / (experts * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        roof.update({"frac_vs_fp8_dense_peak": round(flops / (experts * 1e-3) / 1e12 / FP8_MFMA_PEAK, 4),
                     "traffic": measured_traffic(kname, f"{case.name} M={case.M}", flags)
                     if fused else None,
                     "kernel": kname, "algorithmic_bytes": nb["layer"], "avg_ms": round(experts, 4),
                     "bound_ms": {"hbm": round(t_hbm * 1e3, 4), "mfma": round(t_mfma * 1e3, 4)}})
    else:
        # gate/up roofline: the larger of the two lower bounds on its time binds
        gu_flops = 2.0 * R_valid * case.K * 2 * case.I
        mfma_peak = FP8_MFMA_PEAK if args.fp8_gateup else FP16_MFMA_PEAK
        t_hbm = nb["gate_up"] / (HBM_PEAK_GBS * 1e9)
        t_mfma = gu_flops / (mfma_peak * 1e12)
        kernel = gateup_kernel_name(case, b.sorted_ids.numel(), flags)
        workload = f"{case.name} M={case.M}"
        if t_mfma > t_hbm:
            achieved = gu_flops / (gate_up * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": mfma_peak,
                    "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4),
                    "mfma": "fp8 16x16x128" if args.fp8_gateup else "fp16 16x16x32 (FP8 codes widened)",
                    "algorithmic_flops": gu_flops}
        else:
            achieved = nb["gate_up"] / (gate_up * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        roof["frac_vs_fp8_dense_peak"] = round(gu_flops / (gate_up * 1e-3) / 1e12 / FP8_MFMA_PEAK, 4)
        roof["traffic"] = measured_traffic(kernel, workload, flags)
        roof.update({"kernel": kernel, "algorithmic_bytes": nb["gate_up"], "avg_ms": round(gate_up, 4),
                     "bound_ms": {"hbm": round(t_hbm * 1e3, 4), "mfma": round(t_mfma * 1e3, 4)}})

    t35 = experts
    steps35 = {"ms": round(t35, 4), "algorithmic_bytes": nb["layer"],
               "GB/s": round(nb["layer"] / (t35 * 1e-3) / 1e9, 1),
               "frac_hbm": round(nb["layer"] / (t35 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "TFLOP/s": round(flops / (t35 * 1e-3) / 1e12, 2),
               "frac_fp8_dense_peak": round(flops / (t35 * 1e-3) / 1e12 / FP8_MFMA_PEAK, 4)}

    res = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 x e2m1" if args.w4a8 else "fp8",
        "data": "synthetic",
        "config": {
            "workload": f"{case.name}: E={case.E} K={case.K} I={case.I} top_k={case.top_k} "
                        f"M={case.M} block_m={case.block_m}",
            "M": case.M, "E": case.E, "K": case.K, "I": case.I, "top_k": case.top_k,
            "block_m": case.block_m, "flags": flags, "valid_routes": R_valid,
            "touched_experts": n_touched, "padded_rows": P,
        },
        "stages_ms": {"plan_quant": round(plan_quant, 4), "experts": round(experts, 4),
                      **({} if gate_up is None else {"gate_up": round(gate_up, 4),
                                                     "down_reduce": round(down, 4)})},
        "single_launch": bool(fused),
        "w13_packed": bool(args.prepack),
        "weights": "e2m1 + K32 exponent bytes" if args.w4a8 else "e4m3 + 128x128 fp32 scales",
        "router": bool(args.router),
        "launch": "eager" if args.eager else "hip graph (K steps per replay)",
        "step_call": ("moe_fp8_layer" if (not args.eager and not (args.router or args.w4a8
                                                                   or args.separate_plan_quant))
                      else "plan call + experts call"),
        "weight_sets": nsets,
        "layer_GBs": round(nb["layer"] / (ms * 1e-3) / 1e9, 1),
        "roofline": roof,
        # the basis of both targets: steps 3-5 (gate/up through the reduce)
        "steps35": steps35,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, min(args.cpu_sample_tokens, case.M), args.cpu_runs,
                                           args.w4a8)
    print(f"# generated inputs in {t_gen:.1f} s", file=sys.stderr)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
