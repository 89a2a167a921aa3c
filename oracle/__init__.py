"""CPU oracle for the routed FP8 W8A8 block-scale MoE expert path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code, table or constant generator with the
HIP kernels.

What it computes, step by step, in the order the method takes them (the
method itself is specified across three pages: FlashInfer PR #4287 "add
optimized Blackwell W8A8 expert up/down compute", its PR summary and its
"Public contract and review fixes" section; sglang-glm53-flash-sm120 PR #13,
its description and validation paragraphs; SGLang PR #43556 "Requantize
block-FP8 MoE weights to UE8M0 for DeepGEMM", its motivation and
modifications sections):

* ``e4m3``    -- OCP E4M3FN encode (round to nearest even, saturating at 448)
                and decode, BF16 round-to-nearest-even.
* ``plan``    -- the moe_align_block_size routing plan (stable counting sort
                by expert, each expert padded to a multiple of block_m).
* ``quant``   -- 1x128 activation quantisation, FP32 scale mode and the
                power-of-two (UE8M0) scale mode.
* ``e2m1``    -- E2M1 (FP4) codec and K32 power-of-two block dequantisation
                of the W4A8 variant's weights.
* ``router``  -- softmax top-k routing with renormalised weights, routed
                scaling and an optional shared expert (the router the plan
                can be fused with).
* ``experts`` -- gate/up GEMM with 128x128 block scales, SwiGLU, per-row
                128-group FP8 requantisation, down GEMM, route weighting and
                the reduce-add into the caller's output, all dot products in
                FP64.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
closed forms, library routines and invariants (see each test's docstring).
"""

from .e4m3 import (
    E4M3_MAX,
    FLT_MIN,
    bf16_round_f32,
    bf16_round_f64,
    e4m3_decode,
    e4m3_decode_table,
    e4m3_encode,
)
from .plan import plan_capacity, plan_ref
from .quant import quant_groups_ref, quant_act_ref, ue8m0_exponent
from .experts import experts_ref, experts_w4a8_ref, ExpertsResult
from .e2m1 import E2M1_MAX, dequant_k32, e2m1_decode, e2m1_encode, unpack_e2m1
from .router import router_ref

__all__ = [
    "E4M3_MAX",
    "FLT_MIN",
    "bf16_round_f32",
    "bf16_round_f64",
    "e4m3_decode",
    "e4m3_decode_table",
    "e4m3_encode",
    "plan_capacity",
    "plan_ref",
    "quant_groups_ref",
    "quant_act_ref",
    "ue8m0_exponent",
    "experts_ref",
    "experts_w4a8_ref",
    "ExpertsResult",
    "E2M1_MAX",
    "dequant_k32",
    "e2m1_decode",
    "e2m1_encode",
    "unpack_e2m1",
    "router_ref",
]
