"""Python binding of libmoe_fp8.so, the MI355X (gfx950) routed FP8 W8A8
block-scale MoE expert path.

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch tensors used for their device memory (``data_ptr()``) and
the current HIP stream; nothing here computes any part of the path.  The
functions carry the C ABI's names (see include/moe_fp8.h) and raise
``MoeError`` on a non-OK status.  If the shared library has not been built,
importing this package raises -- there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp8.so")

MOE_OK = 0
MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_CAPACITY, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = \
    1, 2, 3, 4, 5, 6
MOE_IDS_I32, MOE_IDS_I64 = 0, 1
MOE_SCALE_FP32, MOE_SCALE_UE8M0 = 0, 1
MOE_F_INTER_UE8M0 = 1
MOE_F_MMA_E8M0 = 2
MOE_F_FP8_GATEUP = 4
MOE_F_SPLITK_SHIFT = 8
MOE_F_GATEUP_PATH_SHIFT = 16
MOE_F_DOWN_PATH_SHIFT = 18
MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_PERSISTENT, MOE_PATH_COLUMNS = 0, 1, 2, 3
MOE_F_FUSE_SHIFT = 20
MOE_F_W13_PACKED = 0x400000
MOE_FUSE_AUTO, MOE_FUSE_OFF, MOE_FUSE_ON = 0, 1, 2

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN",
                4: "MOE_ERR_CAPACITY", 5: "MOE_ERR_UNSUPPORTED", 6: "MOE_ERR_HIP"}

EXPORTED = ("moe_plan_capacity", "moe_plan_workspace_size", "moe_plan", "moe_quant_act",
            "moe_plan_quant",
            "moe_fp8_experts_workspace_size", "moe_fp8_experts_workspace_layout",
            "moe_fp8_experts_schedule",
            "moe_fp8_experts", "moe_fp8_gate_up", "moe_fp8_down_reduce", "moe_status_str",
            "moe_last_hip_error", "moe_last_error", "moe_debug_e4m3_encode",
            "moe_debug_count_non_pow2", "moe_fp8_experts_noalloc", "moe_route_plan",
            "moe_w4a8_experts_workspace_size", "moe_w4a8_experts", "moe_prepack_w13_size",
            "moe_prepack_w13", "moe_fp8_layer")

MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeError(RuntimeError):
    def __init__(self, status, where, detail):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {detail}")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(or python fp8_block_scale_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

_i32, _i64, _u32, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p
_pi64, _psz = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_size_t)


def _proto(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_c = {
    "moe_plan_capacity": _proto("moe_plan_capacity", _i32, _i64, _i32, _i32, _i32, _pi64, _pi64),
    "moe_plan_workspace_size": _proto("moe_plan_workspace_size", _sz, _i64, _i32, _i32, _i32),
    "moe_plan": _proto("moe_plan", _i32, _vp, _i32, _i64, _i32, _i32, _i32, _vp, _i64, _vp, _i64,
                       _vp, _vp, _sz, _vp),
    "moe_quant_act": _proto("moe_quant_act", _i32, _vp, _i64, _i64, _i64, _vp, _vp, _i32, _vp),
    "moe_route_plan": _proto("moe_route_plan", _i32, _vp, _i64, _i32, _i32, _i32, ctypes.c_float, _i32,
                             _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _sz, _vp, _i64, _i64, _vp,
                             _vp, _i32, _vp),
    "moe_plan_quant": _proto("moe_plan_quant", _i32, _vp, _i32, _i64, _i32, _i32, _i32, _vp, _i64, _vp,
                             _i64, _vp, _vp, _sz, _vp, _i64, _i64, _vp, _vp, _i32, _vp),
    "moe_fp8_experts_workspace_size": _proto("moe_fp8_experts_workspace_size", _sz, _i64, _i64,
                                             _i64, _i32, _i32, _i32, _i64, _u32),
    "moe_fp8_experts_workspace_layout": _proto("moe_fp8_experts_workspace_layout", _i32, _i64, _i64,
                                               _i64, _i32, _i32, _i32, _i64, _u32, _psz, _psz),
    "moe_fp8_experts_schedule": _proto("moe_fp8_experts_schedule", _i32, _i64, _i64, _i64, _i32,
                                       _i32, _i32, _i64, _u32, _vp),
    "moe_fp8_experts": _proto("moe_fp8_experts", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i64, _u32, _vp, _vp, _sz,
                              _vp),
    "moe_fp8_layer": _proto("moe_fp8_layer", _i32, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _vp, _vp,
                            _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp, _i64, _vp, _i64, _vp,
                            _vp, _vp, _vp, _sz, _u32, _vp, _vp, _sz, _vp),
    "moe_fp8_gate_up": _proto("moe_fp8_gate_up", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                              _i64, _i32, _i32, _i32, _i64, _u32, _vp, _sz, _vp),
    "moe_fp8_down_reduce": _proto("moe_fp8_down_reduce", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                  _i64, _i64, _i32, _i32, _i32, _i64, _u32, _vp, _vp, _sz, _vp),
    "moe_fp8_experts_noalloc": _proto("moe_fp8_experts_noalloc", _i32, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32,
                                      _i32, _i64, _u32, _vp, _vp),
    "moe_w4a8_experts_workspace_size": _proto("moe_w4a8_experts_workspace_size", _sz, _i64, _i64,
                                              _i64, _i32, _i32, _i32, _i64, _u32),
    "moe_w4a8_experts": _proto("moe_w4a8_experts", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i64, _u32, _vp, _vp,
                               _sz, _vp),
    "moe_prepack_w13_size": _proto("moe_prepack_w13_size", _sz, _i64, _i64, _i64),
    "moe_prepack_w13": _proto("moe_prepack_w13", _i32, _vp, _i64, _i64, _i64, _vp, _vp),
    "moe_status_str": _proto("moe_status_str", ctypes.c_char_p, _i32),
    "moe_last_hip_error": _proto("moe_last_hip_error", ctypes.c_char_p),
    "moe_last_error": _proto("moe_last_error", ctypes.c_char_p),
    "moe_debug_e4m3_encode": _proto("moe_debug_e4m3_encode", _i32, _vp, _vp, _i64, _vp),
    "moe_debug_count_non_pow2": _proto("moe_debug_count_non_pow2", _i32, _vp, _i64, _vp, _vp),
}


def _check(st, where):
    if st != MOE_OK:
        raise MoeError(st, where, _c["moe_last_hip_error"]().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------ plan --

def moe_plan_capacity(M, top_k, E, block_m):
    sc, bc = ctypes.c_int64(), ctypes.c_int64()
    _check(_c["moe_plan_capacity"](M, top_k, E, block_m, ctypes.byref(sc), ctypes.byref(bc)),
           "moe_plan_capacity")
    return sc.value, bc.value


def moe_plan_workspace_size(M, top_k, E, block_m):
    return _c["moe_plan_workspace_size"](M, top_k, E, block_m)


def _plan_args(topk_ids, E, block_m, sorted_token_ids, expert_ids, num_tokens_post_padded,
               workspace):
    M, top_k = topk_ids.shape
    if topk_ids.dtype == torch.int32:
        dt = MOE_IDS_I32
    elif topk_ids.dtype == torch.int64:
        dt = MOE_IDS_I64
    else:
        raise TypeError("topk_ids must be int32 or int64")
    assert topk_ids.is_contiguous() and sorted_token_ids.dtype == torch.int32
    assert expert_ids.dtype == torch.int32 and num_tokens_post_padded.dtype == torch.int32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(topk_ids), dt, M, top_k, E, block_m, _ptr(sorted_token_ids), sorted_token_ids.numel(),
            _ptr(expert_ids), expert_ids.numel(), _ptr(num_tokens_post_padded), _ptr(workspace),
            ws_bytes)


def _quant_args(x_bf16, x_q, x_s):
    assert x_bf16.dtype == torch.bfloat16 and x_bf16.dim() == 2 and x_bf16.stride(1) == 1
    M, K = x_bf16.shape
    assert x_q.dtype == torch.uint8 and x_q.is_contiguous() and tuple(x_q.shape) == (M, K)
    assert x_s.dtype == torch.float32 and x_s.is_contiguous() and tuple(x_s.shape) == (M, K // 128)
    return M, K, x_bf16.stride(0)


def moe_plan(topk_ids, E, block_m, sorted_token_ids, expert_ids, num_tokens_post_padded,
             workspace=None, stream=None):
    """topk_ids [M, top_k] int32/int64 (device); outputs are preallocated int32 tensors."""
    args = _plan_args(topk_ids, E, block_m, sorted_token_ids, expert_ids, num_tokens_post_padded,
                      workspace)
    _check(_c["moe_plan"](*args, _stream(stream)), "moe_plan")


def moe_plan_quant(topk_ids, E, block_m, sorted_token_ids, expert_ids, num_tokens_post_padded,
                   x_bf16, x_q, x_s, scale_mode=MOE_SCALE_FP32, workspace=None, stream=None):
    """moe_plan and moe_quant_act in one call (one launch fewer); same outputs."""
    args = _plan_args(topk_ids, E, block_m, sorted_token_ids, expert_ids, num_tokens_post_padded,
                      workspace)
    M, K, ld = _quant_args(x_bf16, x_q, x_s)
    assert M == topk_ids.shape[0], "x_bf16 and topk_ids disagree on M"
    _check(_c["moe_plan_quant"](*args, _ptr(x_bf16), K, ld, _ptr(x_q), _ptr(x_s), scale_mode,
                                _stream(stream)), "moe_plan_quant")


def moe_route_plan(router_logits, top_k, n_shared, routed_scaling, block_m, topk_ids,
                   topk_weights, sorted_token_ids, expert_ids, num_tokens_post_padded,
                   workspace=None, x_bf16=None, x_q=None, x_s=None, scale_mode=MOE_SCALE_FP32,
                   stream=None):
    """Router (softmax top-k, routed scaling, optional shared expert) and the
    plan in the plan's launches; with x_bf16 also the activation quantisation.
    router_logits [M, E_routed] fp32; topk_ids int32 / topk_weights fp32
    [M, top_k + n_shared] out; the plan buffers sized for E_routed + n_shared
    experts and top_k + n_shared routes per token."""
    assert router_logits.dtype == torch.float32 and router_logits.is_contiguous()
    M, Er = router_logits.shape
    kk = top_k + n_shared
    assert topk_ids.dtype == torch.int32 and topk_ids.is_contiguous() and tuple(topk_ids.shape) == (M, kk)
    assert topk_weights.dtype == torch.float32 and topk_weights.is_contiguous()
    assert tuple(topk_weights.shape) == (M, kk)
    assert sorted_token_ids.dtype == torch.int32 and expert_ids.dtype == torch.int32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if x_bf16 is not None:
        Mx, K, ld = _quant_args(x_bf16, x_q, x_s)
        assert Mx == M, "x_bf16 and router_logits disagree on M"
    else:
        K, ld = 0, 0
    _check(_c["moe_route_plan"](_ptr(router_logits), M, Er, top_k, n_shared, routed_scaling, block_m,
                                _ptr(topk_ids), _ptr(topk_weights), _ptr(sorted_token_ids),
                                sorted_token_ids.numel(), _ptr(expert_ids), expert_ids.numel(),
                                _ptr(num_tokens_post_padded), _ptr(workspace), ws_bytes,
                                _ptr(x_bf16), K, ld, _ptr(x_q), _ptr(x_s), scale_mode,
                                _stream(stream)), "moe_route_plan")


# ------------------------------------------------------------- quant act --

def moe_quant_act(x_bf16, x_q, x_s, scale_mode=MOE_SCALE_FP32, stream=None):
    """x_bf16 [M, K] bf16 (row stride may exceed K); x_q uint8 [M, K]; x_s fp32 [M, K/128]."""
    M, K, ld = _quant_args(x_bf16, x_q, x_s)
    _check(_c["moe_quant_act"](_ptr(x_bf16), M, K, ld, _ptr(x_q), _ptr(x_s), scale_mode,
                               _stream(stream)), "moe_quant_act")


def moe_debug_e4m3_encode(inp, out, stream=None):
    assert inp.dtype == torch.float32 and out.dtype == torch.uint8 and inp.numel() == out.numel()
    _check(_c["moe_debug_e4m3_encode"](_ptr(inp), _ptr(out), inp.numel(), _stream(stream)),
           "moe_debug_e4m3_encode")


def moe_debug_count_non_pow2(scales, count, stream=None):
    """count[0] = how many of `scales` (FP32, device) are not powers of two in
    [2^-126, 2^127] -- the values MOE_F_MMA_E8M0 cannot take as they are."""
    assert scales.dtype == torch.float32 and scales.is_contiguous()
    assert count.dtype in (torch.int32, torch.uint32) and count.numel() >= 1
    _check(_c["moe_debug_count_non_pow2"](_ptr(scales), scales.numel(), _ptr(count), _stream(stream)),
           "moe_debug_count_non_pow2")


# --------------------------------------------------------------- experts --

def moe_fp8_experts_workspace_size(M, K, I, E, top_k, block_m, sorted_cap, flags=0):
    return _c["moe_fp8_experts_workspace_size"](M, K, I, E, top_k, block_m, sorted_cap, flags)


def moe_fp8_experts_workspace_layout(M, K, I, E, top_k, block_m, sorted_cap, flags=0):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_c["moe_fp8_experts_workspace_layout"](M, K, I, E, top_k, block_m, sorted_cap, flags,
                                                  ctypes.byref(a), ctypes.byref(b)),
           "moe_fp8_experts_workspace_layout")
    return a.value, b.value


def moe_fp8_experts_schedule(M, K, I, E, top_k, block_m, sorted_cap, flags=0):
    """(gate/up kernel (0 per block, 1 persistent, 2 split over intermediate-column
    slices), down kernel (0 per block, 1 persistent, 2 split over output columns),
    split-K factor, K-blocks per split, steps 3-5 as one launch)."""
    info = (ctypes.c_int32 * 5)()
    _check(_c["moe_fp8_experts_schedule"](M, K, I, E, top_k, block_m, sorted_cap, flags, info),
           "moe_fp8_experts_schedule")
    return int(info[0]), int(info[1]), int(info[2]), int(info[3]), bool(info[4])


def moe_fp8_layer(x_bf16, topk_ids, topk_weights, w13, w13_s, w2, w2_s, block_m, sorted_token_ids,
                  expert_ids, num_tokens_post_padded, x_q, x_s, out_bf16, workspace, flags=0,
                  scale_mode=MOE_SCALE_FP32, plan_workspace=None, stream=None):
    """All five steps (moe_plan_quant then moe_fp8_experts) in one call, with
    one launch fewer at decode sizes; same outputs."""
    pa = _plan_args(topk_ids, w13.shape[0], block_m, sorted_token_ids, expert_ids,
                    num_tokens_post_padded, plan_workspace)
    ids_ptr, dt, M, top_k, E, _, s_ptr, s_cap, e_ptr, e_cap, n_ptr, pw_ptr, pw_bytes = pa
    Mx, K, ld = _quant_args(x_bf16, x_q, x_s)
    assert Mx == M, "x_bf16 and topk_ids disagree on M"
    I = w13.shape[1] // 2
    for t in (w13, w13_s, w2, w2_s, topk_weights, out_bf16, workspace):
        assert t.is_contiguous()
    assert out_bf16.dtype == torch.bfloat16 and topk_weights.dtype == torch.float32
    _check(_c["moe_fp8_layer"](_ptr(x_bf16), ld, scale_mode, ids_ptr, dt, _ptr(topk_weights),
                               _ptr(w13), _ptr(w13_s), _ptr(w2), _ptr(w2_s), M, K, I, E, top_k,
                               block_m, s_ptr, s_cap, e_ptr, e_cap, n_ptr, _ptr(x_q), _ptr(x_s),
                               pw_ptr, pw_bytes, flags, _ptr(out_bf16), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_fp8_layer")


def moe_fp8_experts(x_q, x_s, w13, w13_s, w2, w2_s, topk_weights, sorted_token_ids, expert_ids,
                    num_tokens_post_padded, top_k, block_m, out_bf16, workspace, flags=0,
                    stream=None):
    """Steps 3-5; accumulates into out_bf16 [M, K]."""
    M, K = x_q.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    for t in (x_q, x_s, w13, w13_s, w2, w2_s, topk_weights, sorted_token_ids, expert_ids,
              out_bf16, workspace):
        assert t.is_contiguous()
    assert out_bf16.dtype == torch.bfloat16 and topk_weights.dtype == torch.float32
    # the kernels read expert ids of blocks below P only; P / block_m is at
    # most the plan's block capacity and at most sorted_cap / block_m
    assert expert_ids.numel() >= min(moe_plan_capacity(M, top_k, E, block_m)[1],
                                     sorted_token_ids.numel() // block_m), \
        "expert_ids shorter than the plan can need"
    _check(_c["moe_fp8_experts"](_ptr(x_q), _ptr(x_s), _ptr(w13), _ptr(w13_s), _ptr(w2),
                                 _ptr(w2_s), _ptr(topk_weights), _ptr(sorted_token_ids),
                                 _ptr(expert_ids), _ptr(num_tokens_post_padded), M, K, I, E, top_k,
                                 block_m, sorted_token_ids.numel(), flags, _ptr(out_bf16),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)),
           "moe_fp8_experts")


def moe_prepack_w13_size(E, I, K):
    return _c["moe_prepack_w13_size"](E, I, K)


def moe_prepack_w13(w13, out=None, stream=None):
    """W13 [E, 2I, K] uint8 -> its packed tile layout (a new uint8 tensor of
    the same size unless `out` is given); pass MOE_F_W13_PACKED with it."""
    E, twoI, K = w13.shape
    assert w13.dtype == torch.uint8 and w13.is_contiguous()
    if out is None:
        out = torch.empty(moe_prepack_w13_size(E, twoI // 2, K), dtype=torch.uint8,
                          device=w13.device)
    assert out.is_contiguous() and out.numel() == moe_prepack_w13_size(E, twoI // 2, K)
    _check(_c["moe_prepack_w13"](_ptr(w13), E, twoI // 2, K, _ptr(out), _stream(stream)),
           "moe_prepack_w13")
    return out.view(E, twoI, K)


def moe_w4a8_experts_workspace_size(M, K, I, E, top_k, block_m, sorted_cap, flags=0):
    return _c["moe_w4a8_experts_workspace_size"](M, K, I, E, top_k, block_m, sorted_cap, flags)


def moe_w4a8_experts(x_q, x_s, w13, w13_e, w2, w2_e, topk_weights, sorted_token_ids, expert_ids,
                     num_tokens_post_padded, top_k, block_m, out_bf16, workspace, flags=0,
                     stream=None):
    """Steps 3-5 with E2M1 weights (w13 [E, 2I, K/2], w13_e [E, 2I, K/32],
    w2 [E, K, I/2], w2_e [E, K, I/32], all uint8); accumulates into
    out_bf16 [M, K]."""
    M, K = x_q.shape
    E, twoI, half = w13.shape
    I = twoI // 2
    assert 2 * half == K and w2.shape == (E, K, I // 2)
    assert w13_e.shape == (E, twoI, K // 32) and w2_e.shape == (E, K, I // 32)
    for t in (x_q, x_s, w13, w13_e, w2, w2_e, topk_weights, sorted_token_ids, expert_ids,
              out_bf16, workspace):
        assert t.is_contiguous()
    assert w13.dtype == w13_e.dtype == w2.dtype == w2_e.dtype == torch.uint8
    assert out_bf16.dtype == torch.bfloat16 and topk_weights.dtype == torch.float32
    assert expert_ids.numel() >= min(moe_plan_capacity(M, top_k, E, block_m)[1],
                                     sorted_token_ids.numel() // block_m), \
        "expert_ids shorter than the plan can need"
    _check(_c["moe_w4a8_experts"](_ptr(x_q), _ptr(x_s), _ptr(w13), _ptr(w13_e), _ptr(w2),
                                  _ptr(w2_e), _ptr(topk_weights), _ptr(sorted_token_ids),
                                  _ptr(expert_ids), _ptr(num_tokens_post_padded), M, K, I, E, top_k,
                                  block_m, sorted_token_ids.numel(), flags, _ptr(out_bf16),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)),
           "moe_w4a8_experts")


def moe_fp8_experts_noalloc(x_q, x_s, w13, w13_s, w2, w2_s, topk_weights, sorted_token_ids,
                            expert_ids, num_tokens_post_padded, top_k, block_m, out_bf16, flags=0,
                            stream=None):
    """moe_fp8_experts with the library's static per-device scratch as the
    workspace (no allocation anywhere); raises MoeError (MOE_ERR_CAPACITY)
    for sizes whose workspace exceeds MOE_NOALLOC_SCRATCH_BYTES."""
    M, K = x_q.shape
    E, twoI, _ = w13.shape
    for t in (x_q, x_s, w13, w13_s, w2, w2_s, topk_weights, sorted_token_ids, expert_ids,
              out_bf16):
        assert t.is_contiguous()
    assert out_bf16.dtype == torch.bfloat16 and topk_weights.dtype == torch.float32
    _check(_c["moe_fp8_experts_noalloc"](_ptr(x_q), _ptr(x_s), _ptr(w13), _ptr(w13_s), _ptr(w2),
                                         _ptr(w2_s), _ptr(topk_weights), _ptr(sorted_token_ids),
                                         _ptr(expert_ids), _ptr(num_tokens_post_padded), M, K,
                                         twoI // 2, E, top_k, block_m, sorted_token_ids.numel(),
                                         flags, _ptr(out_bf16), _stream(stream)),
           "moe_fp8_experts_noalloc")


def moe_fp8_gate_up(x_q, x_s, w13, w13_s, sorted_token_ids, expert_ids, num_tokens_post_padded,
                    top_k, block_m, workspace, flags=0, stream=None):
    """Steps 3-4 into the workspace (see MoeLayerBuffers.intermediate)."""
    M, K = x_q.shape
    E, twoI, _ = w13.shape
    _check(_c["moe_fp8_gate_up"](_ptr(x_q), _ptr(x_s), _ptr(w13), _ptr(w13_s), _ptr(sorted_token_ids),
                                 _ptr(expert_ids), _ptr(num_tokens_post_padded), M, K, twoI // 2, E,
                                 top_k, block_m, sorted_token_ids.numel(), flags, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_fp8_gate_up")


def moe_fp8_down_reduce(w2, w2_s, topk_weights, sorted_token_ids, expert_ids,
                        num_tokens_post_padded, top_k, block_m, out_bf16, workspace, flags=0,
                        stream=None):
    """Step 5: out_bf16 += weighted down projections of the workspace rows."""
    E, K, I = w2.shape
    M = out_bf16.shape[0]
    _check(_c["moe_fp8_down_reduce"](_ptr(w2), _ptr(w2_s), _ptr(topk_weights), _ptr(sorted_token_ids),
                                     _ptr(expert_ids), _ptr(num_tokens_post_padded), M, K, I, E,
                                     top_k, block_m, sorted_token_ids.numel(), flags,
                                     _ptr(out_bf16), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_fp8_down_reduce")


def moe_status_str(status):
    return _c["moe_status_str"](status).decode()


def moe_last_hip_error():
    return _c["moe_last_hip_error"]().decode()


moe_last_error = moe_last_hip_error


# ------------------------------------------------------------- a layer --

class MoeLayerBuffers:
    """Device buffers for one call of the whole path at a given geometry
    (allocated once with torch; reused across calls)."""

    def __init__(self, M, K, I, E, top_k, block_m, flags=0, device="cuda", w4a8=False):
        self.M, self.K, self.I, self.E, self.top_k, self.block_m = M, K, I, E, top_k, block_m
        self.flags = flags
        self.w4a8 = w4a8
        self.sorted_cap, self.blocks_cap = moe_plan_capacity(M, top_k, E, block_m)
        dev = torch.device(device)
        self.sorted_ids = torch.empty(self.sorted_cap, dtype=torch.int32, device=dev)
        self.expert_ids = torch.empty(self.blocks_cap, dtype=torch.int32, device=dev)
        self.ntp = torch.empty(1, dtype=torch.int32, device=dev)
        self.x_q = torch.empty((M, K), dtype=torch.uint8, device=dev)
        self.x_s = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
        size = moe_w4a8_experts_workspace_size if w4a8 else moe_fp8_experts_workspace_size
        ws = size(M, K, I, E, top_k, block_m, self.sorted_cap, flags)
        if w4a8 and M > 0 and ws == 0:
            raise MoeError(MOE_ERR_SHAPE, "moe_w4a8_experts_workspace_size", moe_last_hip_error())
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        pws = moe_plan_workspace_size(M, top_k, E, block_m)
        self.plan_ws = torch.empty(pws, dtype=torch.uint8, device=dev) if pws else None
        self.h_q_off, self.h_s_off = moe_fp8_experts_workspace_layout(
            M, K, I, E, top_k, block_m, self.sorted_cap, flags)

    def intermediate(self):
        """(h_q [sorted_cap, I] uint8, h_s [sorted_cap, I/128] fp32) views of the workspace."""
        n_q = self.sorted_cap * self.I
        n_s = self.sorted_cap * (self.I // 128)
        hq = self.workspace[self.h_q_off:self.h_q_off + n_q].view(self.sorted_cap, self.I)
        hs = self.workspace[self.h_s_off:self.h_s_off + 4 * n_s].view(torch.float32)
        return hq, hs.view(self.sorted_cap, self.I // 128)


def moe_layer(bufs, x_bf16, topk_ids, topk_weights, w13, w13_s, w2, w2_s, out_bf16,
              act_scale_mode=MOE_SCALE_FP32, stream=None):
    """All five steps on one stream (moe_fp8_layer: plan with activation
    quantisation, experts)."""
    moe_fp8_layer(x_bf16, topk_ids, topk_weights, w13, w13_s, w2, w2_s, bufs.block_m,
                  bufs.sorted_ids, bufs.expert_ids, bufs.ntp, bufs.x_q, bufs.x_s, out_bf16,
                  bufs.workspace, bufs.flags, act_scale_mode, bufs.plan_ws, stream)
