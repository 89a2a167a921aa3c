"""1x128 FP8 group quantisation (activations and the SwiGLU output).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

FlashInfer PR #4287 takes activations as E4M3 codes "[M, K]" with one FP32
scale per token and 128-column group (public-contract section; the retained
measurements section repeats that activation groups are 128 wide), and
requantises the SwiGLU output to FP8 per token (PR summary).  Its review of the
zero-activation scale adds the floor: the decoded scale is clamped to FLT_MIN
before it is inverted, so an all-zero group yields zero codes instead of
0 * infinity, and every non-zero group keeps the ordinary scale.

Scale formula (the reading taken; the pages print amax/448 only for the weight
block scales, and the same rule is used for every group here):
  FP32 mode   s   = max(fl32(amax / 448), FLT_MIN)
              inv = fl32(1 / s)
              code = E4M3(fl32(v * inv))
  UE8M0 mode  (SGLang PR #43556, motivation and modifications: scales rounded
              up to powers of two) s = 2^e with e the least integer such that
              448 * 2^e >= amax, floored at -126; code = E4M3(v * 2^-e), exact.
Both divisions are IEEE FP32 divisions; v is the FP32 value of the input.
"""

import numpy as np

from .e4m3 import FLT_MIN, e4m3_encode

SCALE_FP32 = 0
SCALE_UE8M0 = 1


def ue8m0_exponent(amax):
    """Least integer e with 448 * 2^e >= amax, floored at -126 (exact).

    With amax = f * 2^x, f in [0.5, 1), and 448 = 0.875 * 2^9:
    448 * 2^(x-9) >= amax  <=>  f <= 0.875, else x - 8 is the least exponent.
    """
    a = np.asarray(amax, dtype=np.float64)
    f, x = np.frexp(a)
    e = np.where(f <= 0.875, x - 9, x - 8).astype(np.int64)
    e = np.where(a == 0.0, -126, e)
    return np.maximum(e, -126)


def quant_groups_ref(v, scale_mode=SCALE_FP32):
    """Quantise float32 values [..., G*128] in groups of 128 along the last
    axis.  Returns (codes uint8 [..., G*128], scales float32 [..., G])."""
    v = np.asarray(v, dtype=np.float32)
    shp = v.shape
    assert shp[-1] % 128 == 0
    g = v.reshape(shp[:-1] + (shp[-1] // 128, 128))
    amax = np.max(np.abs(g), axis=-1)                       # exact
    if scale_mode == SCALE_FP32:
        s = np.maximum(amax / np.float32(448.0), FLT_MIN).astype(np.float32)
        inv = (np.float32(1.0) / s).astype(np.float32)
        q = (g * inv[..., None]).astype(np.float32)          # one fp32 rounding
    elif scale_mode == SCALE_UE8M0:
        e = ue8m0_exponent(amax)
        s = np.ldexp(np.float32(1.0), e.astype(np.int32)).astype(np.float32)
        q = np.ldexp(g.astype(np.float64), (-e)[..., None].astype(np.int32))
    else:
        raise ValueError("unknown scale mode")
    codes = e4m3_encode(q).reshape(shp)
    return codes, s


def quant_act_ref(x, scale_mode=SCALE_FP32):
    """Activation quantisation of x (BF16 values given as float32, [M, K])."""
    x = np.asarray(x, dtype=np.float32)
    assert x.ndim == 2 and x.shape[1] % 128 == 0
    return quant_groups_ref(x, scale_mode)
