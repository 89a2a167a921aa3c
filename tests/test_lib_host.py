"""Library loads, exports every symbol include/moe_fp8.h declares, and its host
validation rejects bad arguments before launching anything (CPU only: no
call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe_fp8.h")

import fp8_block_scale_amd as moe  # noqa: E402


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", txt)))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) >= 10
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe_fp8.h but not exported"
    assert set(names) == set(moe.EXPORTED)


def test_no_internal_symbols_exported():
    # the library is built with hidden visibility: only the C ABI is public
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in ("launch_plan", "_ZN3moe11launch_planEPKvbliiiPiS2_S2_P12ihipStream_t"):
        assert not hasattr(lib, n)


def test_status_strings():
    for s in range(7):
        assert moe.moe_status_str(s).startswith(moe.STATUS_NAMES[s])


def test_plan_capacity_values():
    assert moe.moe_plan_capacity(4, 2, 8, 16) == (128, 8)
    assert moe.moe_plan_capacity(1, 9, 257, 16) == (144, 9)
    assert moe.moe_plan_capacity(4096, 8, 288, 64) == (50944, 796)
    assert moe.moe_plan_capacity(2048, 10, 512, 64) == (52736, 824)
    assert moe.moe_plan_capacity(8192, 8, 288, 128) == (102144, 798)
    assert moe.moe_plan_capacity(0, 8, 288, 128) == (0, 0)


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first


def _raw(name):
    return moe._c[name]


def _err(st):
    return moe.STATUS_NAMES[st]


def test_plan_validation():
    f = _raw("moe_plan")
    args = dict(ids=FAKE, dt=0, M=4, k=2, E=8, bm=16, s=FAKE, sc=128, x=FAKE, bc=8, p=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["ids"], a["dt"], a["M"], a["k"], a["E"], a["bm"], a["s"], a["sc"], a["x"],
                 a["bc"], a["p"], None, 0, None)

    assert _err(call(sc=127)) == "MOE_ERR_CAPACITY"
    assert _err(call(bc=7)) == "MOE_ERR_CAPACITY"
    assert _err(call(sc=128, bc=9)) == "MOE_ERR_CAPACITY"     # sorted_cap < blocks_cap * block_m
    assert _err(call(dt=2)) == "MOE_ERR_SHAPE"
    assert _err(call(E=0)) == "MOE_ERR_SHAPE"
    assert _err(call(E=1025)) == "MOE_ERR_UNSUPPORTED"
    assert _err(call(bm=257)) == "MOE_ERR_UNSUPPORTED"
    assert _err(call(M=-1)) == "MOE_ERR_SHAPE"
    assert _err(call(p=None)) == "MOE_ERR_NULL"
    assert _err(call(ids=None)) == "MOE_ERR_NULL"
    assert _err(call(M=1 << 28, k=8)) == "MOE_ERR_SHAPE"     # R overflows int32
    assert "capacity" in moe.moe_last_error() or "int32" in moe.moe_last_error()


def test_quant_validation():
    f = _raw("moe_quant_act")
    assert _err(f(FAKE, 4, 100, 100, FAKE, FAKE, 0, None)) == "MOE_ERR_SHAPE"    # K % 128
    assert _err(f(FAKE, 4, 256, 128, FAKE, FAKE, 0, None)) == "MOE_ERR_SHAPE"    # ld < K
    assert _err(f(FAKE, 4, 256, 260, FAKE, FAKE, 0, None)) == "MOE_ERR_ALIGN"    # ld % 8
    assert _err(f(ctypes.c_void_p(0x10008), 4, 256, 256, FAKE, FAKE, 0, None)) == "MOE_ERR_ALIGN"
    assert _err(f(FAKE, 4, 256, 256, FAKE, FAKE, 7, None)) == "MOE_ERR_SHAPE"    # scale mode
    assert _err(f(None, 4, 256, 256, FAKE, FAKE, 0, None)) == "MOE_ERR_NULL"
    assert _err(f(None, 0, 256, 256, None, None, 0, None)) == "MOE_OK"           # M = 0: no work


def test_experts_validation():
    f = _raw("moe_fp8_experts")
    base = dict(M=4, K=256, I=256, E=8, k=2, bm=16, sc=128, fl=0, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(base, **kw)
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["M"], a["K"], a["I"],
                 a["E"], a["k"], a["bm"], a["sc"], a["fl"], FAKE, a["ws"], a["wsb"], None)

    assert _err(call(K=200)) == "MOE_ERR_SHAPE"
    assert _err(call(I=100)) == "MOE_ERR_SHAPE"
    assert _err(call(bm=4)) == "MOE_ERR_UNSUPPORTED"
    assert _err(call(bm=48)) == "MOE_ERR_UNSUPPORTED"
    assert _err(call(sc=120)) == "MOE_ERR_SHAPE"
    assert _err(call(fl=moe.MOE_F_MMA_E8M0)) == "MOE_ERR_SHAPE"
    assert _err(call(fl=1 << 24)) == "MOE_ERR_SHAPE"                          # unknown bit
    assert _err(call(fl=3 << moe.MOE_F_FUSE_SHIFT)) == "MOE_ERR_SHAPE"        # fuse choice 3
    assert _err(call(wsb=16)) == "MOE_ERR_CAPACITY"
    assert _err(call(ws=None)) == "MOE_ERR_NULL"
    assert _err(call(ws=ctypes.c_void_p(0x10010))) == "MOE_ERR_ALIGN"
    assert _err(call(M=0)) == "MOE_OK"


def test_workspace_size_monotone_and_layout():
    a = moe.moe_fp8_experts_workspace_size(4096, 4096, 1024, 288, 8, 64, 50944)
    b = moe.moe_fp8_experts_workspace_size(8192, 4096, 1024, 288, 8, 64, 83712)
    assert 0 < a < b
    hq, hs = moe.moe_fp8_experts_workspace_layout(4096, 4096, 1024, 288, 8, 64, 50944)
    assert hq % 256 == 0 and hs % 256 == 0 and hs >= hq + 50944 * 1024
    # forcing a split-K factor grows the workspace by the partial sums
    s1 = moe.moe_fp8_experts_workspace_size(4, 256, 256, 8, 2, 16, 128, 1 << 8)
    s2 = moe.moe_fp8_experts_workspace_size(4, 256, 256, 8, 2, 16, 128, 2 << 8)
    assert s2 > s1


def test_plan_workspace_size():
    # one-workgroup build below 4096 routes; above, one int32 per (workgroup of
    # ~1024 routes, at least 16 workgroups, expert)
    assert moe.moe_plan_workspace_size(1, 9, 257, 16) == 0
    assert moe.moe_plan_workspace_size(511, 8, 288, 64) == 0
    assert moe.moe_plan_workspace_size(512, 8, 288, 64) == 16 * 288 * 4
    assert moe.moe_plan_workspace_size(4096, 8, 288, 64) == 32 * 288 * 4
    # the scan keeps G * E + E + 16 ints in 64 KB of LDS
    assert moe.moe_plan_workspace_size(10 ** 6, 8, 64, 64) == 254 * 64 * 4
    assert moe.moe_plan_workspace_size(10 ** 6, 8, 1024, 64) == 14 * 1024 * 4
    assert moe.moe_plan_workspace_size(0, 8, 288, 64) == 0


def test_experts_schedule():
    """Kernel families per stage: the per-block gate/up while experts hold
    few routes on average, the persistent kernels for large grids; overrides
    and their validation."""
    sched = moe.moe_fp8_experts_schedule
    GU, DN = moe.MOE_F_GATEUP_PATH_SHIFT, moe.MOE_F_DOWN_PATH_SHIFT
    # decode: per-block gate/up; the split fills ~3/4 of the chip in one
    # round with the plan blocks expected under uniform routing: M=1 (~9
    # blocks x 2 column tiles) 10 ways of 6 K-blocks, M=4 (~34 blocks) 3
    # ways, M=16 (~112 blocks) no split.  The down stage splits the output
    # columns (route sum included) wherever that applies (I = 256, block_m
    # 8 or 16, at most 192 routes), else goes persistent once its
    # (block, 256-column) items reach twice the CU count
    COLS, PERS, BLOCK = 2, 1, 0
    assert sched(1, 7168, 256, 257, 9, 16, 144) == (False, COLS, 10, 6, False)
    assert sched(4, 7168, 256, 257, 9, 16, 576)[2:4] == (3, 19)
    assert sched(16, 7168, 256, 257, 9, 16, 2304)[2] == 1
    assert sched(4, 7168, 256, 257, 9, 16, 576)[:2] == (False, COLS)
    assert sched(16, 7168, 256, 257, 9, 16, 2304)[:2] == (False, COLS)
    assert sched(21, 7168, 256, 257, 9, 8, 2304)[1] == COLS          # 189 routes
    # the tiny workload (K = 256, 8 routes): the column-slice gate/up too
    assert sched(4, 256, 256, 8, 2, 16, 128)[:3] == (2, COLS, 1)
    assert sched(4, 256, 256, 8, 2, 16, 128, 1 << GU)[:2] == (0, COLS)
    assert sched(32, 7168, 256, 257, 9, 16, 4608)[:2] == (False, PERS)  # 288 routes
    assert sched(16, 7168, 256, 257, 9, 32, 4608)[1] == PERS         # block_m 32
    # forced: the per-block or the persistent down; the column split past
    # 192 routes is refused
    assert sched(16, 7168, 256, 257, 9, 16, 2304, 1 << DN)[1] == BLOCK
    assert sched(16, 7168, 256, 257, 9, 16, 2304, 2 << DN)[1] == PERS
    assert sched(32, 7168, 256, 257, 9, 16, 4608, 1 << DN)[1] == BLOCK
    with pytest.raises(moe.MoeError) as ei:                          # 216 routes
        sched(24, 7168, 256, 257, 9, 16, 4608, 3 << DN)
    assert moe.STATUS_NAMES[ei.value.status] == "MOE_ERR_UNSUPPORTED"
    # the column-slice gate/up (2): no split-K, with the column-split down
    # only; refused with another down path, FP8 products, packed W13 or a
    # forced split-K factor, and past 192 routes
    SLICES = 2
    assert sched(1, 7168, 256, 257, 9, 16, 144, 3 << GU)[:4] == (SLICES, COLS, 1, 56)
    assert sched(4, 7168, 256, 257, 9, 8, 576, (3 << GU) | (3 << DN))[:2] == (SLICES, COLS)
    for bad in ((3 << GU) | (1 << DN), (3 << GU) | (2 << DN), (3 << GU) | moe.MOE_F_FP8_GATEUP,
                (3 << GU) | moe.MOE_F_W13_PACKED, (3 << GU) | (4 << moe.MOE_F_SPLITK_SHIFT)):
        with pytest.raises(moe.MoeError) as ei:
            sched(1, 7168, 256, 257, 9, 16, 144, bad)
        assert moe.STATUS_NAMES[ei.value.status] == "MOE_ERR_SHAPE", hex(bad)
    with pytest.raises(moe.MoeError) as ei:
        sched(24, 7168, 256, 257, 9, 16, 4608, 3 << GU)
    assert moe.STATUS_NAMES[ei.value.status] == "MOE_ERR_UNSUPPORTED"
    # its FP32 rows take sorted_cap x I x 4 more bytes of workspace
    ws = moe.moe_fp8_experts_workspace_size
    assert ws(1, 7168, 256, 257, 9, 16, 144, 3 << GU) >= 144 * 256 * 4
    # page-1 M=16 and M=1024: per-block gate/up, persistent down
    assert sched(16, 4096, 1024, 288, 8, 64, 8192)[:2] == (False, True)
    assert sched(1024, 4096, 1024, 288, 8, 64, 26368)[:2] == (False, True)
    # page-1 M=4096 (the bench configuration): both persistent, no split, two launches
    assert sched(4096, 4096, 1024, 288, 8, 64, 50944) == (True, True, 1, 32, False)
    # steps 3-5 as one launch: only on request (the fuse field)
    FU = moe.MOE_F_FUSE_SHIFT
    assert sched(16, 7168, 256, 257, 9, 16, 2304)[4] is False
    assert sched(16, 7168, 256, 257, 9, 16, 2304, moe.MOE_FUSE_ON << FU)[4] is True
    assert sched(16, 7168, 256, 257, 9, 16, 2304, moe.MOE_FUSE_OFF << FU)[4] is False
    assert sched(4096, 4096, 1024, 288, 8, 64, 50944, moe.MOE_FUSE_ON << FU)[:2] == (False, False)
    assert sched(4096, 4096, 1024, 288, 8, 64, 50944, moe.MOE_FUSE_ON << FU)[4] is True
    assert sched(16, 4096, 1024, 288, 8, 64, 8192)[4] is False       # persistent down stage
    # overrides
    assert sched(16, 4096, 1024, 288, 8, 64, 8192, 2 << GU)[:2] == (True, True)
    assert sched(16, 4096, 1024, 288, 8, 64, 8192, 1 << DN)[:2] == (False, False)
    assert sched(4096, 4096, 1024, 288, 8, 64, 50944, (1 << GU) | (1 << DN))[:2] == (False, False)
    # a forced split-K factor selects the per-block gate/up
    assert sched(4096, 4096, 1024, 288, 8, 64, 50944, 2 << moe.MOE_F_SPLITK_SHIFT)[0] == 0
    for bad, status in ((3 << GU, "MOE_ERR_UNSUPPORTED"), (3 << DN, "MOE_ERR_UNSUPPORTED"),
                        ((2 << GU) | (2 << moe.MOE_F_SPLITK_SHIFT), "MOE_ERR_SHAPE"),
                        (1 << 24, "MOE_ERR_SHAPE"), (3 << FU, "MOE_ERR_SHAPE"),
                        ((2 << FU) | (2 << DN), "MOE_ERR_SHAPE")):
        with pytest.raises(moe.MoeError) as ei:
            sched(16, 4096, 1024, 288, 8, 64, 8192, bad)
        assert moe.STATUS_NAMES[ei.value.status] == status
    with pytest.raises(moe.MoeError):       # the persistent kernels need K <= 32768
        sched(16, 65536, 1024, 288, 8, 64, 8192, 2 << DN)
    with pytest.raises(moe.MoeError) as ei:  # the single launch's down rows fit in LDS
        sched(16, 4096, 8192, 288, 8, 64, 8192, moe.MOE_FUSE_ON << FU)
    assert moe.STATUS_NAMES[ei.value.status] == "MOE_ERR_UNSUPPORTED"


def test_plan_quant_validation():
    """moe_plan_quant validates both halves before launching anything."""
    f = _raw("moe_plan_quant")
    base = dict(ids=FAKE, dt=0, M=4, k=2, E=8, bm=16, s=FAKE, sc=128, e=FAKE, bc=8, p=FAKE,
                x=FAKE, K=256, ld=256, q=FAKE, qs=FAKE, mode=0)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["ids"], a["dt"], a["M"], a["k"], a["E"], a["bm"], a["s"], a["sc"], a["e"], a["bc"],
                 a["p"], None, 0, a["x"], a["K"], a["ld"], a["q"], a["qs"], a["mode"], None)

    assert _err(call(sc=127)) == "MOE_ERR_CAPACITY"
    assert _err(call(dt=2)) == "MOE_ERR_SHAPE"
    assert _err(call(K=200, ld=200)) == "MOE_ERR_SHAPE"
    assert _err(call(ld=128)) == "MOE_ERR_SHAPE"
    assert _err(call(mode=5)) == "MOE_ERR_SHAPE"
    assert _err(call(x=None)) == "MOE_ERR_NULL"
    assert _err(call(ld=260)) == "MOE_ERR_ALIGN"
    assert _err(call(p=None)) == "MOE_ERR_NULL"


def test_layer_validation():
    """moe_fp8_layer validates the plan, the quantisation and the experts
    arguments before launching anything (these calls run without a GPU)."""
    f = _raw("moe_fp8_layer")
    base = dict(x=FAKE, ld=256, mode=0, ids=FAKE, dt=0, w=FAKE, M=4, K=256, I=256, E=8, k=2, bm=16,
                s=FAKE, sc=128, e=FAKE, bc=8, p=FAKE, ws=FAKE, wsb=1 << 30, fl=0, out=FAKE)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["x"], a["ld"], a["mode"], a["ids"], a["dt"], a["w"], FAKE, FAKE, FAKE, FAKE,
                 a["M"], a["K"], a["I"], a["E"], a["k"], a["bm"], a["s"], a["sc"], a["e"], a["bc"],
                 a["p"], FAKE, FAKE, None, 0, a["fl"], a["out"], a["ws"], a["wsb"], None)

    assert _err(call(sc=127)) == "MOE_ERR_CAPACITY"             # plan
    assert _err(call(mode=5)) == "MOE_ERR_SHAPE"                # quantisation
    assert _err(call(x=None)) == "MOE_ERR_NULL"
    assert _err(call(wsb=16)) == "MOE_ERR_CAPACITY"             # experts workspace
    assert _err(call(w=None)) == "MOE_ERR_NULL"
    assert _err(call(out=None)) == "MOE_ERR_NULL"
    assert _err(call(I=200)) == "MOE_ERR_SHAPE"
    assert _err(call(fl=1 << 24)) == "MOE_ERR_SHAPE"


def test_noalloc_validation_before_any_device_call():
    """moe_fp8_experts_noalloc validates like moe_fp8_experts and rejects
    sizes whose workspace exceeds the static scratch, all before touching the
    device (these calls run without a GPU)."""
    f = _raw("moe_fp8_experts_noalloc")

    def call(M, K, I, E, k, bm, fl=0):
        sc = moe.moe_plan_capacity(M, k, E, bm)[0]
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, K, I, E, k, bm, sc,
                 fl, FAKE, None)

    assert _err(call(4096, 4096, 1024, 288, 8, 64)) == "MOE_ERR_CAPACITY"     # page-1 M=4096
    assert "static scratch" in moe.moe_last_hip_error()
    assert _err(call(4, 200, 256, 8, 2, 16)) == "MOE_ERR_SHAPE"
    assert _err(call(4, 256, 256, 8, 2, 48)) == "MOE_ERR_UNSUPPORTED"
    assert _err(call(4, 256, 256, 8, 2, 16, fl=moe.MOE_F_MMA_E8M0)) == "MOE_ERR_SHAPE"
    assert _err(call(0, 256, 256, 8, 2, 16)) == "MOE_OK"                      # M = 0: no work
    # the decode shapes fit the scratch
    for M in (1, 4, 16):
        sc = moe.moe_plan_capacity(M, 9, 257, 16)[0]
        need = moe.moe_fp8_experts_workspace_size(M, 7168, 256, 257, 9, 16, sc, 0)
        assert 0 < need <= moe.MOE_NOALLOC_SCRATCH_BYTES, (M, need)


def test_route_plan_validation():
    """moe_route_plan's host checks (no GPU needed: nothing is launched)."""
    f = _raw("moe_route_plan")

    def call(M=4, Er=8, k=2, ns=0, scale=1.0, bm=16, sc=None, bc=None, ws=None, wsb=0, x=None):
        try:
            scap, bcap = moe.moe_plan_capacity(M, k + ns, Er + ns, bm)
        except moe.MoeError:
            scap, bcap = 128, 8
        return f(FAKE, M, Er, k, ns, scale, bm, FAKE, FAKE, FAKE, scap if sc is None else sc, FAKE,
                 bcap if bc is None else bc, FAKE, ws, wsb, x, 256, 256, FAKE, FAKE, 0, None)

    assert _err(call(k=0)) == "MOE_ERR_SHAPE"
    assert _err(call(k=9)) == "MOE_ERR_SHAPE"                 # top_k > E_routed
    assert _err(call(Er=64, k=33)) == "MOE_ERR_SHAPE"         # top_k > 32
    assert _err(call(ns=2)) == "MOE_ERR_SHAPE"
    assert _err(call(Er=1024, k=8, ns=1)) == "MOE_ERR_SHAPE"  # 1025 experts
    assert _err(call(scale=float("inf"))) == "MOE_ERR_SHAPE"
    assert _err(call(sc=8)) == "MOE_ERR_CAPACITY"
    assert _err(call(x=ctypes.c_void_p(0x10008))) == "MOE_ERR_ALIGN"
    # 100000 routes need the plan workspace
    assert _err(call(M=20000, Er=256, k=4, ns=1)) == "MOE_ERR_CAPACITY"
    assert _err(call(M=0)) in ("MOE_OK", "MOE_ERR_HIP")      # M = 0: only the P fill


def test_w4a8_validation_before_any_device_call():
    """moe_w4a8_experts rejects what does not apply to E2M1 weights and bad
    shapes before touching the device (these calls run without a GPU)."""
    f = _raw("moe_w4a8_experts")
    base = dict(M=4, K=256, I=256, E=8, k=2, bm=16, sc=128, fl=0, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(base, **kw)
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["M"], a["K"], a["I"],
                 a["E"], a["k"], a["bm"], a["sc"], a["fl"], FAKE, a["ws"], a["wsb"], None)

    for fl in (moe.MOE_F_FP8_GATEUP, moe.MOE_F_INTER_UE8M0 | moe.MOE_F_MMA_E8M0,
               moe.MOE_FUSE_ON << moe.MOE_F_FUSE_SHIFT, moe.MOE_F_W13_PACKED,
               moe.MOE_PATH_COLUMNS << moe.MOE_F_GATEUP_PATH_SHIFT):
        assert _err(call(fl=fl)) == "MOE_ERR_UNSUPPORTED", fl
        assert moe.moe_w4a8_experts_workspace_size(4, 256, 256, 8, 2, 16, 128, fl) == 0
    # the column-split down takes E2M1 weights too (at most 192 routes)
    cols = moe.MOE_PATH_COLUMNS << moe.MOE_F_DOWN_PATH_SHIFT
    assert moe.moe_w4a8_experts_workspace_size(4, 256, 256, 8, 2, 16, 128, cols) > 0
    assert moe.moe_w4a8_experts_workspace_size(100, 256, 256, 8, 2, 16, 512, cols) == 0
    # the per-block down kernel keeps a block's intermediate rows in LDS:
    # I / 128 <= 512 / 64 at block_m 64 (unless the down stage is persistent)
    assert _err(call(I=2048, bm=64, sc=128)) == "MOE_ERR_UNSUPPORTED"
    persist_dn = moe.MOE_PATH_PERSISTENT << moe.MOE_F_DOWN_PATH_SHIFT
    assert moe.moe_w4a8_experts_workspace_size(4, 256, 2048, 8, 2, 64, 128, persist_dn) > 0
    assert _err(call(I=1024, bm=64, sc=128, wsb=16)) == "MOE_ERR_CAPACITY"
    assert _err(call(K=200)) == "MOE_ERR_SHAPE"
    assert _err(call(wsb=16)) == "MOE_ERR_CAPACITY"
    assert _err(call(ws=None)) == "MOE_ERR_NULL"
    assert _err(call(M=0)) == "MOE_OK"
    # explicit stream paths are accepted; the workspace is that of those paths
    stream = (moe.MOE_PATH_STREAM << moe.MOE_F_GATEUP_PATH_SHIFT) | \
             (moe.MOE_PATH_STREAM << moe.MOE_F_DOWN_PATH_SHIFT)
    w4 = moe.moe_w4a8_experts_workspace_size(4096, 4096, 1024, 288, 8, 64, 50944)
    assert w4 == moe.moe_w4a8_experts_workspace_size(4096, 4096, 1024, 288, 8, 64, 50944, stream)
    assert w4 == moe.moe_fp8_experts_workspace_size(4096, 4096, 1024, 288, 8, 64, 50944, stream)


def test_prepack_validation_before_any_device_call():
    f = _raw("moe_prepack_w13")
    assert moe.moe_prepack_w13_size(2, 256, 384) == 2 * 512 * 384
    assert moe.moe_prepack_w13_size(2, 100, 384) == 0
    assert moe.moe_prepack_w13_size(0, 256, 384) == 0
    assert _err(f(FAKE, 2, 100, 384, ctypes.c_void_p(0x20000000), None)) == "MOE_ERR_SHAPE"
    assert _err(f(None, 2, 256, 384, FAKE, None)) == "MOE_ERR_NULL"
    assert _err(f(ctypes.c_void_p(0x10008), 2, 256, 384, FAKE, None)) == "MOE_ERR_ALIGN"
    # overlapping source and destination
    assert _err(f(ctypes.c_void_p(0x10000000), 2, 256, 384, ctypes.c_void_p(0x10000100),
                  None)) == "MOE_ERR_SHAPE"
    # the W4A8 entry point does not take packed FP8 weights
    w4 = _raw("moe_w4a8_experts")
    assert _err(w4(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 256, 256, 8, 2, 16,
                   128, moe.MOE_F_W13_PACKED, FAKE, FAKE, 1 << 30, None)) == "MOE_ERR_UNSUPPORTED"
