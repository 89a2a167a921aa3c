// Steps 3 + 4 up to SwiGLU for small route counts: the gate/up GEMM split
// over intermediate columns and over K inside one workgroup, so no
// workgroup waits for another and nothing has to be cleared beforehand.
//
// Same arithmetic as gateup.hip (FlashInfer PR #4287, PR summary and
// public-contract section): for plan row p of block b (expert e, route r,
// token t = r / top_k)
//   g[p, n] = sum_kb x_s[t, kb] * w13_s[e, n / 128, kb]
//                    * sum_{k in kb} x_q[t, k] * W13[e, n, k]        (FP32)
//   h[p, j] = silu(g[p, j]) * g[p, I + j]
// written as FP32 rows h32[p, :]; the FP8 group requantisation of h (the
// rest of step 4) is done by the column-split down kernel as it loads the
// rows, with the same rule and rounding points as the other gate/up
// kernels' epilogue.
//
// Work split.  One workgroup = one plan block x SW intermediate columns (16:
// its 16 gate and 16 up rows of W13 as two MFMA tiles; 8: its 8 gate and 8
// up rows as one tile), all of K; wave w of the eight takes the K-blocks
// [w nkb / 8, (w + 1) nkb / 8).  At decode sizes (a few routes per expert)
// the item is a weight stream of 2 SW rows: each lane loads its MFMA operand
// slices straight into registers, four K-blocks ahead, so the whole slab of
// a workgroup is in flight at once; the codes are widened exactly to FP16
// (v_cvt_scalef32_pk_f16_fp8, every E4M3 value is an FP16 normal) and
// multiplied with v_mfma_f32_16x16x32_f16 (exact products, FP32
// accumulation), the per-K-block scale product applied in FP32.  The eight
// waves' partial sums are added in wave order in LDS -- deterministic --
// before SwiGLU.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kNT = 512;                // eight waves
constexpr int kDepth = 4;               // K-blocks in flight per wave

typedef const __attribute__((address_space(4))) int32_t *const_i32_p;
typedef const __attribute__((address_space(4))) float *const_f32_p;

// SW intermediate columns per workgroup: 16 (a gate and an up MFMA tile per
// K-block) or 8 (one MFMA tile of 8 gate and 8 up rows; twice the
// workgroups, each half the bytes, two workgroups per CU).
template <int BM, int SW>
__global__ void __launch_bounds__(kNT, SW == 8 ? 2 : 1)
gateup_slices_kernel(GateUpArgs a) {
    static_assert(BM <= 16, "one 16-row MFMA tile per plan block");
    static_assert(SW == 8 || SW == 16, "slice width");
    __shared__ __attribute__((aligned(16))) float sPart[8][16][2 * SW];  // [wave][plan row][gate cols, up cols]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t I = a.I, K = a.K;
    const int nsl = (int)(I / SW);
    const int b = blockIdx.x / nsl, s = blockIdx.x % nsl;

    const int ntp = __builtin_amdgcn_readfirstlane(((const_i32_p)a.ntp)[0]);
    if ((int64_t)b * BM >= ntp) return;                 // padded block
    const int e = __builtin_amdgcn_readfirstlane(((const_i32_p)a.eids)[b]);
    if (e < 0 || e >= a.E) return;

    // this lane's plan row (l16) and its token; rows without a route read
    // the block's first valid row (their sums are never stored)
    const int64_t p = (int64_t)b * BM + (l16 < BM ? l16 : 0);
    const int r = a.sorted[p];
    const bool valid = l16 < BM && r >= 0 && (int64_t)r < a.R;
    const uint64_t vm = __ballot(valid);
    if (vm == 0) return;                                 // (uniform)
    const int first = __builtin_ctzll(vm);
    const int rf = __shfl(r, first, 64);
    const int t = (valid ? r : rf) / a.top_k;

    const int nkb = a.nkb;
    const int kb0 = w * nkb / 8, kb1 = (w + 1) * nkb / 8;
    // W13 rows: SW = 16, gate row SW s + l16 and up row I + SW s + l16 in
    // two tiles; SW = 8, one tile whose rows 0-7 are gate rows SW s + l16 and
    // rows 8-15 up rows I + SW s + l16 - 8
    const int64_t wrow = SW == 16 ? (int64_t)s * SW + l16
                                  : (l16 < 8 ? (int64_t)s * SW + l16 : I + (int64_t)s * SW + l16 - 8);
    const uint8_t *wg = a.w13 + ((int64_t)e * 2 * I + wrow) * K + 16 * g;
    const uint8_t *wu = wg + I * K;                      // (SW = 16)
    const uint8_t *xr = a.xq + (int64_t)t * K + 16 * g;
    const float *xsr = a.xs + (int64_t)t * nkb;
    // block scales of the gate and the up rows (scalar loads)
    const int nb13 = (int)(2 * I / 128);
    const const_f32_p sgp = (const_f32_p)a.w13s + ((int64_t)e * nb13 + (s * SW) / 128) * nkb;
    const const_f32_p sup = (const_f32_p)a.w13s + ((int64_t)e * nb13 + (I + s * SW) / 128) * nkb;

    struct Ld {
        u32x4 g0, g1, u0, u1, x0, x1;
        float xs;
    };
    Ld q[kDepth];
    auto load = [&](Ld &d, int kb) {
        const int64_t o = (int64_t)kb * 128;
        d.g0 = *reinterpret_cast<const u32x4 *>(wg + o);
        d.g1 = *reinterpret_cast<const u32x4 *>(wg + o + 64);
        if constexpr (SW == 16) {
            d.u0 = *reinterpret_cast<const u32x4 *>(wu + o);
            d.u1 = *reinterpret_cast<const u32x4 *>(wu + o + 64);
        }
        d.x0 = *reinterpret_cast<const u32x4 *>(xr + o);
        d.x1 = *reinterpret_cast<const u32x4 *>(xr + o + 64);
        d.xs = xsr[kb];
    };
    v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = accg;
    auto compute = [&](const Ld &d, int kb) {
        v8h ah[4], gh[4];
        e4m3x32_to_f16(d.x0, d.x1, ah);
        e4m3x32_to_f16(d.g0, d.g1, gh);
        const v4f tg = mfma16x16x128_f16(gh, ah);
        if constexpr (SW == 16) {
            v8h uh[4];
            e4m3x32_to_f16(d.u0, d.u1, uh);
            const v4f tu = mfma16x16x128_f16(uh, ah);
            accg = tg * (d.xs * sgp[kb]) + accg;
            accu = tu * (d.xs * sup[kb]) + accu;
        } else {
            // lane group g holds tile rows 4 g .. 4 g + 3: gate rows for g < 2
            accg = tg * (d.xs * (g < 2 ? sgp[kb] : sup[kb])) + accg;
        }
    };
    // a ring of kDepth register sets, refilled as each is used (the
    // compiler's own load counts order each use after its loads)
#pragma unroll
    for (int i = 0; i < kDepth; ++i)
        if (kb0 + i < kb1) load(q[i], kb0 + i);
    for (int kb = kb0; kb < kb1; kb += kDepth) {
#pragma unroll
        for (int i = 0; i < kDepth; ++i) {
            const int k = kb + i;
            if (k >= kb1) break;
            compute(q[i], k);
            if (k + kDepth < kb1) load(q[i], k + kDepth);
        }
    }
    // lane (plan row l16, group g) holds tile rows 4g .. 4g + 3 of its plan
    // row; every lane stores (keeps the MFMAs out of any lane condition).
    // SW = 8: tile rows 0-7 are the gate columns, 8-15 the up columns, as
    // the layout [gate SW][up SW] wants.
    *reinterpret_cast<v4f *>(&sPart[w][l16][4 * g]) = accg;
    if constexpr (SW == 16) *reinterpret_cast<v4f *>(&sPart[w][l16][SW + 4 * g]) = accu;
    __syncthreads();

    // ---- the eight waves' sums in wave order, SwiGLU, FP32 rows out
    if (tid < 16 * SW) {
        const int row = tid / SW, col = tid % SW;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            gs += sPart[v][row][col];
            us += sPart[v][row][SW + col];
        }
        const int rr = __shfl(r, row, 64);               // (lanes 0..15 of any wave hold rows 0..15)
        const bool ok = row < BM && rr >= 0 && (int64_t)rr < a.R;
        if (ok) a.h32[((int64_t)b * BM + row) * I + (int64_t)s * SW + col] = swiglu(gs, us);
    }
}

template <int BM, int SW>
hipError_t launch_gs(const GateUpArgs &a, hipStream_t st) {
    const int64_t grid = (int64_t)a.nblocks * (a.I / SW);
    if (grid == 0) return hipSuccess;
    gateup_slices_kernel<BM, SW><<<(unsigned)grid, kNT, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup_slices(const GateUpArgs &a, int block_m, int slice, hipStream_t st) {
    if (!a.h32 || a.I % 16 != 0) return hipErrorInvalidValue;
    if (slice == 8) {
        if (block_m == 8) return launch_gs<8, 8>(a, st);
        if (block_m == 16) return launch_gs<16, 8>(a, st);
    } else if (slice == 16) {
        if (block_m == 8) return launch_gs<8, 16>(a, st);
        if (block_m == 16) return launch_gs<16, 16>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
