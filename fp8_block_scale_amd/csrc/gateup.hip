// Steps 3 + 4: gate/up grouped GEMM with 128x128 FP32 weight block scales,
// SwiGLU, and FP8 requantisation of the SwiGLU output per plan row and
// 128-column group.
//
// What is computed (FlashInfer PR #4287, PR summary and public-contract
// section): for plan row p of block b (expert e = expert_ids[b], route
// r = sorted[p], token t = r / top_k)
//   g[p, n] = sum_kb x_s[t, kb] * w13_s[e, n / 128, kb]
//                    * sum_{k in kb} x_q[t, k] * W13[e, n, k]        (FP32)
//   h[p, j] = silu(g[p, j]) * g[p, I + j],  silu(v) = v / (1 + e^-v)
//   h_q[p, j], h_s[p, j / 128] = FP8 group quantisation of h (FP32 or
//   power-of-two scale rule; the FLT_MIN floor keeps all-zero rows finite).
//
// Tiling (gfx950, wave64): one workgroup = one plan block (BM rows) x one
// 128-wide intermediate tile (its 128 gate rows and 128 up rows of W13)
// x one K-range.  Four waves split the 128 columns 32 apiece, so each wave
// holds matching gate and up accumulators and SwiGLU needs no exchange.  The
// weights are the A operand (16 rows of W13), the gathered activations B
// (16 tokens); one 16x16 tile per 128-deep K-block is exactly one scale
// block, and each lane's four results share one token, so the FP32 scale is
// one multiply and four FMAs.
//
// Three MMA modes:
//   kExact  (default) the E4M3 codes are widened exactly to FP16 in registers
//           and multiplied with v_mfma_f32_16x16x32_f16 (exact products, FP32
//           accumulation), so the SwiGLU input carries only FP32 rounding --
//           what the requantised codes need to match an exact reference;
//   kFp8    v_mfma_f32_16x16x128_f8f6f4 on the codes directly (twice the
//           peak rate; its internal sum keeps ~15 bits below the largest
//           product, so a few 1e-3 of the requantised codes move one step);
//   kFp8E8  as kFp8 with power-of-two scales applied inside the MFMA as E8M0
//           exponents (no VALU scale multiply).
// Weights stream from HBM straight into registers (each wave reads rows no
// other wave reads); activation rows are gathered once per workgroup into
// LDS (double buffered) and shared by the waves.  Blocks at or beyond the
// device-side padded length exit before touching memory.
//
// Small grids (decode) split K; partial sums of the valid rows go to the
// workspace and the last workgroup of a tile to arrive (atomic counter) adds
// them in split order -- deterministic -- before SwiGLU.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

template <int BM>
struct GUCfg {
    static constexpr int TM = BM < 64 ? BM : 64;   // tokens per wave
    static constexpr int WM = BM / TM;             // waves along tokens
    static constexpr int NW = 4 * WM;              // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int NU = TM / 16;             // 16-token subtiles per wave
    static constexpr int ROWB = 144;               // LDS row stride (128 + 16 pad)
    static constexpr int CHUNKS = BM * 8;          // 16-byte chunks of one A tile
    static constexpr int CPT = (CHUNKS + NT - 1) / NT;
};

__device__ __forceinline__ v8i join8(const u32x4 &lo, const u32x4 &hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

enum { kExact = 0, kFp8 = 1, kFp8E8 = 2 };

template <int BM, int MODE>
__global__ void __launch_bounds__(GUCfg<BM>::NT)
gateup_kernel(GateUpArgs a) {
    using C = GUCfg<BM>;
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * C::ROWB];
    __shared__ float sSa[2][BM];
    __shared__ int sTok[BM];
    __shared__ float sRed[4][BM];
    __shared__ int sFlag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int wn = w & 3, wm = w >> 2;
    const int l16 = lane & 15, g = lane >> 4;

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int b = L % a.nblocks;
    const int rest = L / a.nblocks;
    const int split = rest % a.nsplit;
    const int jt = rest / a.nsplit;

    if (b * BM >= a.ntp[0]) return;              // padded-block early exit
    const int e = a.eids[b];
    if (e < 0 || e >= a.E) return;

    if (tid < BM) {
        int r = a.sorted[(int64_t)b * BM + tid];
        const bool ok = r >= 0 && (int64_t)r < a.R;
        sTok[tid] = ok ? r / a.top_k : -1;
        if (ok && jt == 0 && split == 0) a.rpos[r] = b * BM + tid;   // inverse plan map
    }
    __syncthreads();

    const int kb0 = split * a.kb_per_split;
    const int kb1 = kb0 + a.kb_per_split < a.nkb ? kb0 + a.kb_per_split : a.nkb;
    const int64_t I = a.I, K = a.K;
    const int64_t twoI = 2 * I;
    const int nb13 = (int)(twoI >> 7);

    // this lane's W13 rows: subtiles 0,1 gate, 2,3 up
    const uint8_t *wrow[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        int64_t n = (s < 2 ? 0 : I) + (int64_t)jt * 128 + 32 * wn + 16 * (s & 1) + l16;
        wrow[s] = a.w13 + ((int64_t)e * twoI + n) * K + 16 * g;
    }
    const float *sg_ptr = a.w13s + ((int64_t)e * nb13 + jt) * a.nkb;
    const float *su_ptr = a.w13s + ((int64_t)e * nb13 + (I >> 7) + jt) * a.nkb;

    v4f acc[4][C::NU];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < C::NU; ++u) acc[s][u] = v4f{0.f, 0.f, 0.f, 0.f};

    v8i wcur[4], wnxt[4];
    u32x4 abuf[C::CPT];
    float sa_reg = 0.f;

    auto load_w = [&](int kb, v8i (&dst)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(wrow[s] + (int64_t)kb * 128);
            dst[s] = join8(p[0], p[4]);
        }
    };
    auto load_a = [&](int kb) {
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            int c = tid + i * C::NT;
            if (c < C::CHUNKS) {
                int t = sTok[c >> 3];
                abuf[i] = t >= 0 ? *reinterpret_cast<const u32x4 *>(a.xq + (int64_t)t * K +
                                                                     (int64_t)kb * 128 + (c & 7) * 16)
                                 : u32x4{0u, 0u, 0u, 0u};
            }
        }
        if (tid < BM) {
            int t = sTok[tid];
            sa_reg = t >= 0 ? a.xs[(int64_t)t * a.nkb + kb] : 0.f;
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            int c = tid + i * C::NT;
            if (c < C::CHUNKS)
                *reinterpret_cast<u32x4 *>(&sA[buf][(c >> 3) * C::ROWB + (c & 7) * 16]) = abuf[i];
        }
        if (tid < BM) sSa[buf][tid] = sa_reg;
    };

    if (kb0 < kb1) {
        load_w(kb0, wcur);
        load_a(kb0);
        store_a(0);
    }
    __syncthreads();

    for (int kb = kb0; kb < kb1; ++kb) {
        const int buf = (kb - kb0) & 1;
        const bool more = kb + 1 < kb1;
        if (more) {
            load_w(kb + 1, wnxt);
            load_a(kb + 1);
        }
        const float sbg = sg_ptr[kb];
        const float sbu = su_ptr[kb];
        v8h wh[4][4];
        if constexpr (MODE == kExact) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 lo = {(unsigned)wcur[s][0], (unsigned)wcur[s][1], (unsigned)wcur[s][2],
                                  (unsigned)wcur[s][3]};
                const u32x4 hi = {(unsigned)wcur[s][4], (unsigned)wcur[s][5], (unsigned)wcur[s][6],
                                  (unsigned)wcur[s][7]};
                e4m3x32_to_f16(lo, hi, wh[s]);
            }
        }
#pragma unroll
        for (int u = 0; u < C::NU; ++u) {
            const int row = wm * C::TM + u * 16 + l16;
            const uint8_t *bp = &sA[buf][row * C::ROWB + 16 * g];
            v8i B = join8(*reinterpret_cast<const u32x4 *>(bp),
                          *reinterpret_cast<const u32x4 *>(bp + 64));
            const float sa = sSa[buf][row];
            if constexpr (MODE == kExact) {
                v8h Bh[4];
                e4m3x32_to_f16(*reinterpret_cast<const u32x4 *>(bp),
                               *reinterpret_cast<const u32x4 *>(bp + 64), Bh);
                const float fg = sa * sbg, fu = sa * sbu;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    v4f t = mfma16x16x128_f16(wh[s], Bh);
                    const float f = s < 2 ? fg : fu;
                    acc[s][u] = t * f + acc[s][u];
                }
            } else if constexpr (MODE == kFp8E8) {
                const int eb = e8m0_of(sa);
                const int eg = e8m0_of(sbg), eu = e8m0_of(sbu);
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc[s][u] = mfma16x16x128_e8m0(wcur[s], B, acc[s][u], s < 2 ? eg : eu, eb);
            } else {
                const float fg = sa * sbg, fu = sa * sbu;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    v4f t = mfma16x16x128(wcur[s], B);
                    const float f = s < 2 ? fg : fu;
                    acc[s][u] = t * f + acc[s][u];
                }
            }
        }
        if (more) {
            store_a(buf ^ 1);
#pragma unroll
            for (int s = 0; s < 4; ++s) wcur[s] = wnxt[s];
        }
        __syncthreads();
    }

    // ---- split-K: publish partial sums, last arriver reduces in split order
    if (a.nsplit > 1) {
        const int tile = jt * a.nblocks + b;
        float *base = a.part + (size_t)tile * a.nsplit * BM * 256;
#pragma unroll
        for (int u = 0; u < C::NU; ++u) {
            const int row = wm * C::TM + u * 16 + l16;
            if (sTok[row] >= 0) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int n = (s < 2 ? 0 : 128) + 32 * wn + 16 * (s & 1) + 4 * g;
                    *reinterpret_cast<v4f *>(base + ((size_t)split * BM + row) * 256 + n) = acc[s][u];
                }
            }
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            unsigned old = atomicAdd(&a.cnt[tile], 1u);
            sFlag = old == (unsigned)(a.nsplit - 1);
        }
        __syncthreads();
        if (!sFlag) return;
        __threadfence();
#pragma unroll
        for (int u = 0; u < C::NU; ++u) {
            const int row = wm * C::TM + u * 16 + l16;
            const bool valid = sTok[row] >= 0;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int n = (s < 2 ? 0 : 128) + 32 * wn + 16 * (s & 1) + 4 * g;
                v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
                if (valid)
                    for (int sp = 0; sp < a.nsplit; ++sp)
                        sum += *reinterpret_cast<const v4f *>(base + ((size_t)sp * BM + row) * 256 + n);
                acc[s][u] = sum;
            }
        }
        if (tid == 0) a.cnt[tile] = 0u;
    }

    // ---- SwiGLU + per-row 128-group FP8 requantisation
    float h[C::NU][2][4];
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
        float amax = 0.f;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gt = acc[s][u][i];
                const float up = acc[s + 2][u][i];
                const float hv = gt / (1.0f + expf(-gt)) * up;
                h[u][s][i] = hv;
                amax = fmaxf(amax, fabsf(hv));
            }
        amax = wave_max_xor(amax, 16);
        amax = wave_max_xor(amax, 32);
        if (g == 0) sRed[wn][wm * C::TM + u * 16 + l16] = amax;
    }
    __syncthreads();
    const bool ue = a.inter_ue8m0 != 0;
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
        const int row = wm * C::TM + u * 16 + l16;
        const float amax = fmaxf(fmaxf(sRed[0][row], sRed[1][row]), fmaxf(sRed[2][row], sRed[3][row]));
        float s, inv;
        group_scale(amax, ue, s, inv);
        const int64_t p = (int64_t)b * BM + row;
        uint8_t *dst = a.hq + p * I + (int64_t)jt * 128 + 32 * wn + 4 * g;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint32_t code = pack_e4m3x4(h[u][s2][0] * inv, h[u][s2][1] * inv,
                                        h[u][s2][2] * inv, h[u][s2][3] * inv);
            *reinterpret_cast<uint32_t *>(dst + 16 * s2) = code;
        }
        if (wn == 0 && g == 0) a.hs[p * (I >> 7) + jt] = s;
    }
}

template <int BM, int MODE>
hipError_t launch_gu(const GateUpArgs &a, hipStream_t st) {
    int64_t grid = (int64_t)a.nblocks * a.jtiles * a.nsplit;
    if (grid == 0) return hipSuccess;
    gateup_kernel<BM, MODE><<<(unsigned)grid, GUCfg<BM>::NT, 0, st>>>(a);
    return hipGetLastError();
}

template <int BM>
hipError_t launch_gu_mode(const GateUpArgs &a, int mode, hipStream_t st) {
    switch (mode) {
        case kExact: return launch_gu<BM, kExact>(a, st);
        case kFp8: return launch_gu<BM, kFp8>(a, st);
        case kFp8E8: return launch_gu<BM, kFp8E8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gateup(const GateUpArgs &a, int block_m, bool fp8_mma, bool e8m0,
                         hipStream_t st) {
    const int mode = !fp8_mma ? kExact : (e8m0 ? kFp8E8 : kFp8);
    switch (block_m) {
        case 16: return launch_gu_mode<16>(a, mode, st);
        case 32: return launch_gu_mode<32>(a, mode, st);
        case 64: return launch_gu_mode<64>(a, mode, st);
        case 128: return launch_gu_mode<128>(a, mode, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
