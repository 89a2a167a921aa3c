// Step 5: down-projection GEMM over the requantised SwiGLU rows, weighting
// by the router probability, and the reduce-add into the caller's output.
//
// What is computed (FlashInfer PR #4287, PR summary and the FP32-scale note
// of its final kernel performance section): for plan row p of block b
// (expert e, route r, token t = r / top_k)
//   y[r, c] = sum_jb h_s[p, jb] * w2_s[e, c / 128, jb]
//                    * sum_{j in jb} h_q[p, j] * W2[e, c, j]           (FP32)
//   out[t, c] += topk_weights[r] * y[r, c]
// Each route's row goes to a route-indexed buffer y[r, :] (plain stores, no
// atomics) as FP16 values with one FP32 scale per 64 columns (amax / 2^15:
// 2^-12 relative rounding, FP32's range, half the bytes of FP32); the
// finalize kernel then adds, per token, its top_k rows times their router
// weights in route order to the caller's BF16 output and rounds once -- the
// output is an accumulator, and the reduction is deterministic.
//
// Tiling: one workgroup = one plan block (BM rows) x 256 output columns; four
// waves take 64 columns each (four 16-row W2 subtiles, all inside one
// 128-column scale block).  The intermediate rows of a block are contiguous
// in the workspace (plan-row order), so the B tile is a plain 128-byte-row
// copy into LDS; W2 rows stream into registers as in the gate/up kernel.
#include <type_traits>

#include "common.h"
#include "down_item.h"
#include "internal.h"

namespace moe {

namespace {

using namespace ds;

template <int BM>
struct DNCfg {
    static constexpr int TM = BM < 16 ? 16 : (BM < 64 ? BM : 64);   // MFMA rows per wave row
    static constexpr int WM = BM > TM ? BM / TM : 1;
    static constexpr int ROWS = TM * WM;           // tile rows (block_m = 8: 8 masked)
    static constexpr int NW = 4 * WM;
    static constexpr int NT = 64 * NW;
    static constexpr int NU = TM / 16;
    static constexpr int ROWB = 144;
    static constexpr int CHUNKS = BM * 8;
    static constexpr int CPT = (CHUNKS + NT - 1) / NT;
};

__device__ __forceinline__ v8i join8d(const u32x4 &lo, const u32x4 &hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

template <int BM, bool E8M0>
__global__ void __launch_bounds__(DNCfg<BM>::NT)
down_kernel(DownArgs a) {
    using C = DNCfg<BM>;
    __shared__ __attribute__((aligned(16))) uint8_t sH[2][C::ROWS * C::ROWB];
    __shared__ float sHs[2][C::ROWS];
    __shared__ int sRt[C::ROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int wn = w & 3, wm = w >> 2;
    const int l16 = lane & 15, g = lane >> 4;

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int b = L % a.nblocks;
    const int ct = L / a.nblocks;

    if (b * BM >= a.ntp[0]) return;              // padded-block early exit
    const int e = __builtin_amdgcn_readfirstlane(a.eids[b]);   // uniform: scalar descriptors
    if (e < 0 || e >= a.E) return;

    if (tid < C::ROWS) {
        int r = tid < BM ? a.sorted[(int64_t)b * BM + tid] : -1;
        sRt[tid] = (r >= 0 && (int64_t)r < a.R) ? r : -1;
        if (tid >= BM) sHs[0][tid] = sHs[1][tid] = 0.f;   // rows past the block: scale 0
    }
    __syncthreads();

    const int64_t I = a.I, K = a.K;
    const int64_t col0 = (int64_t)ct * 256 + 64 * wn;   // this wave's first column
    const bool wave_on = col0 < K;
    const int njb = a.njb;

    const uint8_t *wrow[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        int64_t c = wave_on ? col0 + 16 * s + l16 : 0;
        wrow[s] = a.w2 + ((int64_t)e * K + c) * I + 16 * g;
    }
    const float *sb_ptr = a.w2s + ((int64_t)e * (K >> 7) + (wave_on ? (col0 >> 7) : 0)) * njb;
    const uint8_t *hbase = a.hq + (int64_t)b * BM * I;
    const float *hsbase = a.hs + (int64_t)b * BM * njb;

    v4f acc[4][C::NU];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < C::NU; ++u) acc[s][u] = v4f{0.f, 0.f, 0.f, 0.f};

    v8i wcur[4], wnxt[4];
    u32x4 hbuf[C::CPT];
    float hs_reg = 0.f;

    auto load_w = [&](int jb, v8i (&dst)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(wrow[s] + (int64_t)jb * 128);
            dst[s] = join8d(p[0], p[4]);
        }
    };
    auto load_h = [&](int jb) {
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            int c = tid + i * C::NT;
            if (c < C::CHUNKS)
                hbuf[i] = *reinterpret_cast<const u32x4 *>(hbase + (int64_t)(c >> 3) * I +
                                                           (int64_t)jb * 128 + (c & 7) * 16);
        }
        if (tid < BM) hs_reg = hsbase[(int64_t)tid * njb + jb];
    };
    auto store_h = [&](int buf) {
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            int c = tid + i * C::NT;
            if (c < C::CHUNKS)
                *reinterpret_cast<u32x4 *>(&sH[buf][(c >> 3) * C::ROWB + (c & 7) * 16]) = hbuf[i];
        }
        if (tid < BM) sHs[buf][tid] = hs_reg;
    };

    if (wave_on) load_w(0, wcur);
    load_h(0);
    store_h(0);
    __syncthreads();

    for (int jb = 0; jb < njb; ++jb) {
        const int buf = jb & 1;
        const bool more = jb + 1 < njb;
        if (more) {
            if (wave_on) load_w(jb + 1, wnxt);
            load_h(jb + 1);
        }
        if (wave_on) {
            const float sb = sb_ptr[jb];
#pragma unroll
            for (int u = 0; u < C::NU; ++u) {
                const int row = wm * C::TM + u * 16 + l16;
                const uint8_t *bp = &sH[buf][row * C::ROWB + 16 * g];
                v8i B = join8d(*reinterpret_cast<const u32x4 *>(bp),
                               *reinterpret_cast<const u32x4 *>(bp + 64));
                const float sa = sHs[buf][row];
                if constexpr (E8M0) {
                    const int ea = e8m0_of(sb), eb = e8m0_of(sa);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        acc[s][u] = mfma16x16x128_e8m0(wcur[s], B, acc[s][u], ea, eb);
                } else {
                    const float f = sa * sb;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        v4f t = mfma16x16x128(wcur[s], B);
                        acc[s][u] = t * f + acc[s][u];
                    }
                }
            }
        }
        if (more) {
            store_h(buf ^ 1);
#pragma unroll
            for (int s = 0; s < 4; ++s) wcur[s] = wnxt[s];
        }
        __syncthreads();
    }

    if (!wave_on) return;
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
        const int row = wm * C::TM + u * 16 + l16;
        // the row's 64 columns of this wave: 16 values in each of 4 lanes
        float m = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(acc[s][u][i]));
        m = wave_max_xor(m, 16);
        m = wave_max_xor(m, 32);
        const int r = sRt[row];
        if (r < 0) continue;
        float sc, inv;
        y16_scale(m, sc, inv);
        uint16_t *dst = a.y16 + (int64_t)r * K + col0 + 4 * g;
#pragma unroll
        for (int s = 0; s < 4; ++s) *reinterpret_cast<uint2 *>(dst + 16 * s) = f32x4_to_f16x4(acc[s][u], inv);
        if (g == 0) a.ys[(int64_t)r * (K >> 6) + (col0 >> 6)] = sc;
    }
}

template <int BM, bool E8M0, bool W4 = false>
__global__ void __launch_bounds__(512)
down_stream_kernel(DownArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int ncw = (a.ctiles + a.nct - 1) / a.nct;     // column groups
    int L = blockIdx.x;
    const int b = L % a.nblocks;
    L /= a.nblocks;
    const int cw = L % ncw;
    const int pass = L / ncw;
    down_item<BM, E8M0, false, W4>(a, smem, b, cw, pass, nullptr);
}

__global__ void __launch_bounds__(256)
fill_kernel(uint32_t *__restrict__ p, size_t n, uint32_t v) {
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    size_t stride = (size_t)gridDim.x * 256;
    for (; i < n; i += stride) p[i] = v;
}

// Route sum + accumulate into the BF16 output, one thread per 8 consecutive
// outputs of a token row (finalize8).
__global__ void __launch_bounds__(256)
finalize_kernel(uint16_t *__restrict__ out, const uint16_t *__restrict__ y16,
                const float *__restrict__ ys, const float *__restrict__ topk_w,
                const int32_t *__restrict__ rpos, int64_t M, int64_t K, int top_k) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;   // element of out
    if (i >= M * K) return;
    const int64_t t = i / K;
    finalize8<false>(out, y16, ys, topk_w, rpos, t, i - t * K, K, top_k);
}

template <int BM, bool E8M0>
hipError_t launch_dn(const DownArgs &a, hipStream_t st) {
    int64_t grid = (int64_t)a.nblocks * a.ctiles;
    if (grid == 0) return hipSuccess;
    down_kernel<BM, E8M0><<<(unsigned)grid, DNCfg<BM>::NT, 0, st>>>(a);
    return hipGetLastError();
}

template <int BM, bool E8M0, bool W4 = false>
hipError_t launch_ds(DownArgs a, hipStream_t st) {
    using C = DSCfg<BM>;
    if (a.njb > C::JMAX) {                           // rows too long for the LDS tile
        if constexpr (W4) return hipErrorInvalidValue;
        else return launch_dn<BM, E8M0>(a, st);
    }
    // column tiles per workgroup: enough workgroups to cover the chip first
    const int64_t units = (int64_t)a.nblocks * a.ctiles * C::NPASS;
    int nct = (int)(units / 1024);
    nct = nct < 1 ? 1 : (nct > C::NCTMAX ? C::NCTMAX : nct);
    a.nct = nct;
    const int64_t grid = (int64_t)a.nblocks * ((a.ctiles + nct - 1) / nct) * C::NPASS;
    if (grid == 0) return hipSuccess;
    const int lds = DSLayout(C::RP, a.njb, nct, C::YROW).total;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e =
        raise_lds_limit(lds_set, (const void *)down_stream_kernel<BM, E8M0, W4>, 160 * 1024);
    if (e != hipSuccess) return e;
    down_stream_kernel<BM, E8M0, W4><<<(unsigned)grid, C::NT, lds, st>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_down(const DownArgs &a, int block_m, bool e8m0, hipStream_t st) {
    switch (block_m) {
        case 8: return e8m0 ? launch_ds<8, true>(a, st) : launch_ds<8, false>(a, st);
        case 16: return e8m0 ? launch_ds<16, true>(a, st) : launch_ds<16, false>(a, st);
        case 32: return e8m0 ? launch_ds<32, true>(a, st) : launch_ds<32, false>(a, st);
        case 64: return e8m0 ? launch_ds<64, true>(a, st) : launch_ds<64, false>(a, st);
        case 128: return e8m0 ? launch_ds<128, true>(a, st) : launch_ds<128, false>(a, st);
        default: return hipErrorInvalidValue;
    }
}

int down_w4_max_njb(int block_m) {
    switch (block_m) {
        case 8: return DSCfg<8>::JMAX;
        case 16: return DSCfg<16>::JMAX;
        case 32: return DSCfg<32>::JMAX;
        case 64: return DSCfg<64>::JMAX;
        case 128: return DSCfg<128>::JMAX;
        default: return 0;
    }
}

hipError_t launch_down_w4(const DownArgs &a, int block_m, hipStream_t st) {
    switch (block_m) {
        case 8: return launch_ds<8, false, true>(a, st);
        case 16: return launch_ds<16, false, true>(a, st);
        case 32: return launch_ds<32, false, true>(a, st);
        case 64: return launch_ds<64, false, true>(a, st);
        case 128: return launch_ds<128, false, true>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fill(uint32_t *p, size_t n_words, uint32_t value, hipStream_t st) {
    if (n_words == 0) return hipSuccess;
    size_t blocks = (n_words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    fill_kernel<<<(unsigned)blocks, 256, 0, st>>>(p, n_words, value);
    return hipGetLastError();
}

hipError_t launch_finalize(uint16_t *out, const uint16_t *y16, const float *ys, const float *topk_w,
                           const int32_t *rpos, int64_t M, int64_t K, int top_k, hipStream_t st) {
    int64_t blocks = (M * K / 8 + 255) / 256;
    if (blocks == 0) return hipSuccess;
    finalize_kernel<<<(unsigned)blocks, 256, 0, st>>>(out, y16, ys, topk_w, rpos, M, K, top_k);
    return hipGetLastError();
}

}  // namespace moe
