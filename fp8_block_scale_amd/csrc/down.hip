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
#include "internal.h"

namespace moe {

namespace {

template <int BM>
struct DNCfg {
    static constexpr int TM = BM < 64 ? BM : 64;
    static constexpr int WM = BM / TM;
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
    __shared__ __attribute__((aligned(16))) uint8_t sH[2][BM * C::ROWB];
    __shared__ float sHs[2][BM];
    __shared__ int sRt[BM];

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

    if (tid < BM) {
        int r = a.sorted[(int64_t)b * BM + tid];
        sRt[tid] = (r >= 0 && (int64_t)r < a.R) ? r : -1;
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

// ---------------------------------------------------------------------------
// Small-grid down GEMM: a weight stream, as the small-grid gate/up kernel.
// One workgroup = one plan block (its valid rows, in passes of at most 64) x
// nct consecutive 256-column tiles of the output; eight waves take 32
// columns of each tile.  The block's SwiGLU rows (all of I) are DMA'd into
// LDS once; the W2 rows stream into registers through a buffer descriptor,
// four (tile, K-block) units per stage, two stages in flight.  A finished
// tile's FP32 results are parked in LDS (no global store inside the loop, so
// the loop's vmcnt waits count only its own loads) and written, weighted by
// the router probability, after the loop.
template <int BM>
struct DSCfg {
    static constexpr int RP = BM < 64 ? BM : 64;   // plan rows per pass
    static constexpr int NPASS = BM / RP;
    static constexpr int NU = RP / 16;
    static constexpr int NT = 512;
    static constexpr int S = 2;                    // units per stage
    static constexpr int LPS = 4 * S;
    static constexpr int JMAX = 512 / RP;          // I / 128 limit (64 KB row tile)
    static constexpr int NCTMAX = 64 / RP;         // column tiles per workgroup
    static constexpr int YROW = 260;               // floats per parked row
};

// LDS carve-up, sized per launch: the row tile (rows of roundup(njb, 8)
// K-blocks, so one DMA run never leaves its row), the parked results
// [nct][RP][YROW], the row scales [RP][njb], the W2 scales [nct][2][njb],
// routes, flags.
struct DSLayout {
    int hrowb, y, hs, ws, tok, misc, total;
    __host__ __device__ DSLayout(int rp, int njb, int nct, int yrow) {
        hrowb = ((njb + 7) & ~7) * 128;
        y = rp * hrowb;
        hs = y + nct * rp * yrow * 4;
        ws = hs + rp * njb * 4;
        tok = ws + nct * 2 * njb * 4;
        misc = tok + rp * 4;
        total = misc + 16;
    }
};

template <int BM, bool E8M0>
__global__ void __launch_bounds__(512)
down_stream_kernel(DownArgs a) {
    using C = DSCfg<BM>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const DSLayout Ld(C::RP, a.njb, a.nct, C::YROW);
    uint8_t *sH = smem;
    float *sY = reinterpret_cast<float *>(smem + Ld.y);
    float *sHs = reinterpret_cast<float *>(smem + Ld.hs);
    float *sWs = reinterpret_cast<float *>(smem + Ld.ws);
    int *sTok = reinterpret_cast<int *>(smem + Ld.tok);
    int *sMisc = reinterpret_cast<int *>(smem + Ld.misc);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;

    const int ncw = (a.ctiles + a.nct - 1) / a.nct;     // column groups
    int L = blockIdx.x;
    const int b = L % a.nblocks;
    L /= a.nblocks;
    const int cw = L % ncw;
    const int pass = L / ncw;
    const int row0 = pass * C::RP;
    const int ct0 = cw * a.nct;
    const int nct = a.ctiles - ct0 < a.nct ? a.ctiles - ct0 : a.nct;

    int r = -1;
    if (w == 0 && lane < C::RP) r = a.sorted[(int64_t)b * BM + row0 + lane];
    const int ntp = a.ntp[0];
    if (b * BM >= ntp) return;                          // padded block
    const int e = __builtin_amdgcn_readfirstlane(a.eids[b]);   // uniform: scalar descriptors
    if (e < 0 || e >= a.E) return;

    const int njb = a.njb;
    const int64_t K = a.K, I = a.I;
    for (int i = tid; i < C::RP * njb; i += C::NT) sHs[i] = 0.f;
    for (int i = tid; i < a.nct * 2 * njb; i += C::NT) sWs[i] = 0.f;
    if (w == 0) {
        if (lane < C::RP) {
            r = (r >= 0 && (int64_t)r < a.R) ? r : -1;
            sTok[lane] = r;
        }
        const uint64_t m = __ballot(r >= 0);
        if (lane == 0) sMisc[0] = m ? 64 - __builtin_clzll(m) : 0;
    }
    __syncthreads();
    const int nvp = sMisc[0];
    if (nvp == 0) return;
    const int nvpad = (nvp + 15) & ~15;

    // ---- W2 stream: units (tile t, K-block jb), jb fastest
    const int nunits = nct * njb;
    const int nst = (nunits + C::S - 1) / C::S;
    const uint8_t *wbase = a.w2 + ((int64_t)e * K + (int64_t)ct0 * 256) * I;
    const int64_t rows_here = K - (int64_t)ct0 * 256 < (int64_t)nct * 256 ? K - (int64_t)ct0 * 256
                                                                           : (int64_t)nct * 256;
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void *)wbase, (short)0, (int)(rows_here * I), 0x00020000);
    const int past = (int)(rows_here * I);
    const int rowoff0 = (32 * w + l16) * (int)I + 16 * g;   // subtile 0; subtile 1 is 16 rows on
    u32x4 wb[2][C::S][4];
    auto issue = [&](int st, auto BUF) {
        constexpr int bf = decltype(BUF)::value;
#pragma unroll
        for (int kk = 0; kk < C::S; ++kk) {
            const int u = st * C::S + kk;
            const int t = u / njb, jb = u - t * njb;
            const int vo = u < nunits ? rowoff0 + (t * 256) * (int)I + jb * 128 : past;
            wb[bf][kk][0] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo, 0, 0);
            wb[bf][kk][1] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo + 64, 0, 0);
            wb[bf][kk][2] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo + 16 * (int)I, 0, 0);
            wb[bf][kk][3] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo + 16 * (int)I + 64, 0, 0);
        }
    };

    // ---- SwiGLU rows [0, nvpad) of the block (all of I) by LDS DMA, their
    // scales, the W2 scales; then the weight stream
    {
        const int ipr = Ld.hrowb >> 10;                   // 1 KB DMA runs per row
        const uint8_t *hrow0 = a.hq + ((int64_t)b * BM + row0) * I;
        for (int q = w; q < nvpad * ipr; q += C::NT / 64) {
            const int row = q / ipr, slot0 = (q - row * ipr) * 64;
            if (slot0 < njb * 8) {
                const int c = (slot0 + lane) ^ (row & 7);
                const int jbl = (c >> 3) < njb ? (c >> 3) : 0;
                lds_dma16(hrow0 + (int64_t)row * I + jbl * 128 + (c & 7) * 16,
                          sH + row * Ld.hrowb + slot0 * 16);
            }
        }
        static_assert(C::RP * C::JMAX <= C::NT, "one row scale per thread");
        float hs = 0.f;
        int hsi = -1;
        if (tid < nvp * njb) {
            const int row = tid / njb, jb = tid - row * njb;
            if (sTok[row] >= 0) {
                hs = a.hs[((int64_t)b * BM + row0 + row) * njb + jb];
                hsi = row * njb + jb;
            }
        }
        float ws = 0.f;
        int wsi = -1;
        const int nwb = nct * 2 * njb;                    // (tile, 128-col block, jb)
        if (tid < nwb) {
            const int tb = tid / njb, jb = tid - tb * njb;     // tb = 2 * tile + col block
            const int64_t cb = (int64_t)ct0 * 2 + tb;
            if (cb * 128 < K) {
                ws = a.w2s[((int64_t)e * (K >> 7) + cb) * njb + jb];
                wsi = tb * njb + jb;
            }
        }
        issue(0, std::integral_constant<int, 0>{});
        issue(1, std::integral_constant<int, 1>{});
        wait_vmcnt<2 * C::LPS>();
        if (hsi >= 0) sHs[hsi] = hs;
        if (wsi >= 0) sWs[wsi] = ws;
    }
    __syncthreads();

    v4f acc[2][C::NU];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int u = 0; u < C::NU; ++u) acc[s][u] = v4f{0.f, 0.f, 0.f, 0.f};

    // units past the stream carry zero scales (their weights read as zeros
    // and the row tile holds finite codes in every K-block slot they touch)
    auto compute = [&](int st, auto BUF) {
        constexpr int bf = decltype(BUF)::value;
#pragma unroll
        for (int kk = 0; kk < C::S; ++kk) {
            const int un = st * C::S + kk;
            const int t = un / njb, jb = un - t * njb;
            const bool live = un < nunits;
            const float sb = live ? sWs[(2 * (live ? t : 0) + (w >> 2)) * njb + jb] : 0.f;
            const u32x4 &a0 = wb[bf][kk][0], &a1 = wb[bf][kk][1];
            const u32x4 &b0 = wb[bf][kk][2], &b1 = wb[bf][kk][3];
            const v8i A0 = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                            (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            const v8i A1 = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                            (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
#pragma unroll
            for (int u = 0; u < C::NU; ++u) {
                if (16 * u >= nvp) break;
                const int row = 16 * u + l16;
                const uint8_t *hp = sH + row * Ld.hrowb + jb * 128;
                const u32x4 lo = lds_read16(hp + ((g ^ (row & 7)) << 4));
                const u32x4 hi = lds_read16(hp + (((4 + g) ^ (row & 7)) << 4));
                const v8i B = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                const float sa = live ? sHs[row * njb + jb] : 0.f;
                if constexpr (E8M0) {
                    const int ea = e8m0_of(sb), eb = e8m0_of(sa);
                    acc[0][u] = mfma16x16x128_e8m0(A0, B, acc[0][u], ea, eb);
                    acc[1][u] = mfma16x16x128_e8m0(A1, B, acc[1][u], ea, eb);
                } else {
                    const float f = sa * sb;
                    acc[0][u] = mfma16x16x128(A0, B) * f + acc[0][u];
                    acc[1][u] = mfma16x16x128(A1, B) * f + acc[1][u];
                }
            }
            if (live && jb == njb - 1) {                // tile t finished: park it
#pragma unroll
                for (int u = 0; u < C::NU; ++u) {
                    if (16 * u >= nvp) break;
                    float *yp = sY + (t * C::RP + 16 * u + l16) * C::YROW + 32 * w + 4 * g;
                    *reinterpret_cast<v4f *>(yp) = acc[0][u];
                    *reinterpret_cast<v4f *>(yp + 16) = acc[1][u];
                    acc[0][u] = v4f{0.f, 0.f, 0.f, 0.f};
                    acc[1][u] = v4f{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    };
    // (pairs of stages, then an odd last one: no exit from the middle of
    // the loop body, which keeps the compiler's own waits at the stage
    // boundaries)
    int st = 0;
    for (; st + 1 < nst; st += 2) {
        wait_vmcnt<C::LPS>();
        compute(st, std::integral_constant<int, 0>{});
        issue(st + 2, std::integral_constant<int, 0>{});
        wait_vmcnt<C::LPS>();
        compute(st + 1, std::integral_constant<int, 1>{});
        issue(st + 3, std::integral_constant<int, 1>{});
    }
    if (st < nst) {
        wait_vmcnt<C::LPS>();
        compute(st, std::integral_constant<int, 0>{});
    }
    __syncthreads();

    // ---- y[r, c] = parked results, valid rows and columns only.  Lanes
    // 16q .. 16q + 15 of a wave hold one row's 64-column group (the trip
    // count is a multiple of 64, so whole waves iterate together).
    for (int idx = tid; idx < nct * nvp * 64; idx += C::NT) {
        const int c4 = idx & 63;
        const int rest = idx >> 6;
        const int row = rest % nvp, t = rest / nvp;
        const int rt = sTok[row];
        const int64_t col = (int64_t)(ct0 + t) * 256 + 4 * c4;
        const bool ok = rt >= 0 && col < K;
        const v4f v = *reinterpret_cast<const v4f *>(sY + (t * C::RP + row) * C::YROW + 4 * c4);
        float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        m = wave_max_xor(m, 1);
        m = wave_max_xor(m, 2);
        m = wave_max_xor(m, 4);
        m = wave_max_xor(m, 8);
        if (!ok) continue;
        float sc, inv;
        y16_scale(m, sc, inv);
        *reinterpret_cast<uint2 *>(a.y16 + (int64_t)rt * K + col) = f32x4_to_f16x4(v, inv);
        if ((c4 & 15) == 0) a.ys[(int64_t)rt * (K >> 6) + (col >> 6)] = sc;
    }
}

__global__ void __launch_bounds__(256)
fill_kernel(uint32_t *__restrict__ p, size_t n, uint32_t v) {
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    size_t stride = (size_t)gridDim.x * 256;
    for (; i < n; i += stride) p[i] = v;
}

// Route sum + accumulate into the BF16 output: four columns of one token per
// thread.  All of the token's route rows are loaded at once (a masked
// route's row is never written, so its value is selected away, not
// multiplied), then added in route order (deterministic), then the previous
// output, then one round to nearest even BF16.
// One thread per 8 consecutive outputs of a token row: 16-byte loads of each
// route's FP16 partials, one scale per route (8 | 64), 16-byte output update.
__global__ void __launch_bounds__(256)
finalize_kernel(uint16_t *__restrict__ out, const uint16_t *__restrict__ y16,
                const float *__restrict__ ys, const float *__restrict__ topk_w,
                const int32_t *__restrict__ rpos, int64_t M, int64_t K, int top_k) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;   // element of out
    if (i >= M * K) return;
    const int64_t t = i / K;
    const int64_t c = i - t * K;
    const uint16_t *src = y16 + t * top_k * K + c;
    const float *ssrc = ys + t * top_k * (K >> 6) + (c >> 6);
    const int32_t *rp = rpos + t * top_k;
    const float *wt = topk_w + t * top_k;
    v4f f0 = v4f{0.f, 0.f, 0.f, 0.f}, f1 = f0;
    for (int j0 = 0; j0 < top_k; j0 += 8) {
        u32x4 v[8];
        float sw[8];
        bool ok[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            ok[q] = false;
            if (j0 + q < top_k) {
                ok[q] = rp[j0 + q] >= 0;
                v[q] = *reinterpret_cast<const u32x4 *>(src + (int64_t)(j0 + q) * K);
                sw[q] = ssrc[(int64_t)(j0 + q) * (K >> 6)] * wt[j0 + q];
            }
        }
        // routes that are not in the plan hold stale rows: select, not multiply
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (ok[q]) {
                f0 += f16x4_to_f32x4(uint2{v[q].x, v[q].y}) * sw[q];
                f1 += f16x4_to_f32x4(uint2{v[q].z, v[q].w}) * sw[q];
            }
    }
    const u32x4 o = *reinterpret_cast<const u32x4 *>(out + i);
    const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
    const float fv[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
    uint32_t rw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float lo = bf16_bits_to_f32(ow[k] & 0xffffu) + fv[2 * k];
        const float hi = bf16_bits_to_f32(ow[k] >> 16) + fv[2 * k + 1];
        rw[k] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
    }
    *reinterpret_cast<u32x4 *>(out + i) = u32x4{rw[0], rw[1], rw[2], rw[3]};
}

template <int BM, bool E8M0>
hipError_t launch_dn(const DownArgs &a, hipStream_t st) {
    int64_t grid = (int64_t)a.nblocks * a.ctiles;
    if (grid == 0) return hipSuccess;
    down_kernel<BM, E8M0><<<(unsigned)grid, DNCfg<BM>::NT, 0, st>>>(a);
    return hipGetLastError();
}

template <int BM, bool E8M0>
hipError_t launch_ds(DownArgs a, hipStream_t st) {
    using C = DSCfg<BM>;
    if (a.njb > C::JMAX) return launch_dn<BM, E8M0>(a, st);   // rows too long for the LDS tile
    // column tiles per workgroup: enough workgroups to cover the chip first
    const int64_t units = (int64_t)a.nblocks * a.ctiles * C::NPASS;
    int nct = (int)(units / 1024);
    nct = nct < 1 ? 1 : (nct > C::NCTMAX ? C::NCTMAX : nct);
    a.nct = nct;
    const int64_t grid = (int64_t)a.nblocks * ((a.ctiles + nct - 1) / nct) * C::NPASS;
    if (grid == 0) return hipSuccess;
    const int lds = DSLayout(C::RP, a.njb, nct, C::YROW).total;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = raise_lds_limit(lds_set, (const void *)down_stream_kernel<BM, E8M0>, 160 * 1024);
    if (e != hipSuccess) return e;
    down_stream_kernel<BM, E8M0><<<(unsigned)grid, C::NT, lds, st>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_down(const DownArgs &a, int block_m, bool e8m0, hipStream_t st) {
    switch (block_m) {
        case 16: return e8m0 ? launch_ds<16, true>(a, st) : launch_ds<16, false>(a, st);
        case 32: return e8m0 ? launch_ds<32, true>(a, st) : launch_ds<32, false>(a, st);
        case 64: return e8m0 ? launch_ds<64, true>(a, st) : launch_ds<64, false>(a, st);
        case 128: return e8m0 ? launch_ds<128, true>(a, st) : launch_ds<128, false>(a, st);
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
