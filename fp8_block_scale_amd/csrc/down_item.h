// The per-plan-block down work item (step 5) and the route-sum helper,
// shared by the small-grid down kernel (down.hip) and the single-launch
// expert kernel (fused.hip).
//
// What is computed (FlashInfer PR #4287, PR summary and the FP32-scale note
// of its final kernel performance section): for plan row p of block b
// (expert e, route r, token t = r / top_k)
//   y[r, c] = sum_jb h_s[p, jb] * w2_s[e, c / 128, jb]
//                    * sum_{j in jb} h_q[p, j] * W2[e, c, j]           (FP32)
//   out[t, c] += topk_weights[r] * y[r, c]
// Each route's row goes to a route-indexed buffer y[r, :] as FP16 values with
// one FP32 scale per 64 columns (amax / 2^15); the route sum (finalize8) adds
// a token's rows in route order and rounds the output once.
#pragma once

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moe {
namespace ds {

// Route sum + accumulate into the BF16 output for 8 consecutive outputs
// [c, c + 8) of token t: 16-byte loads of each route's FP16 partials, one
// scale per route (8 | 64), all of the token's routes loaded at once (a
// masked route's row is never written, so its value is selected away, not
// multiplied), added in route order (deterministic), then the previous
// output, then one round to nearest even BF16, 16-byte output update.
// COHERENT: y, its scales and the route map come from other workgroups of
// the same launch (agent-coherent loads).
template <bool COHERENT>
__device__ __forceinline__ void finalize8(uint16_t *__restrict__ out, const uint16_t *__restrict__ y16,
                                          const float *__restrict__ ys,
                                          const float *__restrict__ topk_w,
                                          const int32_t *__restrict__ rpos, int64_t t, int64_t c,
                                          int64_t K, int top_k) {
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
                const int64_t j = j0 + q;
                if constexpr (COHERENT) {
                    ok[q] = (int)load_coherent(reinterpret_cast<const uint32_t *>(rp + j)) >= 0;
                    const uint64_t *yp = reinterpret_cast<const uint64_t *>(src + j * K);
                    const uint64_t lo = load_coherent(yp), hi = load_coherent(yp + 1);
                    v[q] = u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
                    sw[q] = __uint_as_float(load_coherent(
                                reinterpret_cast<const uint32_t *>(ssrc + j * (K >> 6)))) * wt[j];
                } else {
                    ok[q] = rp[j] >= 0;
                    v[q] = *reinterpret_cast<const u32x4 *>(src + j * K);
                    sw[q] = ssrc[j * (K >> 6)] * wt[j];
                }
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
    uint16_t *op = out + t * K + c;
    const u32x4 o = *reinterpret_cast<const u32x4 *>(op);
    const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
    const float fv[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
    uint32_t rw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float lo = bf16_bits_to_f32(ow[k] & 0xffffu) + fv[2 * k];
        const float hi = bf16_bits_to_f32(ow[k] >> 16) + fv[2 * k + 1];
        rw[k] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
    }
    *reinterpret_cast<u32x4 *>(op) = u32x4{rw[0], rw[1], rw[2], rw[3]};
}

// Bounded wait of one thread until *c >= target.  A valid schedule always
// gets there (the items it waits for hold lower tickets and are running);
// the bound turns a broken invariant into an error flag instead of a hang.
__device__ __forceinline__ bool wait_count(uint32_t *c, uint32_t target, uint32_t *err) {
    for (uint32_t i = 0; i < (1u << 24); ++i) {
        if (load_coherent(c) >= target) return true;
        __builtin_amdgcn_s_sleep(4);
    }
    store_coherent(err, 1u);
    return false;
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
    // A pass is one MFMA row tile of RP rows (16..64) holding RPV plan rows
    // of the block (block_m = 8: the block's 8 rows, then 8 masked rows).
    static constexpr int RP = BM < 16 ? 16 : (BM < 64 ? BM : 64);
    static constexpr int RPV = BM < RP ? BM : RP;
    static constexpr int NPASS = BM > RP ? BM / RP : 1;
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
// The single-launch kernel adds the rows' valid-route counts [RP] and the
// (token, tile) pairs this item completes [RP * nct].
struct DSLayout {
    int hrowb, y, hs, ws, tok, misc, nv, fin, total;
    __host__ __device__ DSLayout(int rp, int njb, int nct, int yrow) {
        hrowb = ((njb + 7) & ~7) * 128;
        y = rp * hrowb;
        hs = y + nct * rp * yrow * 4;
        ws = hs + rp * njb * 4;
        tok = ws + nct * 2 * njb * 4;
        misc = tok + rp * 4;
        nv = misc + 16;
        fin = nv + rp * 4;
        total = fin + rp * nct * 8;
    }
};

// W4 (the W4A8 variant): W2 rows are E2M1 codes with one exponent byte per
// 32 K.  In the mixed-format MFMA an E2M1 A operand holds K [32 g, 32 g + 32)
// in lane group g (one 16-byte load of the row), whose E8M0 scale is that
// lane's byte g of the K-block's exponent dword; the E4M3 B operand keeps
// the layout of the FP8 tile (bytes 0-15: K [16 g, +16), bytes 16-31:
// K [64 + 16 g, +16); measured on gfx950 with one-hot operands), so the
// intermediate rows are read exactly as in the FP8 path, and h_s is
// applied per K-block in FP32 as before.
// One work item: plan block b, row pass `pass`, column group cw (nct tiles
// of 256 output columns).  Every early return is taken by the whole
// workgroup.  FUSED (the single-launch path, f != nullptr): the W2 stream
// starts before the item waits for its block's intermediate rows (cnt_h);
// the rows and scales handed over by other
// workgroups are read agent-coherent, y is written through, and the item
// that brings a (token, tile)'s count of written route rows to the token's
// valid routes adds them into the output (finalize8, route order).
template <int BM, bool E8M0, bool FUSED, bool W4 = false>
__device__ __forceinline__ void down_item(const DownArgs &a, uint8_t *smem, int b, int cw, int pass,
                                          const FusedArgs *f) {
    static_assert(!(W4 && (E8M0 || FUSED)), "W4 runs on the two-stage FP32-scale path");
    using C = DSCfg<BM>;
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

    const int row0 = pass * C::RP;
    const int ct0 = cw * a.nct;
    const int nct = a.ctiles - ct0 < a.nct ? a.ctiles - ct0 : a.nct;

    int r = -1;
    if (w == 0 && lane < C::RPV) r = a.sorted[(int64_t)b * BM + row0 + lane];
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
    const int64_t rows_here = K - (int64_t)ct0 * 256 < (int64_t)nct * 256 ? K - (int64_t)ct0 * 256
                                                                           : (int64_t)nct * 256;
    // bytes per W2 row (E2M1: two codes a byte) and per exponent row (W4)
    const int wrb = W4 ? (int)(I >> 1) : (int)I, erb = (int)(I >> 5);
    const uint8_t *wbase = a.w2 + ((int64_t)e * K + (int64_t)ct0 * 256) * wrb;
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void *)wbase, (short)0, (int)(rows_here * wrb), 0x00020000);
    const int past = (int)(rows_here * wrb);
    __amdgpu_buffer_rsrc_t re = rw;
    if constexpr (W4)
        re = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.w2e + ((int64_t)e * K + (int64_t)ct0 * 256) * erb), (short)0,
            (int)(rows_here * erb), 0x00020000);
    const int epast = (int)(rows_here * erb);
    // subtile 0 of this lane; subtile 1 is 16 rows on
    const int rowoff0 = (32 * w + l16) * wrb + 16 * g;
    const int eoff0 = (32 * w + l16) * erb;
    u32x4 wb[2][C::S][4];
    auto issue = [&](int st, auto BUF) {
        constexpr int bf = decltype(BUF)::value;
#pragma unroll
        for (int kk = 0; kk < C::S; ++kk) {
            const int u = st * C::S + kk;
            const int t = u / njb, jb = u - t * njb;
            if constexpr (W4) {
                // 64 bytes of codes per row and K-block; the exponent dword
                // of the K-block (four K32 groups) in .x
                const int vo = u < nunits ? rowoff0 + (t * 256) * wrb + jb * 64 : past;
                const int eo = u < nunits ? eoff0 + (t * 256) * erb + jb * 4 : epast;
                wb[bf][kk][0] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo, 0, 0);
                wb[bf][kk][1] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo + 16 * wrb, 0, 0);
                wb[bf][kk][2].x = __builtin_amdgcn_raw_buffer_load_b32(re, eo, 0, 0);
                wb[bf][kk][3].x = __builtin_amdgcn_raw_buffer_load_b32(re, eo + 16 * erb, 0, 0);
            } else {
                const int vo = u < nunits ? rowoff0 + (t * 256) * wrb + jb * 128 : past;
                wb[bf][kk][0] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo, 0, 0);
                wb[bf][kk][1] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo + 64, 0, 0);
                wb[bf][kk][2] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo + 16 * wrb, 0, 0);
                wb[bf][kk][3] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo + 16 * wrb + 64, 0, 0);
            }
        }
    };

    // ---- SwiGLU rows [0, nvpad) of the block (all of I) by LDS DMA, their
    // scales, the W2 scales; then the weight stream
    {
        const int ipr = Ld.hrowb >> 10;                   // 1 KB DMA runs per row
        const uint8_t *hrow0 = a.hq + ((int64_t)b * BM + row0) * I;
        float ws = 0.f;
        int wsi = -1;
        const int nwb = W4 ? 0 : nct * 2 * njb;           // (tile, 128-col block, jb)
        if (tid < nwb) {
            const int tb = tid / njb, jb = tid - tb * njb;     // tb = 2 * tile + col block
            const int64_t cb = (int64_t)ct0 * 2 + tb;
            if (cb * 128 < K) {
                ws = a.w2s[((int64_t)e * (K >> 7) + cb) * njb + jb];
                wsi = tb * njb + jb;
            }
        }
        if constexpr (FUSED) {
            // the weights do not depend on this launch: stream them first
            issue(0, std::integral_constant<int, 0>{});
            issue(1, std::integral_constant<int, 1>{});
            if (tid == 0) sMisc[1] = wait_count(f->cnt_h + b * C::NPASS + pass, (uint32_t)njb, f->err);
            __syncthreads();
            if (!sMisc[1]) {                              // gave up (error flag set)
                wait_vmcnt<0>();
                return;
            }
        }
        static_assert(C::RP * C::JMAX <= C::NT, "one row scale per thread");
        // rows past the block's own (block_m = 8) are never read from the
        // workspace: they belong to the next block, or lie past the plan
        const int nvdma = nvpad < C::RPV ? nvpad : C::RPV;
        for (int q = w; q < nvdma * ipr; q += C::NT / 64) {
            const int row = q / ipr, slot0 = (q - row * ipr) * 64;
            if (slot0 < njb * 8) {
                const int c = (slot0 + lane) ^ (row & 7);
                const int jbl = (c >> 3) < njb ? (c >> 3) : 0;
                const uint8_t *src = hrow0 + (int64_t)row * I + jbl * 128 + (c & 7) * 16;
                uint8_t *dst = sH + row * Ld.hrowb + slot0 * 16;
                if constexpr (FUSED)
                    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kCacheAgent);
                else
                    lds_dma16(src, dst);
            }
        }
        float hs = 0.f;
        int hsi = -1;
        if (tid < nvp * njb) {
            const int row = tid / njb, jb = tid - row * njb;
            if (sTok[row] >= 0) {
                const float *hp = a.hs + ((int64_t)b * BM + row0 + row) * njb + jb;
                hs = FUSED ? __uint_as_float(load_coherent(reinterpret_cast<const uint32_t *>(hp))) : *hp;
                hsi = row * njb + jb;
            }
        }
        if constexpr (FUSED) {
            wait_vmcnt<0>();
        } else {
            issue(0, std::integral_constant<int, 0>{});
            issue(1, std::integral_constant<int, 1>{});
            wait_vmcnt<2 * C::LPS>();
        }
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
            if constexpr (W4) {
                const u32x4 &a0 = wb[bf][kk][0], &a1 = wb[bf][kk][1];
                const v8i A0 = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
                const v8i A1 = {(int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w, 0, 0, 0, 0};
                const int ea0 = (int)((wb[bf][kk][2].x >> (8 * g)) & 0xffu);
                const int ea1 = (int)((wb[bf][kk][3].x >> (8 * g)) & 0xffu);
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
                    acc[0][u] = mfma16x16x128_e2m1_e4m3(A0, B, ea0) * sa + acc[0][u];
                    acc[1][u] = mfma16x16x128_e2m1_e4m3(A1, B, ea1) * sa + acc[1][u];
                }
            } else {
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
        const uint2 hv = f32x4_to_f16x4(v, inv);
        uint16_t *yp = a.y16 + (int64_t)rt * K + col;
        float *sp = a.ys + (int64_t)rt * (K >> 6) + (col >> 6);
        if constexpr (FUSED) {
            store_coherent(reinterpret_cast<uint64_t *>(yp), ((uint64_t)hv.y << 32) | hv.x);
            if ((c4 & 15) == 0) store_coherent(reinterpret_cast<uint32_t *>(sp), __float_as_uint(sc));
        } else {
            *reinterpret_cast<uint2 *>(yp) = hv;
            if ((c4 & 15) == 0) *sp = sc;
        }
    }
    if constexpr (FUSED) {
        // y rows are written through; count them per (token, tile) and let
        // the item that completes a (token, tile) add it into the output
        int *sNv = reinterpret_cast<int *>(smem + Ld.nv);
        int2 *sFin = reinterpret_cast<int2 *>(smem + Ld.fin);
        wait_vmcnt<0>();
        if (tid < nvp) {
            const int rt = sTok[tid];
            int nv = 0;
            if (rt >= 0) {
                const int64_t t = rt / a.top_k;
                for (int j = 0; j < a.top_k; ++j)
                    nv += (int)load_coherent(reinterpret_cast<const uint32_t *>(f->rpos + t * a.top_k + j)) >= 0;
            }
            sNv[tid] = nv;
        }
        if (tid == 0) sMisc[2] = 0;
        __syncthreads();
        for (int idx = tid; idx < nvp * nct; idx += C::NT) {
            const int row = idx % nvp, ti = idx / nvp;
            const int rt = sTok[row];
            if (rt < 0) continue;
            const int t = rt / a.top_k;
            const unsigned old = __hip_atomic_fetch_add(&f->cnt_t[(int64_t)t * a.ctiles + ct0 + ti], 1u,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((int)old + 1 == sNv[row]) sFin[atomicAdd(&sMisc[2], 1)] = make_int2(t, ct0 + ti);
        }
        __syncthreads();
        const int nfin = sMisc[2];
        for (int idx = tid; idx < nfin * 32; idx += C::NT) {
            const int2 tc = sFin[idx >> 5];
            const int64_t c = (int64_t)tc.y * 256 + (idx & 31) * 8;
            if (c < K)
                finalize8<true>(f->out, a.y16, a.ys, a.topk_w, f->rpos, tc.x, c, K, a.top_k);
        }
    }
}

}  // namespace ds
}  // namespace moe
