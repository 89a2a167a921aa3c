// The per-plan-block gate/up work item (steps 3 + 4), shared by the
// small-grid gate/up kernel (gateup.hip) and the single-launch expert kernel
// (fused.hip).
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
// Here the weights are the whole cost: a block holds one or two valid rows,
// so the item is a weight stream.  One item = one plan block (its valid
// rows, in passes of at most 64) x one 128-wide intermediate tile (128 gate
// rows + 128 up rows of W13) x one K-range; eight waves take 16 gate and the
// matching 16 up rows each.  The weights go through a ring of one-K-block LDS
// stages filled by global_load_lds_dwordx4, eight lanes per 128-byte row
// segment: every load instruction reads whole 128-byte lines.  (Loading the
// MFMA operand slices straight into registers -- 16 rows x 64 bytes per
// instruction -- streamed the same bytes about 30% slower.)  The stage also
// carries the pass's activation rows and the K-block's scales.
//
// The MMA is the 16x16 tile with weights as the A operand (16 rows) and
// tokens as B (16 columns); lane (l % 16, l / 16) ends with four consecutive
// rows of one token.  Three MMA modes:
//   kExact  (default) E4M3 codes widened exactly to FP16 in registers and
//           multiplied with v_mfma_f32_16x16x32_f16 (exact products, FP32
//           accumulation);
//   kFp8    v_mfma_f32_16x16x128_f8f6f4 on the codes directly;
//   kFp8E8  as kFp8 with power-of-two scales applied inside the MFMA;
//   kW4     E2M1 weights with one power-of-two scale per 32 K (the W4A8
//           variant): each weight row's K32 exponents are taken relative to
//           their largest over the item's K-range, R (found in a prologue);
//           the codes are widened to FP16 with 2^(s - R) folded into the
//           conversion (exact while the row's exponents span at most 23
//           binades: every E2M1 value has two significant bits), multiplied
//           as in kExact with x_s per K-block, and each output row is scaled
//           by 2^(R - 127) once at the end (split partials included).
//
// K is split over items; each writes the partial sums of its valid rows to
// the workspace and the last one of a tile to arrive (atomic counter) adds
// them in split order -- deterministic -- and finishes the tile.
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {
namespace gs {

// kExactE8: the exact path with power-of-two scales folded into the FP16
// widening (2^(a_kb - A) on the activations, 2^(b_kb - B) on W13, A and B the
// largest exponents over this item's K-range) and accumulated across
// K-blocks in the MFMA chain; the sums are scaled by 2^A * 2^B once at the
// end, so split partials share one scale and add as before.
enum { kExact = 0, kFp8 = 1, kFp8E8 = 2, kExactE8 = 3, kW4 = 4 };

template <int BM, int NSO = 0, bool W4 = false>
struct GSCfg {
    static_assert(NSO == 0 || (NSO >= 2 && NSO <= 4), "ring depth 2..4");
    // A pass is one MFMA row tile of RP rows (16..64); it holds RPV plan rows
    // of the block (block_m = 8: the 8 rows of the block, then 8 masked rows).
    static constexpr int RP = BM < 16 ? 16 : (BM < 64 ? BM : 64);
    static constexpr int RPV = BM < RP ? BM : RP;
    static constexpr int NPASS = BM > RP ? BM / RP : 1;
    static constexpr int NU = RP / 16;             // 16-token subtiles
    static constexpr int NT = 512;                 // eight waves
    static constexpr int GROW = 260;               // row stride of the FP32 tile
    // LDS: a ring of NS stages {W13 tile 256 x 128 B, activation rows RP x
    // 128 B, scales: a 16-float run per wave}, reused after the K loop as the
    // FP32 tile [RP][GROW]; then routes, row tokens, a DMA sink, flags.
    // W4: the W13 tile is 256 x 64 B of E2M1 codes and each wave's scale run
    // is 256 B: the K32 exponent dwords of 32 weight rows, then 8 x_s.  With
    // passes of up to 32 rows (EGRP) the exponent dwords instead come four
    // K-blocks at a time into one of two group slots [256 rows][4 K-blocks]
    // outside the ring (decode M=16 steps 3-5 10% faster; with 64-row passes
    // 2.6% slower at page-1 M=1024, so those keep one load per K-block).
    static constexpr int NS = NSO ? NSO : (RP <= 32 ? 4 : 3);
    static constexpr bool EGRP = W4 && RP <= 32;    // exponents in groups of four K-blocks
    static constexpr int WB = 256 * (W4 ? 64 : 128);
    static constexpr int XB = RP * 128;
    static constexpr int SB = W4 ? 8 * 256 : 8 * 16 * 4;
    static constexpr int STB = WB + XB + SB;
    static constexpr int RING = NS * STB;
    static constexpr int GT = RP * GROW * 4;
    static constexpr int TOK = RING > GT ? RING : GT;
    static constexpr int XT = TOK + RP * 4;
    static constexpr int SINK = XT + RP * 4;
    static constexpr int MISC = SINK + 8 * 256;
    static constexpr int EXP = MISC + 16;          // kExactE8: [RP] row, [2] gate/up exponents
    static constexpr int RW = EXP + (RP + 4) * 4;  // kW4: [256] weight-row exponents
    static constexpr int EG = RW + (W4 ? 256 * 4 : 0);  // EGRP: [2][256][4] exponent dwords
    static constexpr int TOTAL = EG + (EGRP ? 2 * 256 * 16 : 0);
    static constexpr int NPS = W4 ? 4 : 6;         // DMA instructions per wave per stage
    static constexpr int NPE = EGRP ? 2 : 0;       // more on stages that start an exponent group
};

// One work item: plan block b, pass `pass` of its rows, j-tile jt, K-split
// `split`.  Every early return is taken by the whole workgroup.  FUSED (the
// single-launch path): the route map is built elsewhere, the intermediate
// rows are stored agent-coherent (write-through, for workgroups on other
// XCDs) and, once a (block, pass, j-tile)'s rows are written, its count in
// cnt_h goes up by one.
template <int BM, int MODE, int NSO, bool FUSED>
__device__ __forceinline__ void gateup_item(const GateUpArgs &a, uint8_t *smem, int b, int split,
                                            int jt, int pass, uint32_t *cnt_h) {
    constexpr bool W4 = MODE == kW4;
    using C = GSCfg<BM, NSO, W4>;
    static_assert(C::TOTAL <= 160 * 1024, "LDS budget");
    float *sG = reinterpret_cast<float *>(smem);    // reuses the ring after the loop
    int *sTok = reinterpret_cast<int *>(smem + C::TOK);    // route of each row, -1 if none
    int *sXt = reinterpret_cast<int *>(smem + C::XT);      // token whose x row fills the row
    uint8_t *sSink = smem + C::SINK;
    int *sMisc = reinterpret_cast<int *>(smem + C::MISC);
    int *sExp = reinterpret_cast<int *>(smem + C::EXP);
    int *sRw = reinterpret_cast<int *>(smem + C::RW);
    uint8_t *sEg = smem + C::EG;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int row0 = pass * C::RP;

    // the plan entries of this pass (every entry below sorted_cap is
    // readable); the block's expert only once the block is known to lie
    // below P (expert_ids may be sized by the plan's blocks_cap)
    int r = -1;
    if (w == 0 && lane < C::RPV) r = a.sorted[(int64_t)b * BM + row0 + lane];
    const int ntp = a.ntp[0];
    if (b * BM >= ntp) return;                          // padded block
    const int e = __builtin_amdgcn_readfirstlane(a.eids[b]);   // uniform: scalar descriptors
    if (e < 0 || e >= a.E) return;

    // this pass's routes (wave 0), the valid-row extent, the inverse plan map
    if (w == 0) {
        if (lane < C::RP) {
            r = (r >= 0 && (int64_t)r < a.R) ? r : -1;
            sTok[lane] = r;
            if (!FUSED && r >= 0 && jt == 0 && split == 0) a.rpos[r] = b * BM + row0 + lane;
        }
        const uint64_t m = __ballot(r >= 0);
        const int nv = m ? 64 - __builtin_clzll(m) : 0;
        const int t = r >= 0 ? r / a.top_k : -1;
        const int tlast = __shfl(t, nv > 0 ? nv - 1 : 0, 64);
        if (lane < C::RP) sXt[lane] = t >= 0 ? t : tlast;
        if (lane == 0) sMisc[0] = nv;
    }
    __syncthreads();
    const int nvp = sMisc[0];                   // rows [0, nvp) hold every valid row
    if (nvp == 0) return;                       // whole pass masked (same for all splits)
    const int nvpad = (nvp + 15) & ~15;

    const int kb0 = split * a.kb_per_split;
    const int kb1 = kb0 + a.kb_per_split < a.nkb ? kb0 + a.kb_per_split : a.nkb;
    const int nk = kb1 - kb0;
    if (nk <= 0) return;
    const int64_t K = a.K, I = a.I;

    // ---- DMA sources of this lane.  Every wave issues NPS instructions per
    // stage (the waits count on it): four W13 segments (8 rows x 128 B each,
    // 16-byte chunks XOR-swizzled by row & 7), one activation segment (rows
    // 8w.., waves w < RP / 8; the others a 4-byte load into a sink), and one
    // scale load (lanes 0-7: x_s of rows 8w..; lanes 8, 9: the gate and up
    // weight-block scales).  Masked and padding rows read the last valid
    // row's token (sXt); their columns are never stored.
    // W4: two W13 segments (16 rows x 64 B each, 16-byte chunks XOR-swizzled
    // by w4_swizzle(row)), the activation segment, and one 4-byte load: lanes
    // 0-31 the K32 exponent dword of weight rows 32w.., lanes 32-39 x_s of rows
    // 8w...  EGRP: lanes 0-31 idle in that load; instead, on stages whose
    // K-block starts a group of four, two more 4-byte loads bring the
    // exponent dwords of weight rows 32w.. for the group's four K-blocks, a
    // row's four dwords from consecutive lanes (one cache line), so a row's
    // exponents cost one line request per four K-blocks.
    const int sub = lane >> 3, slot = lane & 7;
    const uint8_t *wsrc[4];
    if constexpr (W4) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = (w * 2 + i) * 16 + (lane >> 2);          // tile row 0..255
            const int64_t n = (row < 128 ? 0 : I - 128) + (int64_t)jt * 128 + row;
            wsrc[i] = a.w13 + ((int64_t)e * 2 * I + n) * (K >> 1) + (int64_t)kb0 * 64 +
                      ((lane & 3) ^ w4_swizzle(row)) * 16;
        }
        wsrc[2] = wsrc[3] = nullptr;
    } else if (a.w13_packed) {
        // the packed tile is the stage image: each instruction copies 1 KB
        const uint8_t *tile = a.w13 + (((int64_t)e * a.jtiles + jt) * a.nkb + kb0) * kPackedTile;
#pragma unroll
        for (int i = 0; i < 4; ++i) wsrc[i] = tile + (w * 4 + i) * 1024 + lane * 16;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (w * 4 + i) * 8 + sub;                  // tile row 0..255
            const int64_t n = (row < 128 ? 0 : I - 128) + (int64_t)jt * 128 + row;
            wsrc[i] = a.w13 + ((int64_t)e * 2 * I + n) * K + (int64_t)kb0 * 128 + (slot ^ (row & 7)) * 16;
        }
    }
    // bytes between consecutive K-blocks of a weight source
    const int64_t wstep = W4 ? 64 : (a.w13_packed ? kPackedTile : 128);
    const bool xw = w < C::RP / 8;
    const uint8_t *xsrc;
    {
        const int row = xw ? 8 * w + sub : 0;
        xsrc = a.xq + (int64_t)sXt[row] * K + (int64_t)kb0 * 128 + (slot ^ (row & 7)) * 16;
    }
    // 4-byte scale source of this lane, advanced by 4 bytes per K-block
    const uint8_t *ssrc;
    const uint8_t *esrc[2] = {nullptr, nullptr};   // W4: exponent rows 32w + 16i + lane / 4
    if constexpr (W4) {
        if (!C::EGRP && lane < 32) {
            const int row = 32 * w + lane;
            const int64_t n = (row < 128 ? 0 : I - 128) + (int64_t)jt * 128 + row;
            ssrc = a.w13e + ((int64_t)e * 2 * I + n) * (K >> 5) + (int64_t)kb0 * 4;
        } else {
            const int row = 8 * w + (lane & 7) < C::RP ? 8 * w + (lane & 7) : 0;
            ssrc = reinterpret_cast<const uint8_t *>(a.xs + (int64_t)sXt[row] * a.nkb + kb0);
        }
        if constexpr (C::EGRP) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int er = 32 * w + 16 * i + (lane >> 2);
                const int64_t n = (er < 128 ? 0 : I - 128) + (int64_t)jt * 128 + er;
                esrc[i] = a.w13e + ((int64_t)e * 2 * I + n) * (K >> 5) + (int64_t)kb0 * 4;
            }
        }
    } else if (lane < 8) {
        const int row = 8 * w + lane < C::RP ? 8 * w + lane : 0;
        ssrc = reinterpret_cast<const uint8_t *>(a.xs + (int64_t)sXt[row] * a.nkb + kb0);
    } else {
        const int nb13 = (int)(2 * I / 128);
        ssrc = reinterpret_cast<const uint8_t *>(
            a.w13s + ((int64_t)e * nb13 + (lane == 9 ? (int)(I / 128) : 0) + jt) * a.nkb + kb0);
    }
    // An expert with this one plan block streams its W13 tile exactly once:
    // those loads take the non-temporal policy (6.6 against 5.9 TB/s on a
    // 411 MB slab stream); experts with several blocks keep theirs cacheable,
    // for the other blocks' workgroups to find in L2.
    const bool once = (b == 0 || a.eids[b - 1] != e) &&
                      ((int64_t)(b + 1) * BM >= ntp || a.eids[b + 1] != e);
    auto issue = [&](int st, int kbl) {
        uint8_t *base = smem + st * C::STB;
        constexpr int NW = W4 ? 2 : 4;
        if (once) {
#pragma unroll
            for (int i = 0; i < NW; ++i) lds_dma16_nt(wsrc[i] + kbl * wstep, base + (w * NW + i) * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < NW; ++i) lds_dma16(wsrc[i] + kbl * wstep, base + (w * NW + i) * 1024);
        }
        if (xw)
            lds_dma16(xsrc + kbl * 128, base + C::WB + w * 1024);
        else
            lds_dma4(xsrc + kbl * 128, sSink + w * 256);
        if (C::EGRP ? (lane >= 32 && lane < 40) : lane < (W4 ? 40 : 10))
            lds_dma4(ssrc + kbl * 4, base + C::WB + C::XB + w * (C::SB / 8));
        if (C::EGRP && (kbl & 3) == 0) {
            // the group's K-blocks, the last one repeated past the item's range
            const int kq = kbl + (lane & 3) < nk ? kbl + (lane & 3) : nk - 1;
            uint8_t *eg = sEg + ((kbl >> 2) & 1) * (256 * 16);
#pragma unroll
            for (int i = 0; i < 2; ++i) lds_dma4(esrc[i] + kq * 4, eg + (32 * w + 16 * i) * 16);
        }
    };

    if constexpr (MODE == kExactE8) {
        // largest biased exponent over this item's K-range: of each row's
        // activation scales (8 threads a row) and of the gate / up weight
        // scales (waves 0 / 1)
        const int row = tid >> 3, part = tid & 7;
        if (row < C::RP) {
            const float *xs = a.xs + (int64_t)sXt[row] * a.nkb;
            int m = 1;
            for (int kb = kb0 + part; kb < kb1; kb += 8) m = max(m, biased_exp(xs[kb]));
            m = max(m, __shfl_xor(m, 1, 64));
            m = max(m, __shfl_xor(m, 2, 64));
            m = max(m, __shfl_xor(m, 4, 64));
            if (part == 0) sExp[row] = m;
        }
        if (w < 2) {
            const int nb13 = (int)(2 * I / 128);
            const float *ws = a.w13s + ((int64_t)e * nb13 + (w == 1 ? (int)(I / 128) : 0) + jt) * a.nkb;
            int mb = 1;
            for (int kb = kb0 + lane; kb < kb1; kb += 64) mb = max(mb, biased_exp(ws[kb]));
            for (int off = 32; off >= 1; off >>= 1) mb = max(mb, __shfl_xor(mb, off, 64));
            if (lane == 0) sExp[C::RP + w] = mb;
        }
        __syncthreads();
    }
    if constexpr (W4) {
        // largest exponent byte of each W13 row of the tile over [kb0, kb1)
        // (two threads a row, one dword = one K-block's four K32 groups)
        const int row = tid >> 1, half = tid & 1;
        const int64_t n = (row < 128 ? 0 : I - 128) + (int64_t)jt * 128 + row;
        const uint32_t *ep = reinterpret_cast<const uint32_t *>(a.w13e + ((int64_t)e * 2 * I + n) * (K >> 5));
        int m = max_byte_strided(ep, kb0 + half, kb1, 2);
        m = max(m, __shfl_xor(m, 1, 64));
        if (half == 0) sRw[row] = m;
        __syncthreads();
    }

    // kW4: the reference exponents of this lane's gate and up operand rows
    int rwa[2] = {0, 0};
    if constexpr (W4) {
        rwa[0] = sRw[16 * w + l16];
        rwa[1] = sRw[128 + 16 * w + l16];
    }
    v4f accg[C::NU], accu[C::NU];
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
        accg[u] = v4f{0.f, 0.f, 0.f, 0.f};
        accu[u] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    auto compute_w4 = [&](int st, int kbl) {
        const uint8_t *Ws = smem + st * C::STB;
        const uint8_t *Eg = sEg + ((kbl >> 2) & 1) * (256 * 16) + (kbl & 3) * 4;
        const uint8_t *Xs = Ws + C::WB;
        const uint8_t *Sb = Ws + C::WB + C::XB;
        // weight rows: this lane's A rows (gate / up), widened with their
        // K32 scales relative to the row's reference exponent
        v8h W[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 128 * h + 16 * w + l16;
            // whole 16-byte chunks through lds_read16 (typed 16-byte reads
            // are what lets the compiler keep these reads clear of the
            // in-flight LDS refills; 8-byte reads drew a full vmcnt(0) wait
            // every K-block), then this lane group's half of each
            const uint8_t *rp = Ws + row * 64;
            const u32x4 c01 = lds_read16(rp + (((g >> 1) ^ w4_swizzle(row)) << 4));
            const u32x4 c23 = lds_read16(rp + (((2 + (g >> 1)) ^ w4_swizzle(row)) << 4));
            const uint2 d01 = (g & 1) ? uint2{c01.z, c01.w} : uint2{c01.x, c01.y};
            const uint2 d23 = (g & 1) ? uint2{c23.z, c23.w} : uint2{c23.x, c23.y};
            const uint32_t sw = C::EGRP
                ? *reinterpret_cast<const uint32_t *>(Eg + row * 16)
                : *reinterpret_cast<const uint32_t *>(Sb + (row >> 5) * 256 + (row & 31) * 4);
            const int R = rwa[h];
            const int dlo = (int)((sw >> (8 * (g >> 1))) & 0xffu) - R;
            const int dhi = (int)((sw >> (8 * (2 + (g >> 1)))) & 0xffu) - R;
            // below 2^-30 every product rounds to zero in FP16 either way
            const float flo = __uint_as_float((uint32_t)(127 + (dlo < -30 ? -30 : dlo)) << 23);
            const float fhi = __uint_as_float((uint32_t)(127 + (dhi < -30 ? -30 : dhi)) << 23);
            W[h][0] = e2m1x8_to_f16(d01.x, flo);
            W[h][1] = e2m1x8_to_f16(d01.y, flo);
            W[h][2] = e2m1x8_to_f16(d23.x, fhi);
            W[h][3] = e2m1x8_to_f16(d23.y, fhi);
        }
#pragma unroll
        for (int u = 0; u < C::NU; ++u) {
            if (16 * u >= nvp) break;
            const int row = 16 * u + l16;
            const uint8_t *xp = Xs + row * 128;
            const u32x4 lo = lds_read16(xp + ((g ^ (row & 7)) << 4));
            const u32x4 hi = lds_read16(xp + (((4 + g) ^ (row & 7)) << 4));
            const float sa = *reinterpret_cast<const float *>(Sb + (row >> 3) * 256 + 128 + (row & 7) * 4);
            v8h Bh[4];
            e4m3x32_to_f16(lo, hi, Bh);
            const v4f tg = mfma16x16x128_f16(W[0], Bh);
            const v4f tu = mfma16x16x128_f16(W[1], Bh);
            accg[u] = tg * sa + accg[u];
            accu[u] = tu * sa + accu[u];
        }
    };

    auto compute = [&](int st) {
        const uint8_t *Ws = smem + st * C::STB;
        const uint8_t *Xs = Ws + C::WB;
        const float *Ss = reinterpret_cast<const float *>(Ws + C::WB + C::XB);
        const float sg = Ss[8], su = Ss[9];     // wave 0's run
        u32x4 wlo[2], whi[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 128 * h + 16 * w + l16;
            const uint8_t *rp = Ws + row * 128;
            wlo[h] = lds_read16(rp + ((g ^ (row & 7)) << 4));
            whi[h] = lds_read16(rp + (((4 + g) ^ (row & 7)) << 4));
        }
        v8h Wg[4], Wu[4];
        if constexpr (MODE == kExact) {
            e4m3x32_to_f16(wlo[0], whi[0], Wg);
            e4m3x32_to_f16(wlo[1], whi[1], Wu);
        } else if constexpr (MODE == kExactE8) {
            e4m3x32_to_f16(wlo[0], whi[0], Wg, sg * pow2_neg_biased(sExp[C::RP]));
            e4m3x32_to_f16(wlo[1], whi[1], Wu, su * pow2_neg_biased(sExp[C::RP + 1]));
        }
#pragma unroll
        for (int u = 0; u < C::NU; ++u) {
            if (16 * u >= nvp) break;
            const int row = 16 * u + l16;
            const uint8_t *xp = Xs + row * 128;
            const u32x4 lo = lds_read16(xp + ((g ^ (row & 7)) << 4));
            const u32x4 hi = lds_read16(xp + (((4 + g) ^ (row & 7)) << 4));
            const float sa = Ss[(row >> 3) * 16 + (row & 7)];
            if constexpr (MODE == kExactE8) {
                v8h Bh[4];
                e4m3x32_to_f16(lo, hi, Bh, sa * pow2_neg_biased(sExp[row]));
                accg[u] = mfma16x16x128_f16_acc(Wg, Bh, accg[u]);
                accu[u] = mfma16x16x128_f16_acc(Wu, Bh, accu[u]);
            } else if constexpr (MODE == kExact) {
                v8h Bh[4];
                e4m3x32_to_f16(lo, hi, Bh);
                const v4f tg = mfma16x16x128_f16(Wg, Bh);
                const v4f tu = mfma16x16x128_f16(Wu, Bh);
                accg[u] = tg * (sa * sg) + accg[u];
                accu[u] = tu * (sa * su) + accu[u];
            } else {
                const v8i B = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                const v8i Ag = {(int)wlo[0].x, (int)wlo[0].y, (int)wlo[0].z, (int)wlo[0].w,
                                (int)whi[0].x, (int)whi[0].y, (int)whi[0].z, (int)whi[0].w};
                const v8i Au = {(int)wlo[1].x, (int)wlo[1].y, (int)wlo[1].z, (int)wlo[1].w,
                                (int)whi[1].x, (int)whi[1].y, (int)whi[1].z, (int)whi[1].w};
                if constexpr (MODE == kFp8E8) {
                    const int eb = e8m0_of(sa);
                    accg[u] = mfma16x16x128_e8m0(Ag, B, accg[u], e8m0_of(sg), eb);
                    accu[u] = mfma16x16x128_e8m0(Au, B, accu[u], e8m0_of(su), eb);
                } else {
                    accg[u] = mfma16x16x128(Ag, B) * (sa * sg) + accg[u];
                    accu[u] = mfma16x16x128(Au, B) * (sa * su) + accu[u];
                }
            }
        }
    };

    // Ring: stages 0 .. NS-2 up front; step kb waits for its stage (loads
    // complete in issue order, so only the later stages already issued may
    // still be in flight), then a barrier makes the stage visible and frees
    // the slot of kb - 1 for the refill of kb + NS - 1.
#pragma unroll
    for (int s0 = 0; s0 < C::NS - 1; ++s0)
        if (s0 < nk) issue(s0, s0);
    for (int kb = 0; kb < nk; ++kb) {
        // stages kb .. kb + min(NS - 2, ahead) are in flight; all but the
        // later min(NS - 2, ahead) of them must have landed
        // (EGRP: a stage whose K-block starts an exponent group carries NPE
        // more; of two consecutive stages at most one does)
        const int ahead = nk - 1 - kb;
        const bool eg1 = C::EGRP && ((kb + 1) & 3) == 0, eg2 = C::EGRP && ((kb + 2) & 3) == 0;
        if (C::NS > 3 && ahead >= 2) {
            if (eg1 || eg2)
                wait_vmcnt<(C::NS > 3 ? 2 : 1) * C::NPS + C::NPE>();
            else
                wait_vmcnt<(C::NS > 3 ? 2 : 1) * C::NPS>();
        } else if (C::NS > 2 && ahead >= 1) {
            if (eg1)
                wait_vmcnt<C::NPS + C::NPE>();
            else
                wait_vmcnt<C::NPS>();
        } else {
            wait_vmcnt<0>();
        }
        stage_barrier();
        if (kb + C::NS - 1 < nk) issue((kb + C::NS - 1) % C::NS, kb + C::NS - 1);
        if constexpr (W4)
            compute_w4(kb % C::NS, kb);
        else
            compute(kb % C::NS);
    }

    if constexpr (W4) {
        // 2^(R - 127) of the four output rows of this lane (gate, up)
        const int og = 16 * w + 4 * g;
        const v4f Fg = v4f{pow2_int(sRw[og] - 127), pow2_int(sRw[og + 1] - 127),
                           pow2_int(sRw[og + 2] - 127), pow2_int(sRw[og + 3] - 127)};
        const v4f Fu = v4f{pow2_int(sRw[128 + og] - 127), pow2_int(sRw[129 + og] - 127),
                           pow2_int(sRw[130 + og] - 127), pow2_int(sRw[131 + og] - 127)};
#pragma unroll
        for (int u = 0; u < C::NU; ++u) {
            accg[u] = accg[u] * Fg;
            accu[u] = accu[u] * Fu;
        }
    }
    if constexpr (MODE == kExactE8) {
        const float fbg = pow2_biased(sExp[C::RP]), fbu = pow2_biased(sExp[C::RP + 1]);
#pragma unroll
        for (int u = 0; u < C::NU; ++u) {
            const float fa = pow2_biased(sExp[(16 * u + l16) < C::RP ? 16 * u + l16 : 0]);
            accg[u] = (accg[u] * fa) * fbg;
            accu[u] = (accu[u] * fa) * fbu;
        }
    }
    // ---- FP32 tile of the pass: sG[row][n], gate n < 128, up n >= 128
    __syncthreads();                            // every wave is done with the x tile
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
        if (16 * u >= nvp) break;
        float *gp = sG + (16 * u + l16) * C::GROW + 16 * w + 4 * g;
        *reinterpret_cast<v4f *>(gp) = accg[u];
        *reinterpret_cast<v4f *>(gp + 128) = accu[u];
    }
    __syncthreads();

    if (a.nsplit > 1) {
        // Partial sums travel through memory with agent-coherent accesses
        // (sc1: stores write through this XCD's L2, loads miss in it), so the
        // hand-off needs only the stores' completion before the counter
        // bump -- no cache-wide write-back or invalidate.
        const int tile = jt * a.nblocks + b;
        const int sstride = BM * 256 * 4;       // bytes between splits
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.part + (size_t)tile * a.nsplit * BM * 256 + (size_t)row0 * 256), (short)0,
            a.nsplit * sstride, 0x00020000);
        constexpr int kAgent = 16;              // cache policy: sc1
        for (int idx = tid; idx < nvp * 64; idx += C::NT) {
            const int row = idx >> 6, c4 = idx & 63;
            if (sTok[row] >= 0)
                __builtin_amdgcn_raw_buffer_store_b128(
                    *reinterpret_cast<const u32x4 *>(sG + row * C::GROW + 4 * c4), rp,
                    split * sstride + (row * 256 + 4 * c4) * 4, 0, kAgent);
        }
        wait_vmcnt<0>();
        __syncthreads();
        if (tid == 0) {
            const unsigned old = __hip_atomic_fetch_add(&a.cnt[tile * C::NPASS + pass], 1u,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sMisc[1] = old == (unsigned)(a.nsplit - 1);
        }
        __syncthreads();
        if (!sMisc[1]) return;
        for (int idx = tid; idx < nvp * 64; idx += C::NT) {
            const int row = idx >> 6, c4 = idx & 63;
            if (sTok[row] < 0) continue;
            const int off = (row * 256 + 4 * c4) * 4;
            v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < a.nsplit; s0 += 16) {
                u32x4 v[16];
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (s0 + q < a.nsplit)
                        v[q] = __builtin_amdgcn_raw_buffer_load_b128(rp, (s0 + q) * sstride + off, 0, kAgent);
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (s0 + q < a.nsplit) {
                        sum.x += __uint_as_float(v[q].x);
                        sum.y += __uint_as_float(v[q].y);
                        sum.z += __uint_as_float(v[q].z);
                        sum.w += __uint_as_float(v[q].w);
                    }
            }
            *reinterpret_cast<v4f *>(sG + row * C::GROW + 4 * c4) = sum;
        }
        __syncthreads();
    }

    // ---- SwiGLU + per-row 128-group FP8 requantisation: 32 lanes per row
    const bool ue = a.inter_ue8m0 != 0;
    for (int base = 0; base < nvpad * 32; base += C::NT) {
        const int idx = base + tid;
        const int row = idx >> 5, q = idx & 31;
        const float *gp = sG + row * C::GROW + 4 * q;
        const v4f gv = *reinterpret_cast<const v4f *>(gp);
        const v4f uv = *reinterpret_cast<const v4f *>(gp + 128);
        float h[4], amax = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = swiglu(gv[i], uv[i]);
            amax = fmaxf(amax, fabsf(h[i]));
        }
        amax = wave_max_xor(amax, 1);
        amax = wave_max_xor(amax, 2);
        amax = wave_max_xor(amax, 4);
        amax = wave_max_xor(amax, 8);
        amax = wave_max_xor(amax, 16);
        float s, inv;
        group_scale(amax, ue, s, inv);
        if (row < nvp && sTok[row] >= 0) {
            const int64_t p = (int64_t)b * BM + row0 + row;
            const uint32_t code = pack_e4m3x4(h[0] * inv, h[1] * inv, h[2] * inv, h[3] * inv);
            uint32_t *hq = reinterpret_cast<uint32_t *>(a.hq + p * I + (int64_t)jt * 128 + 4 * q);
            if constexpr (FUSED) {
                store_coherent(hq, code);
                if (q == 0) store_coherent(reinterpret_cast<uint32_t *>(a.hs + p * (I >> 7) + jt),
                                           __float_as_uint(s));
            } else {
                *hq = code;
                if (q == 0) a.hs[p * (I >> 7) + jt] = s;
            }
        }
    }
    if constexpr (FUSED) {
        wait_vmcnt<0>();                        // the rows are written through
        __syncthreads();
        if (tid == 0)
            __hip_atomic_fetch_add(&cnt_h[b * C::NPASS + pass], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace gs
}  // namespace moe
