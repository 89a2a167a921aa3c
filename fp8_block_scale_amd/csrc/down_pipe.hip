// Step 5 for large grids: the down-projection GEMM as a persistent kernel
// whose LDS ring (three stages, four with 32-row tiles) runs without a break
// across all of a workgroup's work items.
//
// Same arithmetic as down.hip (FlashInfer PR #4287, PR summary and the FP32
// scale note of its final kernel performance section): for plan row p of
// expert e holding route r,
//   y[r, c] = sum_jb h_s[p, jb] * w2_s[e, c / 128, jb]
//                  * sum_{j in jb} h_q[p, j] * W2[e, c, j]              (FP32)
// written to the route-indexed buffer y[r, :] as FP16 with one FP32 scale per
// 64 columns (the finalize kernel adds a token's routes, times their router
// weights, in route order).
//
// Work items are (row tile, 256 output columns); the row tiles are the ones
// the gate/up prep kernel listed in the workspace (up to 128 consecutive plan
// rows of one expert, or up to 32 when the gate/up stage runs per plan block
// and block_m <= 32).  Items all cost about the same, so the schedule is
// static: the item list is cut into one contiguous range per XCD (workgroup
// i runs on XCD i mod 8), and the XCD's workgroups take its items round
// robin -- at any moment an XCD works on two or three row tiles, whose
// intermediate rows its L2 then holds for all their column tiles.
//
// Pipeline.  A workgroup's items form one sequence of 128-deep steps of the
// intermediate dimension.  Per step a stage holds the W2 tile (256 rows x
// 128 B), the item's intermediate rows (128 x 128 B, contiguous in plan
// order) and a per-wave metadata slot (16 intermediate-row scales, the two
// W2 block scales, 16 route ids), all brought by direct global->LDS loads two
// steps ahead (three with 32-row tiles) -- across item boundaries too, so an
// item's first steps are already in flight while the previous item finishes.
// The W2 tile loads carry the non-temporal cache policy: each W2 tile is read
// by one item (measured at the decode shape, M=16: down stage 49.6 -> 43.8 us
// with 128-row tiles, 40.7 us with 32-row tiles; page-1 M=4096 unchanged).  Rows are XOR-swizzled
// in LDS (the intermediate rows as in the gate/up pipeline, the W2 rows by
// w2_swizzle below).  FP8 MFMA (v_mfma_f32_16x16x128_f8f6f4) with the FP32
// scale product applied per step, or with power-of-two scales as E8M0
// exponents inside the MFMA.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kNT = 512;
constexpr int kMeta = 64;                     // floats per wave and stage
constexpr int kMetaRt = 18;                   // route ids start here

// W4 (the W4A8 variant): a stage's W2 tile is 256 rows x 64 B of E2M1 codes
// (four 16-byte chunks, one per K32 group, stored at chunk c ^ ((r >> 4) & 3)
// so that the 16 rows of an operand read phase hit distinct banks) plus the
// rows' exponent dwords; lane group g of an operand takes chunk g of its row
// and byte g of the row's dword as the E8M0 A scale of the mixed-format MFMA.
// RT: rows of a row tile, 128 or (for row tiles of at most 32 rows, cut
// when the gate/up stage runs per plan block) 32.  The small tile leaves LDS
// for more stages in flight: four of W2 (FP8) instead of three.  With RT = 32
// a stage's 4 KB of intermediate rows is one DMA instruction per wave over
// its first 32 lanes.
template <bool W4, int RT>
struct DPCfg {
    static constexpr int Rows = RT;
    static constexpr int WBytes = 256 * (W4 ? 64 : 128);
    static constexpr int EBytes = W4 ? 256 * 4 : 0;
    static constexpr int HBytes = RT * 128;
    static constexpr int WInstr = WBytes / 1024 / 8;
    static constexpr int HInstr = RT == 32 ? 1 : HBytes / 1024 / 8;
    static constexpr int HRowsPerWave = HBytes / 8 / 128;     // 16 (RT 128) or 4 (RT 32)
    static constexpr int NU = RT / 32;                        // 16-row subtiles per wave
    static constexpr int PerStage = WInstr + HInstr + 1 + (W4 ? 1 : 0);
    static constexpr size_t StageBytes = (size_t)WBytes + HBytes + EBytes + 8 * kMeta * 4;
    static constexpr int Stages = RT == 32 ? 4 : 3;
    static constexpr size_t Smem = (size_t)Stages * StageBytes;
    static_assert(RT == 32 || RT == 128, "row tiles of 32 or 128 rows");
    static_assert(Smem <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ v8i join8q(const u32x4 &lo, const u32x4 &hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}


// The row-tile list and the plan's expert ids do not change while the
// kernel runs: read through the constant address space, a uniform index
// becomes a scalar load, which does not join the vector loads' in-order
// count (a vector load here would wait for the whole ring).
typedef const __attribute__((address_space(4))) int32_t *const_i32_p;

struct Item {
    int b, nb, e, ct;
    bool ok;            // expert id in range (else: loads from expert 0, nothing computed)
};

// W2 tile rows in LDS: the eight 16-byte chunks of row r sit XOR-swizzled
// by this value.  MFMA operand s of wave wn takes tile rows 64 wn + 16 (m / 4)
// + 4 s + m % 4 for its 16 operand rows m, so that output lane group g holds
// 16 consecutive columns (64 wn + 16 g ..) and a route row leaves in whole
// 16-byte stores; over each 16-lane read phase this swizzle puts the 8 rows
// of either parity on 8 distinct chunks (no bank conflicts).
__device__ __forceinline__ int w2_swizzle(int r) { return (r ^ (r >> 3) ^ (r >> 4)) & 7; }

template <int BM, bool E8M0, bool W4, int RT, bool NT>
__global__ void __launch_bounds__(kNT, 1)
down_pipe_kernel(DownArgs a) {
    using C = DPCfg<W4, RT>;
    constexpr int NS = C::Stages;
    constexpr int HALF = RT / 2;                  // rows of a wm half
    static_assert(!(W4 && E8M0), "W4 takes FP32 intermediate scales");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *sW = smem;                                            // [NS][256][128 or 64]
    uint8_t *sH = smem + NS * C::WBytes;                           // [NS][RT][128]
    uint8_t *sE = sH + NS * C::HBytes;                             // W4: [NS][256] dwords
    float *sMeta = reinterpret_cast<float *>(sE + NS * C::EBytes); // [NS][8][kMeta]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = w & 3, wm = w >> 2;
    const int l16 = lane & 15, g = lane >> 4;
    const int sub = lane >> 3, slot = lane & 7;
    const int64_t I = a.I, K = a.K;
    const int njb = a.njb;

    // ---- static schedule: this workgroup's items are lo + j + k * nwg < hi
    const int64_t N = (int64_t)((const_i32_p)a.tmeta)[0] * a.ctiles;
    const int grid = (int)gridDim.x;
    const int ndom = grid < 8 ? grid : 8;
    const int d = (int)blockIdx.x % ndom, j = (int)blockIdx.x / ndom;
    const int nwg = (grid - d + ndom - 1) / ndom;
    const int64_t lo = N * d / ndom, hi = N * (d + 1) / ndom;
    const int64_t mine = hi - lo > j ? (hi - lo - j + nwg - 1) / nwg : 0;
    const int64_t T = mine * njb;                    // steps
    if (T == 0) return;

    auto item_at = [&](int64_t k) {
        const int64_t item = lo + j + k * nwg;
        const int rt = __builtin_amdgcn_readfirstlane((int)(item / a.ctiles));
        Item it;
        it.ct = __builtin_amdgcn_readfirstlane((int)(item - (int64_t)rt * a.ctiles));
        const const_i32_p tl = (const_i32_p)a.tiles + 4 * (int64_t)rt;   // {first block, blocks, expert, 0}
        it.b = __builtin_amdgcn_readfirstlane(tl[0]);
        it.nb = __builtin_amdgcn_readfirstlane(tl[1]);
        const int e = __builtin_amdgcn_readfirstlane(tl[2]);
        it.ok = e >= 0 && e < a.E;
        it.e = it.ok ? e : 0;
        return it;
    };

    // ---- load side: item and step of the next refill, and this lane's sources
    int64_t kl = 0;
    int jl = 0;
    Item il = item_at(0);
    // (fixed sizes: a local array whose size depends on the template
    // parameters keeps hipcc's host pass from emitting the kernel's stub)
    const uint8_t *wsrc[4];
    const uint8_t *hsrc[2];
    const uint8_t *msrc;
    const uint8_t *esrc = nullptr;                  // W4: exponent dword of row 32w + lane (lanes < 32)
    int mstep;
    auto set_sources = [&](const Item &it) {
        const int nrows = it.nb * BM;
        const int64_t p0 = (int64_t)it.b * BM;
        const int64_t c0 = (int64_t)it.ct * 256;
        const int ncols = K - c0 < 256 ? (int)(K - c0) : 256;     // 128 or 256
        if constexpr (W4) {
#pragma unroll
            for (int i = 0; i < C::WInstr; ++i) {
                const int row = (w * C::WInstr + i) * 16 + (lane >> 2);   // 0..255
                const int64_t c = c0 + (row < ncols ? row : 0);
                wsrc[i] = a.w2 + ((int64_t)it.e * K + c) * (I >> 1) + ((lane & 3) ^ ((row >> 4) & 3)) * 16;
            }
            const int row = 32 * w + (lane & 31);
            const int64_t c = c0 + (row < ncols ? row : 0);
            esrc = a.w2e + ((int64_t)it.e * K + c) * (I >> 5);
        } else {
#pragma unroll
            for (int i = 0; i < C::WInstr; ++i) {
                const int row = (w * C::WInstr + i) * 8 + sub;              // 0..255
                const int64_t c = c0 + (row < ncols ? row : 0);
                wsrc[i] = a.w2 + ((int64_t)it.e * K + c) * I + (slot ^ w2_swizzle(row)) * 16;
            }
        }
#pragma unroll
        for (int i = 0; i < C::HInstr; ++i) {
            const int row = w * C::HRowsPerWave + i * 8 + sub;      // RT 32: lanes < 32 only
            const int64_t p = p0 + (row < nrows ? row : 0);
            hsrc[i] = a.hq + p * I + (slot ^ (row & 7)) * 16;
        }
        // metadata slot of wave w: [0, 16) scales of rows 16w.., [16, 18) the
        // W2 block scales of the item's two 128-column blocks, [18, 34) route
        // ids of rows 16w..
        if (lane < 16) {
            const int row = w * 16 + lane;
            msrc = reinterpret_cast<const uint8_t *>(a.hs + (p0 + (row < nrows ? row : 0)) * njb);
            mstep = 4;
        } else if (lane < kMetaRt) {
            // the W2 block scales (W4: none; the slot re-reads a row scale)
            const int64_t blk = (c0 >> 7) + (lane == 17 && ncols > 128 ? 1 : 0);
            msrc = W4 ? reinterpret_cast<const uint8_t *>(a.hs + p0 * njb)
                      : reinterpret_cast<const uint8_t *>(a.w2s + ((int64_t)it.e * (K >> 7) + blk) * njb);
            mstep = 4;
        } else {
            const int row = w * 16 + lane - kMetaRt;                  // lanes past 33 load nothing
            msrc = reinterpret_cast<const uint8_t *>(a.sorted + p0 + (row < nrows ? row : 0));
            mstep = 0;
        }
    };
    set_sources(il);
    auto issue = [&](int stage) {
        uint8_t *dw = sW + stage * C::WBytes + (w * C::WInstr) * 1024;
#pragma unroll
        for (int i = 0; i < C::WInstr; ++i) {
            if constexpr (NT) lds_dma16_nt(wsrc[i] + (int64_t)jl * (W4 ? 64 : 128), dw + i * 1024);
            else lds_dma16(wsrc[i] + (int64_t)jl * (W4 ? 64 : 128), dw + i * 1024);
        }
        if constexpr (W4)
            if (lane < 32) lds_dma4(esrc + jl * 4, sE + stage * C::EBytes + w * 128);
        uint8_t *dh = sH + stage * C::HBytes + w * C::HRowsPerWave * 128;
        if constexpr (RT == 32) {
            if (lane < 32) lds_dma16(hsrc[0] + (int64_t)jl * 128, dh);
        } else {
#pragma unroll
            for (int i = 0; i < C::HInstr; ++i) lds_dma16(hsrc[i] + (int64_t)jl * 128, dh + i * 1024);
        }
        if (lane < kMetaRt + 16) lds_dma4(msrc + jl * mstep, sMeta + (stage * 8 + w) * kMeta);
        if (++jl == njb && kl + 1 < mine) {
            jl = 0;
            il = item_at(++kl);
            set_sources(il);
        }
    };

    // ---- multiply side
    int64_t kc = 0;
    int jc = 0;
    Item ic = il;
    constexpr int NU = C::NU;
    v4f acc[4][NU];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < NU; ++u) acc[s][u] = v4f{0.f, 0.f, 0.f, 0.f};

    // One step: wait for its stage, barrier, refill the stage the previous
    // step used (every wave is past that multiply), multiply; on an item's
    // last step store its rows.  Loads complete in issue order, so after the
    // refill of step t only the refill of step t + 1 may still be in flight.
    // (An L2 prefetch of the W2 lines a step ahead of the refill, with 4-byte
    // LDS-DMA touches, made the kernel slower: each touch costs the address
    // unit a whole cache line.)  The stage indices are compile-time constants
    // so the compiler can tell the refilled and the read LDS ranges apart.
    auto step = [&](auto st_c, int64_t t) {
        constexpr int ST = decltype(st_c)::value;
        // stages t + 1 .. t + NS - 2 (those issued) may still be in flight
        const int64_t ahead = T - 1 - t;
        if (ahead >= NS - 2)
            wait_vmcnt<(NS - 2) * C::PerStage>();
        else if (ahead == 2)
            wait_vmcnt<2 * C::PerStage>();
        else if (ahead == 1)
            wait_vmcnt<C::PerStage>();
        else
            wait_vmcnt<0>();
        stage_barrier();
        if (t + NS - 1 < T) issue((ST + NS - 1) % NS);

        const int nrows = ic.nb * BM;
        const int64_t c0 = (int64_t)ic.ct * 256;
        const int ncols = K - c0 < 256 ? (int)(K - c0) : 256;
        const bool wave_on = ic.ok && (wm * HALF < nrows) && (64 * wn < ncols);
        const float *meta = sMeta + ST * 8 * kMeta;
        // rows of this wave up to its last valid one (route ids come with
        // every stage): 16-row subtiles past it hold only plan padding and
        // are not multiplied
        int vrows = 0;
        if (wave_on) {
            const int row = wm * HALF + lane;
            const int r = __float_as_int(meta[(row >> 4) * kMeta + kMetaRt + (row & 15)]);
            const uint64_t v = __ballot(lane < HALF && row < nrows && r >= 0 && (int64_t)r < a.R);
            vrows = v ? wm * HALF + 64 - __builtin_clzll(v) : 0;
            vrows = __builtin_amdgcn_readfirstlane(vrows);
        }
        if (W4 && vrows > 0) {
            const uint8_t *Ws = sW + ST * C::WBytes;
            const uint8_t *Hs = sH + ST * C::HBytes;
            const uint8_t *Es = sE + ST * C::EBytes;
            v8i wq[4];
            int ea[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = 64 * wn + 16 * (l16 >> 2) + 4 * s + (l16 & 3);
                const u32x4 c4 = lds_read16(Ws + row * 64 + ((g ^ ((row >> 4) & 3)) * 16));
                wq[s] = v8i{(int)c4.x, (int)c4.y, (int)c4.z, (int)c4.w, 0, 0, 0, 0};
                ea[s] = (int)((*reinterpret_cast<const uint32_t *>(Es + row * 4) >> (8 * g)) & 0xffu);
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (wm * HALF + u * 16 >= vrows) continue;
                const int row = wm * HALF + u * 16 + l16;
                const uint8_t *rp = Hs + row * 128;
                const u32x4 lo4 = lds_read16(rp + ((g ^ (row & 7)) * 16));
                const u32x4 hi4 = lds_read16(rp + (((4 + g) ^ (row & 7)) * 16));
                const v8i B = join8q(lo4, hi4);
                const float sa = meta[(row >> 4) * kMeta + (row & 15)];
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc[s][u] = mfma16x16x128_e2m1_e4m3(wq[s], B, ea[s]) * sa + acc[s][u];
            }
        } else if (vrows > 0) {
            // this wave's 64 columns lie in one 128-column scale block
            const float sb = meta[w * kMeta + 16 + (wn >= 2 ? 1 : 0)];
            const uint8_t *Ws = sW + ST * C::WBytes;
            const uint8_t *Hs = sH + ST * C::HBytes;
            v8i wq[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = 64 * wn + 16 * (l16 >> 2) + 4 * s + (l16 & 3);
                const uint8_t *rp = Ws + row * 128;
                const u32x4 lo4 = lds_read16(rp + ((g ^ w2_swizzle(row)) * 16));
                const u32x4 hi4 = lds_read16(rp + (((4 + g) ^ w2_swizzle(row)) * 16));
                wq[s] = join8q(lo4, hi4);
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (wm * HALF + u * 16 >= vrows) continue;
                const int row = wm * HALF + u * 16 + l16;
                const uint8_t *rp = Hs + row * 128;
                const u32x4 lo4 = lds_read16(rp + ((g ^ (row & 7)) * 16));
                const u32x4 hi4 = lds_read16(rp + (((4 + g) ^ (row & 7)) * 16));
                const v8i B = join8q(lo4, hi4);
                const float sa = meta[(row >> 4) * kMeta + (row & 15)];
                if constexpr (E8M0) {
                    const int ea = e8m0_of(sb), eb = e8m0_of(sa);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        acc[s][u] = mfma16x16x128_e8m0(wq[s], B, acc[s][u], ea, eb);
                } else {
                    const float f = sa * sb;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        v4f tt = mfma16x16x128(wq[s], B);
                        acc[s][u] = tt * f + acc[s][u];
                    }
                }
            }
        }
        if (jc + 1 < njb) {
            ++jc;
            return;
        }
        // last step of the item: its route ids came with this stage; rows go
        // out as FP16 with one scale per (route, this wave's 64 columns)
        if (wave_on) {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int row = wm * HALF + u * 16 + l16;
                float m = 0.f;
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(acc[s][u][i]));
                m = wave_max_xor(m, 16);
                m = wave_max_xor(m, 32);
                if (row >= nrows) continue;
                const int r = __float_as_int(meta[(row >> 4) * kMeta + kMetaRt + (row & 15)]);
                if (r < 0 || (int64_t)r >= a.R) continue;
                float sc, inv;
                y16_scale(m, sc, inv);
                // the lane's 16 columns are consecutive: two 16-byte stores
                uint16_t *dst = a.y16 + (int64_t)r * K + c0 + 64 * wn + 16 * g;
#pragma unroll
                for (int s = 0; s < 4; s += 2) {
                    const uint2 lo = f32x4_to_f16x4(acc[s][u], inv), hi = f32x4_to_f16x4(acc[s + 1][u], inv);
                    *reinterpret_cast<uint4 *>(dst + 4 * s) = uint4{lo.x, lo.y, hi.x, hi.y};
                }
                if (g == 0) a.ys[(int64_t)r * (K >> 6) + ((c0 >> 6) + wn)] = sc;
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int u = 0; u < NU; ++u) acc[s][u] = v4f{0.f, 0.f, 0.f, 0.f};
        if (kc + 1 < mine) {
            jc = 0;
            ic = item_at(++kc);
        }
    };

    for (int q = 0; q < NS - 1; ++q)
        if (q < T) issue(q);
    for (int64_t t = 0; t < T; t += NS) {
        step(std::integral_constant<int, 0>{}, t);
        if (t + 1 < T) step(std::integral_constant<int, 1>{}, t + 1);
        if (t + 2 < T) step(std::integral_constant<int, 2>{}, t + 2);
        if constexpr (NS > 3)
            if (t + 3 < T) step(std::integral_constant<int, 3>{}, t + 3);
    }
    wait_vmcnt<0>();                                 // no load may land after the workgroup ends
}

template <int BM, bool E8M0, bool W4, int RT, bool NT>
hipError_t launch_dn_pipe(const DownArgs &a, hipStream_t st) {
    if (a.nblocks == 0) return hipSuccess;
    int64_t grid = device_cu_count();
    const int64_t max_items = (int64_t)a.nblocks * a.ctiles;
    if (grid > max_items) grid = max_items;
    static std::atomic<uint64_t> lds_set{0};
    constexpr size_t smem = DPCfg<W4, RT>::Smem;
    hipError_t e = raise_lds_limit(lds_set, (const void *)down_pipe_kernel<BM, E8M0, W4, RT, NT>, (int)smem);
    if (e != hipSuccess) return e;
    down_pipe_kernel<BM, E8M0, W4, RT, NT><<<(unsigned)grid, kNT, smem, st>>>(a);
    return hipGetLastError();
}

// 128-row tiles: non-temporal W2 loads when an expert's routes fit one row
// tile on average (each W2 tile is then read once), the default policy when
// several row tiles of one expert re-read it (measured: NT everywhere made
// the down stage 18% slower at 8192 tokens, 228 routes per expert).
template <int BM, bool E8M0, bool W4>
hipError_t launch_dn_big(const DownArgs &a, bool nt, hipStream_t st) {
    return nt ? launch_dn_pipe<BM, E8M0, W4, 128, true>(a, st) : launch_dn_pipe<BM, E8M0, W4, 128, false>(a, st);
}

bool stream_once(const DownArgs &a) { return a.R <= (int64_t)64 * a.E; }

}  // namespace

hipError_t launch_down_pipe_w4(const DownArgs &a, int block_m, bool small, hipStream_t st) {
    if (small) {
        switch (block_m) {
            case 8: return launch_dn_pipe<8, false, true, 32, true>(a, st);
            case 16: return launch_dn_pipe<16, false, true, 32, true>(a, st);
            case 32: return launch_dn_pipe<32, false, true, 32, true>(a, st);
            default: return hipErrorInvalidValue;
        }
    }
    const bool nt = stream_once(a);
    switch (block_m) {
        case 8: return launch_dn_big<8, false, true>(a, nt, st);
        case 16: return launch_dn_big<16, false, true>(a, nt, st);
        case 32: return launch_dn_big<32, false, true>(a, nt, st);
        case 64: return launch_dn_big<64, false, true>(a, nt, st);
        case 128: return launch_dn_big<128, false, true>(a, nt, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_down_pipe(const DownArgs &a, int block_m, bool e8m0, bool small, hipStream_t st) {
    if (small) {
        switch (block_m) {
            case 8: return e8m0 ? launch_dn_pipe<8, true, false, 32, true>(a, st) : launch_dn_pipe<8, false, false, 32, true>(a, st);
            case 16: return e8m0 ? launch_dn_pipe<16, true, false, 32, true>(a, st) : launch_dn_pipe<16, false, false, 32, true>(a, st);
            case 32: return e8m0 ? launch_dn_pipe<32, true, false, 32, true>(a, st) : launch_dn_pipe<32, false, false, 32, true>(a, st);
            default: return hipErrorInvalidValue;
        }
    }
    const bool nt = stream_once(a);
    switch (block_m) {
        case 8: return e8m0 ? launch_dn_big<8, true, false>(a, nt, st) : launch_dn_big<8, false, false>(a, nt, st);
        case 16: return e8m0 ? launch_dn_big<16, true, false>(a, nt, st) : launch_dn_big<16, false, false>(a, nt, st);
        case 32: return e8m0 ? launch_dn_big<32, true, false>(a, nt, st) : launch_dn_big<32, false, false>(a, nt, st);
        case 64: return e8m0 ? launch_dn_big<64, true, false>(a, nt, st) : launch_dn_big<64, false, false>(a, nt, st);
        case 128: return e8m0 ? launch_dn_big<128, true, false>(a, nt, st) : launch_dn_big<128, false, false>(a, nt, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
