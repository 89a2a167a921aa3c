// Steps 3 + 4 for large grids: the gate/up tile kernel with a three-stage
// LDS pipeline fed by direct global->LDS loads.
//
// Same arithmetic as gateup.hip (FlashInfer PR #4287, PR summary and
// public-contract section): per plan row, the gate/up sums over 128-deep
// K-blocks with one activation scale and one 128x128 weight-block scale per
// K-block, SwiGLU, and FP8 requantisation per row and 128-column group.
//
// Tiling.  A work item is up to 128 consecutive plan rows that belong to one
// expert -- several plan blocks when block_m < 128 -- times one 128-wide
// intermediate tile (its 128 gate and 128 up rows of W13), so the W13 tile is
// streamed once for all of the expert's rows it covers.  A one-workgroup
// prep kernel cuts every expert's run of plan blocks into such row tiles
// (a list in the workspace); the gate/up kernel is persistent -- one
// workgroup (8 waves) per CU -- and pulls items from a device-wide counter
// until none are left, so no workgroup is launched only to exit and the
// per-launch set-up is paid once per CU.  The counter is one per XCD: each
// XCD works through its own share of the row tiles, all j-tiles of a row
// tile back to back, so the tile's gathered activation rows come from that
// XCD's L2 after the first fetch; idle XCDs take over the others' leftovers.
//
// Pipeline.  Each K-block stage holds the W13 tile (256 rows x 128 B) and the
// gathered activation tile (128 rows x 128 B) in LDS; all waves issue
// global_load_lds_dwordx4 (64 lanes x 16 B straight into LDS, no registers)
// two stages ahead of the one being multiplied, so ~96 KB per CU are in
// flight while the MFMAs run.  Rows are stored with their eight 16-byte
// chunks XOR-swizzled by (row & 7), so the MFMA operand reads (16 rows at one
// chunk) hit distinct banks.  Waves: wn = 0..3 take 32 gate + 32 up columns,
// wm = 0..1 take 64 rows each.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kRows = 128;        // tile rows
constexpr int kNT = 512;          // threads (8 waves)
constexpr int kStages = 3;
constexpr int kABytes = kRows * 128;          // activation tile per stage
constexpr int kAInstr = kABytes / 1024 / 8;   // DMA instructions per wave per stage (A)
constexpr int kSGroup = 4;                    // K-blocks of activation scales per scale load
constexpr int kMaxKb = 256;                   // K <= 32768

// kExactE8: the exact path with power-of-two scales folded into the FP16
// widening (2^(a_kb - A) on the activations, 2^(b_kb - B) on W13, A and B
// the largest exponents over K) and accumulated across K-blocks in the MFMA
// chain; the item's sums are scaled by 2^A * 2^B once, before SwiGLU.
// kW4 (the W4A8 variant): E2M1 W13 with K32 exponent bytes; a stage holds
// 256 rows x 64 B of codes (16-byte chunks XOR-swizzled by w4_swizzle(row))
// and the rows' exponent dwords.  Each weight row's largest exponent R over K is found
// once per item; the codes are widened to FP16 with 2^(s - R) folded in
// (exact while a row's exponents span at most 23 binades), the K-block sums
// take x_s as in kExact, and each output row is scaled by 2^(R - 127) once,
// before SwiGLU.
enum { kExact = 0, kFp8 = 1, kFp8E8 = 2, kExactE8 = 3, kW4 = 4 };

template <int MODE>
struct PCfg {
    static constexpr bool W4 = MODE == kW4;
    static constexpr int WBytes = 256 * (W4 ? 64 : 128);    // W13 tile per stage
    static constexpr int EBytes = W4 ? 256 * 4 : 0;          // exponent dwords per stage
    static constexpr int WInstr = WBytes / 1024 / 8;         // DMA instructions per wave per stage (W)
    // + 1 on K-blocks that start a scale group
    static constexpr int PerStage = WInstr + kAInstr + (W4 ? 1 : 0);
    static constexpr size_t Smem = (size_t)kStages * (WBytes + kABytes + EBytes) +
                                   2 * kRows * kSGroup * 4 + 2 * kMaxKb * 4 + kRows * 4 +
                                   4 * kRows * 4 + 16 + (kRows + 4) * 4 + (W4 ? 256 * 4 : 0);
    static_assert(Smem <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ v8i join8p(const u32x4 &lo, const u32x4 &hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// Row tiles: every expert's run of blocks [first, first + len) (expert ids of
// a plan are non-decreasing) becomes ceil(len / mb) tiles of <= mb blocks,
// each listed as {first block, blocks, expert, 0}.
// One workgroup: pass 1 marks run starts and counts their tiles, an
// exclusive scan gives each run its first tile slot, pass 2 writes them.
__device__ __forceinline__ void tiles_body(const int32_t *__restrict__ eids,
                                           const int32_t *__restrict__ ntp, int bm, int mb,
                                           int nblocks, int4 *__restrict__ tiles,
                                           int32_t *__restrict__ meta) {
    __shared__ int wsum[16];
    __shared__ int carry;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int nb = ntp[0] / bm;
    nb = nb < nblocks ? nb : nblocks;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < nb; base += 1024) {
        const int b = base + tid;
        int cnt = 0, len = 0, e = 0;
        if (b < nb) {
            e = eids[b];
            if (b == 0 || eids[b - 1] != e) {
                len = 1;
                while (b + len < nb && eids[b + len] == e) ++len;
                cnt = (len + mb - 1) / mb;
            }
        }
        int incl = cnt;
        for (int d = 1; d < 64; d <<= 1) {
            int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        if (lane == 63) wsum[w] = incl;
        __syncthreads();
        int before = carry;
        for (int q = 0; q < w; ++q) before += wsum[q];
        int slot = before + incl - cnt;
        for (int t = 0; t < cnt; ++t) {
            const int first = b + t * mb;
            const int rem = len - t * mb;
            tiles[slot + t] = make_int4(first, rem < mb ? rem : mb, e, 0);
        }
        __syncthreads();
        if (tid == 1023) carry = before + incl;
        __syncthreads();
    }
    if (tid == 0) meta[0] = carry;     // number of row tiles
    if (tid >= 1 && tid <= 8) meta[tid] = 0;    // per-XCD work counters of the gate/up queues
}

// The row tiles (workgroup 0) and the stage's set-up in the same launch
// (workgroups 1..): the route map rpos[0, n_rpos) = -1 and the split-K
// counters cnt[0, n_cnt) = 0.
__global__ void __launch_bounds__(1024)
tiles_kernel(const int32_t *__restrict__ eids, const int32_t *__restrict__ ntp, int bm, int mb,
             int nblocks, int4 *__restrict__ tiles, int32_t *__restrict__ meta,
             uint32_t *__restrict__ rpos, int64_t n_rpos, uint32_t *__restrict__ cnt, int64_t n_cnt) {
    if (blockIdx.x == 0) {
        tiles_body(eids, ntp, bm, mb, nblocks, tiles, meta);
        return;
    }
    const int64_t stride = (int64_t)(gridDim.x - 1) * 1024;
    for (int64_t i = (int64_t)(blockIdx.x - 1) * 1024 + threadIdx.x; i < n_rpos + n_cnt; i += stride) {
        if (i < n_rpos) rpos[i] = 0xffffffffu;
        else cnt[i - n_rpos] = 0u;
    }
}

// workgroups of the set-up part of tiles_kernel
unsigned prep_groups(int64_t n) {
    int64_t g = (n + 1023) / 1024;
    return (unsigned)(g > 256 ? 256 : g);
}

template <int BM, int MODE>
__global__ void __launch_bounds__(kNT, 1)
gateup_pipe_kernel(GateUpArgs a) {
    using C = PCfg<MODE>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *sW = smem;                                        // [kStages][256][128 or 64]
    uint8_t *sA = smem + kStages * C::WBytes;                  // [kStages][128][128]
    uint8_t *sE = sA + kStages * kABytes;                      // kW4: [kStages][256] exponent dwords
    float *sSa = reinterpret_cast<float *>(sE + kStages * C::EBytes);  // [2][128][kSGroup] x_s
    float *sSw = sSa + 2 * kRows * kSGroup;                    // [2][kMaxKb] w13_s gate, up
    int *sTok = reinterpret_cast<int *>(sSw + 2 * kMaxKb);      // [128] token or -1
    float *sRed = reinterpret_cast<float *>(sTok + kRows);      // [4][128]
    int *sItem = reinterpret_cast<int *>(sRed + 4 * kRows);      // [4]
    int *sExp = sItem + 4;                                       // [128] row, [2] gate/up exponents
    int *sRw = sExp + kRows + 4;                                 // kW4: [256] weight-row exponents R

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wn = w & 3, wm = w >> 2;
    const int l16 = lane & 15, g = lane >> 4;

    const int ntiles = a.tmeta[0];
    const int home = blockIdx.x & 7;
    int q = 0;                                       // position in the XCD ranges (thread 0)
    // The next item is claimed by thread 0 while the previous one finishes
    // (its epilogue); the first one here.
    if (tid == 0) sItem[0] = next_xcd_item(a.tmeta + 1, ntiles, a.jtiles, home, q);
    for (;;) {
    __syncthreads();
    const int item = sItem[0];
    if (item < 0) break;                             // every workgroup ends here
    // a row tile's j-tiles are consecutive items on one XCD: its activation
    // rows are fetched into that XCD's L2 once
    const int jt = item % a.jtiles;
    const int4 tl = a.tiles[item / a.jtiles];       // first block, blocks, expert
    const int b = tl.x, nb = tl.y;
    const int e = tl.z;
    if (e < 0 || e >= a.E) {                         // not a plan: skip, keep in step
        __syncthreads();
        if (tid == 0) sItem[0] = next_xcd_item(a.tmeta + 1, ntiles, a.jtiles, home, q);
        continue;
    }
    const int nrows = nb * BM;
    const int64_t p0 = (int64_t)b * BM;

    if (tid < kRows) {
        int t = -1;
        if (tid < nrows) {
            int r = a.sorted[p0 + tid];
            if (r >= 0 && (int64_t)r < a.R) {
                t = r / a.top_k;
                if (jt == 0) a.rpos[r] = (int)(p0 + tid);
            }
        }
        sTok[tid] = t;
    }
    const int64_t I = a.I, K = a.K;
    const int64_t twoI = 2 * I;
    const int nkb = a.nkb;
    const int nb13 = (int)(twoI >> 7);
    if constexpr (!C::W4) {
        const float *sg = a.w13s + ((int64_t)e * nb13 + jt) * nkb;
        const float *su = a.w13s + ((int64_t)e * nb13 + (I >> 7) + jt) * nkb;
        for (int i = tid; i < nkb; i += kNT) {
            sSw[i] = sg[i];
            sSw[kMaxKb + i] = su[i];
        }
    }
    __syncthreads();
    // ---- DMA sources of this lane: W13 rows and gathered activation rows
    const int sub = lane >> 3, slot = lane & 7;
    // (a fixed size: a local array whose size depends on the template
    // parameters keeps hipcc's host pass from emitting the kernel's stub)
    const uint8_t *wsrc[4];
    const uint8_t *esrc = nullptr;                   // kW4: this lane's exponent dword (lanes < 32)
    if constexpr (C::W4) {
#pragma unroll
        for (int i = 0; i < C::WInstr; ++i) {
            const int row = (w * C::WInstr + i) * 16 + (lane >> 2);       // tile row 0..255
            const int64_t n = (row < 128 ? 0 : I - 128) + (int64_t)jt * 128 + row;
            wsrc[i] = a.w13 + ((int64_t)e * twoI + n) * (K >> 1) + ((lane & 3) ^ w4_swizzle(row)) * 16;
        }
        const int row = 32 * w + (lane & 31);
        const int64_t n = (row < 128 ? 0 : I - 128) + (int64_t)jt * 128 + row;
        esrc = a.w13e + ((int64_t)e * twoI + n) * (K >> 5);
    } else if (a.w13_packed) {  // the packed tile is the stage image: 1 KB per instruction
        const uint8_t *tile = a.w13 + ((int64_t)e * a.jtiles + jt) * nkb * (int64_t)kPackedTile;
#pragma unroll
        for (int i = 0; i < C::WInstr; ++i) wsrc[i] = tile + (w * C::WInstr + i) * 1024 + lane * 16;
    } else {
#pragma unroll
        for (int i = 0; i < C::WInstr; ++i) {
            const int row = (w * C::WInstr + i) * 8 + sub;                // tile row 0..255
            const int64_t n = (row < 128 ? 0 : I - 128) + (int64_t)jt * 128 + row;
            const int chunk = slot ^ (row & 7);
            wsrc[i] = a.w13 + ((int64_t)e * twoI + n) * K + chunk * 16;
        }
    }
    // bytes per K-block
    const int64_t wstep = C::W4 ? 64 : (a.w13_packed ? kPackedTile : 128);
    int fallback = sTok[0];
    for (int m = 1; fallback < 0 && m < nrows; ++m) fallback = sTok[m];
    if (fallback < 0) fallback = 0;                  // tile without valid rows: scale 0
    if constexpr (MODE == kExactE8) {
        // largest biased exponent of each row's activation scales (4 threads
        // a row) and of the gate / up weight-block scales (waves 0 / 1)
        const int row = tid >> 2, part = tid & 3;
        const int t = sTok[row] >= 0 ? sTok[row] : fallback;    // the row the tile holds
        int m = 1;
        for (int kb = part; kb < nkb; kb += 4) m = max(m, biased_exp(a.xs[(int64_t)t * nkb + kb]));
        m = max(m, __shfl_xor(m, 1, 64));
        m = max(m, __shfl_xor(m, 2, 64));
        if (part == 0) sExp[row] = m;
        if (w < 2) {
            int mb = 1;
            for (int i = lane; i < nkb; i += 64) mb = max(mb, biased_exp(sSw[w * kMaxKb + i]));
            for (int off = 32; off >= 1; off >>= 1) mb = max(mb, __shfl_xor(mb, off, 64));
            if (lane == 0) sExp[kRows + w] = mb;
        }
        __syncthreads();
    }
    if constexpr (C::W4) {
        // largest exponent byte of each W13 row of the tile over all of K
        // (two threads a row, one dword = four K32 groups at a time)
        const int row = tid >> 1, half = tid & 1;
        const int64_t n = (row < 128 ? 0 : I - 128) + (int64_t)jt * 128 + row;
        const uint32_t *ep = reinterpret_cast<const uint32_t *>(a.w13e + ((int64_t)e * twoI + n) * (K >> 5));
        int m = max_byte_strided(ep, half, nkb, 2);
        m = max(m, __shfl_xor(m, 1, 64));
        if (half == 0) sRw[row] = m;
        __syncthreads();
    }

    const uint8_t *asrc[kAInstr];
#pragma unroll
    for (int i = 0; i < kAInstr; ++i) {
        const int row = (w * kAInstr + i) * 8 + sub;
        const int t = sTok[row] >= 0 ? sTok[row] : fallback;
        const int chunk = slot ^ (row & 7);
        asrc[i] = a.xq + (int64_t)t * K + chunk * 16;
    }
    // Activation scales come kSGroup K-blocks at a time, with the refill of
    // the group's first K-block, into one of two group slots: lane l of wave
    // w fetches row 16w + l / 4, K-block l % 4 of the group (clamped to the
    // last K-block).  One 4-byte load per row and group instead of one per
    // row and K-block: each of those costs the address unit a cache line.
    const float *ssrc;
    {
        const int row = w * 16 + (lane >> 2);
        const int t = sTok[row] >= 0 ? sTok[row] : fallback;
        ssrc = a.xs + (int64_t)t * nkb;
    }
    // Every wave issues PerStage vector-memory instructions per stage, plus
    // one on stages whose K-block starts a scale group (the waits in the main
    // loop count on it), in four parts: W13 rows 0-1, W13 rows 2-3 (kW4: all
    // W13 rows, then the exponent dwords), activation rows, scales.
    static_assert((C::W4 ? C::WInstr == 2 : C::WInstr == 4) && kAInstr == 2, "issue parts");
    auto issue_part = [&](int part, int stage, int kb) {
        if (C::W4 && part == 1) {
            if (lane < 32)
                __builtin_amdgcn_global_load_lds(esrc + kb * 4, sE + stage * C::EBytes + w * 128, 4, 0, 0);
        } else if (part < 2) {
            uint8_t *dw = sW + stage * C::WBytes + (w * C::WInstr) * 1024;
            constexpr int per = C::W4 ? 2 : 2;
#pragma unroll
            for (int i = per * part; i < per * part + per; ++i)
                __builtin_amdgcn_global_load_lds(wsrc[i] + kb * wstep, dw + i * 1024, 16, 0, 0);
        } else if (part == 2) {
            uint8_t *da = sA + stage * kABytes + (w * kAInstr) * 1024;
#pragma unroll
            for (int i = 0; i < kAInstr; ++i)
                __builtin_amdgcn_global_load_lds(asrc[i] + (int64_t)kb * 128, da + i * 1024, 16, 0, 0);
        } else if (kb % kSGroup == 0) {
            const int kq = kb + (lane & (kSGroup - 1));
            __builtin_amdgcn_global_load_lds(ssrc + (kq < nkb ? kq : nkb - 1),
                                             sSa + ((kb / kSGroup) & 1) * (kRows * kSGroup) + w * 64,
                                             4, 0, 0);
        }
    };
    auto issue = [&](int stage, int kb) {
        for (int part = 0; part < 4; ++part) issue_part(part, stage, kb);
    };

    constexpr int NU = 4;
    // Rows of this wave up to its last valid one: 16-row subtiles past it hold
    // only plan padding (the tail of an expert's last block) and are not
    // multiplied.
    int vrows;
    {
        const uint64_t v = __ballot(sTok[wm * 64 + lane] >= 0);
        vrows = v ? wm * 64 + 64 - __builtin_clzll(v) : 0;
        vrows = __builtin_amdgcn_readfirstlane(vrows);
    }
    const bool wave_rows = vrows > 0;

    // kW4: the reference exponent of this lane's four W13 operand rows
    int rw[4] = {0, 0, 0, 0};
    if constexpr (C::W4) {
#pragma unroll
        for (int s = 0; s < 4; ++s) rw[s] = sRw[(s < 2 ? 0 : 128) + 32 * wn + 16 * (s & 1) + l16];
    }

    v4f acc[4][NU];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < NU; ++u) acc[s][u] = v4f{0.f, 0.f, 0.f, 0.f};

    // The prologue fills stages 0 and 1; step kb refills the stage of kb + 2
    // (while one is left).  Loads complete in issue order, so at step kb only
    // the refill of kb + 1 may still be in flight.  (An L2 prefetch of the
    // W13 lines one step ahead of the refill, with 4-byte LDS-DMA touches,
    // made the kernel slower: each touch costs the address unit a whole
    // cache line.)
    issue(0, 0);
    if (nkb > 1) issue(1, 1);

    for (int kb = 0; kb < nkb; ++kb) {
        const int stage = kb % kStages;
        if (kb + 1 >= nkb)
            wait_vmcnt<0>();
        else if ((kb + 1) % kSGroup == 0)
            wait_vmcnt<C::PerStage + 1>();
        else
            wait_vmcnt<C::PerStage>();
        // Every wave has waited for its own part of this stage; the barrier
        // makes the whole stage visible, and every wave is past the multiply
        // of kb - 1, whose stage the refill below overwrites.  A plain
        // s_barrier: __syncthreads() would also drain the loads in flight.
        stage_barrier();
        // The refill of kb + 2 goes out in parts between the
        // token subtiles of the multiply, in their usual order: all waves
        // issuing a whole group at once would queue behind the address unit
        // (64 bytes per clock) instead of multiplying.
        const bool refill = kb + 2 < nkb;
        const int rst = (kb + 2) % kStages;
        auto part = [&](int pi) {
            __builtin_amdgcn_sched_barrier(0);       // keep each part where it is placed
            if (refill) issue_part(pi, rst, kb + 2);
            __builtin_amdgcn_sched_barrier(0);
        };
        part(0);

        if (!wave_rows) {
            part(1);
            part(2);
            part(3);
        } else if constexpr (C::W4) {
            const float *Ss = sSa + ((kb / kSGroup) & 1) * (kRows * kSGroup) + kb % kSGroup;
            const uint8_t *Ws = sW + stage * C::WBytes;
            const uint8_t *As = sA + stage * kABytes;
            const uint8_t *Es = sE + stage * C::EBytes;
            // W13 rows of this wave (tile rows 32wn + 16(s&1), +128 for up),
            // widened with their K32 scales relative to the row's R
            v8h wh[4][4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = (s < 2 ? 0 : 128) + 32 * wn + 16 * (s & 1) + l16;
                // whole 16-byte chunks through lds_read16 (typed 16-byte reads
                // are what lets the compiler keep these reads clear of the
                // in-flight LDS refills; 8-byte reads drew a full vmcnt(0) wait
                // every K-block), then this lane group's half of each
                const uint8_t *rp = Ws + row * 64;
                const u32x4 c01 = lds_read16(rp + (((g >> 1) ^ w4_swizzle(row)) << 4));
                const u32x4 c23 = lds_read16(rp + (((2 + (g >> 1)) ^ w4_swizzle(row)) << 4));
                const uint2 d01 = (g & 1) ? uint2{c01.z, c01.w} : uint2{c01.x, c01.y};
                const uint2 d23 = (g & 1) ? uint2{c23.z, c23.w} : uint2{c23.x, c23.y};
                const uint32_t sw = *reinterpret_cast<const uint32_t *>(Es + row * 4);
                const int dlo = (int)((sw >> (8 * (g >> 1))) & 0xffu) - rw[s];
                const int dhi = (int)((sw >> (8 * (2 + (g >> 1)))) & 0xffu) - rw[s];
                // below 2^-30 every product rounds to zero in FP16 either way
                const float flo = __uint_as_float((uint32_t)(127 + (dlo < -30 ? -30 : dlo)) << 23);
                const float fhi = __uint_as_float((uint32_t)(127 + (dhi < -30 ? -30 : dhi)) << 23);
                wh[s][0] = e2m1x8_to_f16(d01.x, flo);
                wh[s][1] = e2m1x8_to_f16(d01.y, flo);
                wh[s][2] = e2m1x8_to_f16(d23.x, fhi);
                wh[s][3] = e2m1x8_to_f16(d23.y, fhi);
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (u < 3) part(u + 1);
                if (wm * 64 + u * 16 >= vrows) continue;
                const int row = wm * 64 + u * 16 + l16;
                const uint8_t *rp = As + row * 128;
                const u32x4 lo = lds_read16(rp + ((g ^ (row & 7)) * 16));
                const u32x4 hi = lds_read16(rp + (((4 + g) ^ (row & 7)) * 16));
                const float sa = Ss[row * kSGroup];
                v8h bh[4];
                e4m3x32_to_f16(lo, hi, bh);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const v4f t = mfma16x16x128_f16(wh[s], bh);
                    acc[s][u] = t * sa + acc[s][u];
                }
            }
        } else {
            const float sbg = sSw[kb];
            const float sbu = sSw[kMaxKb + kb];
            // this K-block's activation scales: [row][kb % kSGroup] of its group slot
            const float *Ss = sSa + ((kb / kSGroup) & 1) * (kRows * kSGroup) + kb % kSGroup;
            const uint8_t *Ws = sW + stage * C::WBytes;
            const uint8_t *As = sA + stage * kABytes;
            // W operand rows of this wave: tile rows 32wn + 16(s&1) (+128 for up)
            u32x4 wr[4][2];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = (s < 2 ? 0 : 128) + 32 * wn + 16 * (s & 1) + l16;
                const uint8_t *rp = Ws + row * 128;
                wr[s][0] = lds_read16(rp + ((g ^ (row & 7)) * 16));
                wr[s][1] = lds_read16(rp + (((4 + g) ^ (row & 7)) * 16));
            }
            if constexpr (MODE == kExactE8) {
            // every factor is a power of two: the widening takes it exactly
            const float cg = sbg * pow2_neg_biased(sExp[kRows]);
            const float cu = sbu * pow2_neg_biased(sExp[kRows + 1]);
            v8h wh[4][4];
#pragma unroll
            for (int s = 0; s < 4; ++s) e4m3x32_to_f16(wr[s][0], wr[s][1], wh[s], s < 2 ? cg : cu);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (u < 3) part(u + 1);
                if (wm * 64 + u * 16 >= vrows) continue;
                const int row = wm * 64 + u * 16 + l16;
                const uint8_t *rp = As + row * 128;
                const u32x4 lo = lds_read16(rp + ((g ^ (row & 7)) * 16));
                const u32x4 hi = lds_read16(rp + (((4 + g) ^ (row & 7)) * 16));
                v8h bh[4];
                e4m3x32_to_f16(lo, hi, bh, Ss[row * kSGroup] * pow2_neg_biased(sExp[row]));
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[s][u] = mfma16x16x128_f16_acc(wh[s], bh, acc[s][u]);
            }
            } else if constexpr (MODE == kExact) {
            // Hand-pipelined: the activation rows of subtile u + 1 are read
            // from LDS while subtile u multiplies; the W13 widening of s = 2, 3
            // runs behind subtile 0's first chains; and the scale FMAs of one
            // chain go out behind the MFMAs of the next, so the matrix pipe
            // does not drain between chains.  Subtile 0 always has rows here
            // (vrows > 64 wm).
            u32x4 ar[2];
            float sa;
            auto read_a = [&](int u) {
                const int row = wm * 64 + u * 16 + l16;
                const uint8_t *rp = As + row * 128;
                ar[0] = lds_read16(rp + ((g ^ (row & 7)) * 16));
                ar[1] = lds_read16(rp + (((4 + g) ^ (row & 7)) * 16));
                sa = Ss[row * kSGroup];
            };
            read_a(0);
            v8h wh[4][4];
            e4m3x32_to_f16(wr[0][0], wr[0][1], wh[0]);
            e4m3x32_to_f16(wr[1][0], wr[1][1], wh[1]);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (u < 3) part(u + 1);
                if (wm * 64 + u * 16 >= vrows) continue;
                if (u > 0) read_a(u);
                v8h bh[4];
                e4m3x32_to_f16(ar[0], ar[1], bh);
                const float fg = sa * sbg, fu = sa * sbu;
                v4f t0 = mfma16x16x128_f16(wh[0], bh);
                v4f t1 = mfma16x16x128_f16(wh[1], bh);
                __builtin_amdgcn_sched_barrier(0);
                if (u == 0) e4m3x32_to_f16(wr[2][0], wr[2][1], wh[2]);
                acc[0][u] = t0 * fg + acc[0][u];
                t0 = mfma16x16x128_f16(wh[2], bh);
                __builtin_amdgcn_sched_barrier(0);
                if (u == 0) e4m3x32_to_f16(wr[3][0], wr[3][1], wh[3]);
                acc[1][u] = t1 * fg + acc[1][u];
                t1 = mfma16x16x128_f16(wh[3], bh);
                __builtin_amdgcn_sched_barrier(0);
                acc[2][u] = t0 * fu + acc[2][u];
                acc[3][u] = t1 * fu + acc[3][u];
            }
            } else {
            v8i wq[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) wq[s] = join8p(wr[s][0], wr[s][1]);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (u < 3) part(u + 1);
                if (wm * 64 + u * 16 >= vrows) continue;
                const int row = wm * 64 + u * 16 + l16;
                const uint8_t *rp = As + row * 128;
                const u32x4 lo = lds_read16(rp + ((g ^ (row & 7)) * 16));
                const u32x4 hi = lds_read16(rp + (((4 + g) ^ (row & 7)) * 16));
                const float sa = Ss[row * kSGroup];
                if constexpr (MODE == kFp8E8) {
                    const v8i B = join8p(lo, hi);
                    const int eb = e8m0_of(sa), eg = e8m0_of(sbg), eu = e8m0_of(sbu);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        acc[s][u] = mfma16x16x128_e8m0(wq[s], B, acc[s][u], s < 2 ? eg : eu, eb);
                } else {
                    const v8i B = join8p(lo, hi);
                    const float fg = sa * sbg, fu = sa * sbu;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        v4f t = mfma16x16x128(wq[s], B);
                        acc[s][u] = t * (s < 2 ? fg : fu) + acc[s][u];
                    }
                }
            }
            }
        }
    }
    __syncthreads();
    // the next item's claim travels while this one's epilogue computes
    const int ticket = tid == 0 ? claim_begin(a.tmeta + 1, home, q) : 0;

    if constexpr (C::W4) {
        // 2^(R - 127) of each output row (rows 4g..4g+3 of every operand s)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int orow = (s < 2 ? 0 : 128) + 32 * wn + 16 * (s & 1) + 4 * g;
            const v4f F = v4f{pow2_int(sRw[orow] - 127), pow2_int(sRw[orow + 1] - 127),
                              pow2_int(sRw[orow + 2] - 127), pow2_int(sRw[orow + 3] - 127)};
#pragma unroll
            for (int u = 0; u < NU; ++u) acc[s][u] = acc[s][u] * F;
        }
    }
    if constexpr (MODE == kExactE8) {
        const float fbg = pow2_biased(sExp[kRows]), fbu = pow2_biased(sExp[kRows + 1]);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const float fa = pow2_biased(sExp[wm * 64 + u * 16 + l16]);
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[s][u] = (acc[s][u] * fa) * (s < 2 ? fbg : fbu);
        }
    }
    // ---- SwiGLU + per-row 128-group FP8 requantisation
    float h[NU][2][4];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int row = wm * 64 + u * 16 + l16;
        const bool valid = sTok[row] >= 0;
        float amax = 0.f;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gt = acc[s][u][i];
                const float up = acc[s + 2][u][i];
                const float hv = valid ? swiglu(gt, up) : 0.f;
                h[u][s][i] = hv;
                amax = fmaxf(amax, fabsf(hv));
            }
        amax = wave_max_xor(amax, 16);
        amax = wave_max_xor(amax, 32);
        if (g == 0) sRed[wn * kRows + row] = amax;
    }
    __syncthreads();
    const bool ue = a.inter_ue8m0 != 0;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int row = wm * 64 + u * 16 + l16;
        if (row >= nrows) continue;
        const float amax = fmaxf(fmaxf(sRed[row], sRed[kRows + row]),
                                 fmaxf(sRed[2 * kRows + row], sRed[3 * kRows + row]));
        float s, inv;
        group_scale(amax, ue, s, inv);
        const int64_t p = p0 + row;
        uint8_t *dst = a.hq + p * I + (int64_t)jt * 128 + 32 * wn + 4 * g;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint32_t code = pack_e4m3x4(h[u][s2][0] * inv, h[u][s2][1] * inv,
                                        h[u][s2][2] * inv, h[u][s2][3] * inv);
            *reinterpret_cast<uint32_t *>(dst + 16 * s2) = code;
        }
        if (wn == 0 && g == 0) a.hs[p * (I >> 7) + jt] = s;
    }
    if (tid == 0) sItem[0] = claim_end(ticket, a.tmeta + 1, ntiles, a.jtiles, home, q);
    __syncthreads();                                 // LDS is reused by the next item
    }
}

template <int BM, int MODE>
hipError_t launch_pipe(const GateUpArgs &a, hipStream_t st) {
    if (a.nblocks == 0) return hipSuccess;
    tiles_kernel<<<1 + prep_groups(a.R + a.n_cnt), 1024, 0, st>>>(a.eids, a.ntp, BM, kRows / BM, a.nblocks,
                                                                   a.tiles, a.tmeta, (uint32_t *)a.rpos,
                                                                   a.R, a.cnt, a.n_cnt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    int64_t grid = device_cu_count();
    const int64_t max_items = (int64_t)a.nblocks * a.jtiles;
    if (grid > max_items) grid = max_items;
    static std::atomic<uint64_t> lds_set{0};
    constexpr size_t smem = PCfg<MODE>::Smem;
    hipError_t e = raise_lds_limit(lds_set, (const void *)gateup_pipe_kernel<BM, MODE>, (int)smem);
    if (e != hipSuccess) return e;
    gateup_pipe_kernel<BM, MODE><<<(unsigned)grid, kNT, smem, st>>>(a);
    return hipGetLastError();
}

template <int BM>
hipError_t launch_pipe_mode(const GateUpArgs &a, int mode, hipStream_t st) {
    switch (mode) {
        case kExact: return launch_pipe<BM, kExact>(a, st);
        case kFp8: return launch_pipe<BM, kFp8>(a, st);
        case kFp8E8: return launch_pipe<BM, kFp8E8>(a, st);
        case kExactE8: return launch_pipe<BM, kExactE8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_tiles(const GateUpArgs &a, int block_m, int tile_rows, hipStream_t st) {
    if (a.nblocks == 0) return hipSuccess;
    if (block_m != 8 && block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128)
        return hipErrorInvalidValue;
    if ((tile_rows != 32 && tile_rows != kRows) || block_m > tile_rows) return hipErrorInvalidValue;
    tiles_kernel<<<1 + prep_groups(a.R + a.n_cnt), 1024, 0, st>>>(a.eids, a.ntp, block_m, tile_rows / block_m,
                                                                   a.nblocks, a.tiles, a.tmeta,
                                                                   (uint32_t *)a.rpos, a.R, a.cnt, a.n_cnt);
    return hipGetLastError();
}

hipError_t launch_gateup_pipe_w4(const GateUpArgs &a, int block_m, hipStream_t st) {
    switch (block_m) {
        case 8: return launch_pipe<8, kW4>(a, st);
        case 16: return launch_pipe<16, kW4>(a, st);
        case 32: return launch_pipe<32, kW4>(a, st);
        case 64: return launch_pipe<64, kW4>(a, st);
        case 128: return launch_pipe<128, kW4>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gateup_pipe(const GateUpArgs &a, int block_m, bool fp8_mma, bool e8m0,
                              hipStream_t st) {
    const int mode = !fp8_mma ? (e8m0 ? kExactE8 : kExact) : (e8m0 ? kFp8E8 : kFp8);
    switch (block_m) {
        case 8: return launch_pipe_mode<8>(a, mode, st);
        case 16: return launch_pipe_mode<16>(a, mode, st);
        case 32: return launch_pipe_mode<32>(a, mode, st);
        case 64: return launch_pipe_mode<64>(a, mode, st);
        case 128: return launch_pipe_mode<128>(a, mode, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
