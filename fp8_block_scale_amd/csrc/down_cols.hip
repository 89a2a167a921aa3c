// Step 5 for small route counts: the down-projection GEMM split over output
// columns, with the route sum in the same launch.
//
// Same arithmetic as down.hip (FlashInfer PR #4287, PR summary and the FP32
// scale note of its final kernel performance section): for plan row p of
// expert e holding route r = t * top_k + j,
//   y[r, c] = sum_jb h_s[p, jb] * w2_s[e, c / 128, jb]
//                  * sum_{i in jb} h_q[p, i] * W2[e, c, i]              (FP32)
//   out[t, c] = bf16(out[t, c] + sum_j topk_weights[r] * y[r, c])
// with the route terms added in route order in FP32 and one BF16 rounding.
//
// Work split.  One workgroup (eight waves, or four where the LDS is needed
// for many routes' rows) owns 32 output columns.  It first
// puts every valid route's intermediate row and row scales into LDS, indexed
// by route: copied from the FP8 rows of the gate/up stage (each route's plan
// row from that stage's route map), or -- after the column-slice gate/up,
// which leaves FP32 SwiGLU rows -- requantised from those (each route's plan
// row from a scan of the plan); then it
// walks every plan block below num_tokens_post_padded: wave w takes the
// blocks b = w / 2 (mod NW / 2) and the 16 columns of half w % 2.  Per block a wave
// multiplies the block's W2 slab (its expert's 16 rows of W2 for those
// columns, all of I) with the block's routes' rows and keeps each valid
// route's results in LDS (a route lies in one block: nothing to reduce).
// Having every route of its columns, the workgroup adds each token's routes
// itself at the end: no per-route buffer in HBM and no route-sum launch.
// Each W2 slab is read by exactly one wave.
//
// Pipeline.  A ring of NS stages per wave (three with eight waves, five
// with four), each stage one block's W2 slab
// (16-byte chunks XOR-swizzled by row, so the MFMA operand reads hit distinct
// banks) and its route ids, expert id and W2 block scales, by direct
// global->LDS loads NS - 1 blocks ahead, so a block's multiply waits on
// nothing but its stage.  The rings are private to their waves: between the
// copy of the intermediate rows and the route sum there is no barrier, the
// waits are each wave's own load counts.  FP8 MFMA
// (v_mfma_f32_16x16x128_f8f6f4) with the FP32 scale product applied per
// 128-deep K-block, or with power-of-two scales as E8M0 exponents inside the
// MFMA.  With E2M1 weights (the W4A8 variant, sglang-glm53-flash-sm120 PR
// #13, description) a stage holds the slab's E2M1 pairs and their K32
// exponent bytes, and the mixed E2M1 x E4M3 MFMA takes each K32 group's
// exponent as the weight operand's E8M0 scale:
//   y[r, c] = sum_jb h_s[p, jb] * sum_{q in jb} 2^(w2_e[e, c, q] - 127)
//                  * sum_{i in q} h_q[p, i] * W2[e, c, i]               (FP32)
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kCW = 16;                 // output columns per wave
constexpr int kWavesMin = 4;            // waves per workgroup: 4 (5-stage rings) or 8 (3-stage)
constexpr int kWGCols = 2 * kCW;        // output columns per workgroup
constexpr int kIB = 256;                // bytes of an intermediate / W2 row (I)
constexpr int kNJB = kIB / 128;
constexpr int kStagesMin = 5;
constexpr int kStagesMax = 5;
constexpr int64_t kMaxRoutes = 192;                    // routes whose rows fit in LDS
constexpr int kScan = 12;                              // plan entries per thread loaded up front

// A ring stage: one block's W2 slab (its expert's 16 rows of the wave's
// columns, all of I), then -- W4, the E2M1 weights -- the slab rows' K32
// exponent bytes (8 per row), then 128 bytes of metadata: [16] route ids,
// the expert id, (FP8) the two W2 block scales.
template <bool W4>
struct DCStage {
    static constexpr int Slab = kCW * kIB / (W4 ? 2 : 1);
    static constexpr int SlabInstr = Slab / 1024;        // 16-byte DMA per lane
    static constexpr int Exp = W4 ? kCW * kIB / 32 : 0;
    static constexpr int Meta = Slab + Exp;
    static constexpr int Bytes = Meta + 128;
    static constexpr int PerStage = SlabInstr + (W4 ? 1 : 0) + 1;
    static_assert((kStagesMax - 2) * PerStage < 64, "vmcnt range");
};

// LDS carve-up after the rings ([NW waves][NS] stages): intermediate rows
// by route [R][kIB], their scales [R][kNJB], the results [R + 1][kWGCols]
// (FP32; row R takes the rows that hold no route), each route's plan row
// [R] (-1: masked).  At R = 192: 160832 bytes.
template <bool W4, int NW, int NS>
struct DCLayout {
    int h, hs, y, rp, total;
    __host__ __device__ explicit DCLayout(int R) {
        h = NW * NS * DCStage<W4>::Bytes;
        hs = h + R * kIB;
        y = hs + ((R * kNJB * 4 + 15) & ~15);            // 16-byte rows of results
        rp = y + (R + 1) * kWGCols * 4;
        total = rp + R * 4;
    }
};
static_assert(kWavesMin * kStagesMin * DCStage<false>::Bytes + kMaxRoutes * (kIB + kNJB * 4 + kWGCols * 4 + 4) +
                  kWGCols * 4 <= 160 * 1024, "LDS budget at the route limit");

typedef const __attribute__((address_space(4))) int32_t *const_i32_p;

// Workgroup barrier that waits for this wave's LDS (and scalar) accesses
// only: global loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0), vmcnt / expcnt at maximum
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most min(ahead, K) stages' loads are outstanding (ahead is
// wave-uniform: the blocks issued past the one about to be multiplied).
template <int PS, int K>
__device__ __forceinline__ void wait_ahead(int ahead) {
    if constexpr (K == 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= K) wait_vmcnt<K * PS>();
        else wait_ahead<PS, K - 1>(ahead);
    }
}

// step(stage S, block i + S) for S = S0 .. NS - 1 while i + S < nw, with the
// stage index a compile-time constant
template <int S, int NS, typename F>
__device__ __forceinline__ void steps_from(F &step, int i, int nw) {
    if constexpr (S < NS) {
        if (i + S < nw) {
            step(std::integral_constant<int, S>{}, i + S);
            steps_from<S + 1, NS>(step, i, nw);
        }
    }
}

template <int BM, bool E8M0, bool RQ, bool W4, int NW, int NS>
__global__ void __launch_bounds__(64 * NW, 1)
down_cols_kernel(DownArgs a, const int32_t *__restrict__ rpos, ColsRequant rq,
                 uint16_t *__restrict__ out) {
    static_assert(BM <= 16, "one 16-row MFMA tile per plan block");
    static_assert(!W4 || (!E8M0 && !RQ), "E2M1 weights: FP8 intermediate rows, FP32 row scales");
    using SC = DCStage<W4>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int R = (int)a.R;
    const DCLayout<W4, NW, NS> L(R);
    constexpr int kWaves = NW;
    constexpr int NP = NW / 2;                          // block parities (waves per column half)
    uint8_t *sH = smem + L.h;
    float *sHs = reinterpret_cast<float *>(smem + L.hs);
    float *sY = reinterpret_cast<float *>(smem + L.y);
    int *sRp = reinterpret_cast<int *>(smem + L.rp);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = w & 1, parity = w >> 1;
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t K = a.K;
    const int64_t cw0 = (int64_t)blockIdx.x * kWGCols;    // the workgroup's columns
    const int64_t c0 = cw0 + half * kCW;                  // this wave's

    const int ntp = __builtin_amdgcn_readfirstlane(((const_i32_p)a.ntp)[0]);
    int nb = ntp / BM;
    nb = nb < a.nblocks ? nb : a.nblocks;

    uint8_t *ring = smem + w * NS * SC::Bytes;

    // ---- this wave's blocks: b = NP i + parity, i < nw
    const int nw = (nb - parity + NP - 1) / NP;
    auto issue = [&](int st, int i) {
        const int b = NP * i + parity;
        uint8_t *base = ring + st * SC::Bytes;
        const int e0 = __builtin_amdgcn_readfirstlane(((const_i32_p)a.eids)[b]);
        const int e = (e0 >= 0 && e0 < a.E) ? e0 : 0;
        if constexpr (W4) {
            // W2 rows c0 .. c0 + 15 of expert e (128 B of E2M1 pairs each):
            // LDS slot s (16 bytes) holds row s / 8, chunk (s % 8) ^ (row % 8);
            // then their exponent dwords, lane l: row l / 2, K-block l % 2
            const uint8_t *wrow = a.w2 + ((int64_t)e * K + c0) * (kIB / 2);
#pragma unroll
            for (int k = 0; k < SC::SlabInstr; ++k) {
                const int s = k * 64 + lane;
                const int row = s >> 3, pos = s & 7;
                lds_dma16_nt(wrow + (int64_t)row * (kIB / 2) + (pos ^ (row & 7)) * 16, base + k * 1024);
            }
            if (lane < 2 * kCW)
                lds_dma4(a.w2e + ((int64_t)e * K + c0 + (lane >> 1)) * (kIB / 32) + 4 * (lane & 1),
                         base + SC::Slab);
        } else {
            // W2 rows c0 .. c0 + 15 of expert e: LDS slot s (16 bytes) of the
            // slab holds row s / 16, chunk (s % 16) ^ row
            const uint8_t *wrow = a.w2 + ((int64_t)e * K + c0) * kIB;
#pragma unroll
            for (int k = 0; k < SC::SlabInstr; ++k) {
                const int s = k * 64 + lane;
                const int row = s >> 4, pos = s & 15;
                lds_dma16_nt(wrow + (int64_t)row * kIB + (pos ^ row) * 16, base + k * 1024);
            }
        }
        // metadata in one 4-byte DMA: lanes 0-15 the route ids, lane 16 the
        // expert id, lanes 17 .. 16 + kNJB the W2 block scales (FP8)
        const void *msrc;
        if (lane < 16)
            msrc = a.sorted + (int64_t)b * BM + (lane < BM ? lane : 0);
        else if (lane == 16 || W4)
            msrc = a.eids + b;
        else
            msrc = a.w2s + ((int64_t)e * (K >> 7) + (c0 >> 7)) * kNJB + (lane < 17 + kNJB ? lane - 17 : 0);
        if (lane < (W4 ? 17 : 17 + kNJB)) lds_dma4(msrc, base + SC::Meta);
    };

    auto compute = [&](int st) {
        const uint8_t *base = ring + st * SC::Bytes;
        const int *meta = reinterpret_cast<const int *>(base + SC::Meta);
        const int r = meta[l16], e0 = meta[16];
        const bool ok = l16 < BM && r >= 0 && r < R && e0 >= 0 && e0 < a.E;
        const int rr = ok ? r : 0;
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        const uint8_t *ha = sH + (int64_t)rr * kIB;
#pragma unroll
        for (int jb = 0; jb < kNJB; ++jb) {
            const int clo = jb * 8 + g, chi = jb * 8 + 4 + g;
            const u32x4 b0 = lds_read16(ha + (clo ^ (rr & 15)) * 16);
            const u32x4 b1 = lds_read16(ha + (chi ^ (rr & 15)) * 16);
            const v8i B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            const float sa = sHs[rr * kNJB + jb];
            if constexpr (W4) {
                // lane group g: K [32 g, 32 g + 32) of this K-block, chunk
                // 4 jb + g of the row, and that group's exponent byte
                const uint8_t *wa = base + l16 * (kIB / 2);
                const u32x4 a0 = lds_read16(wa + ((4 * jb + g) ^ (l16 & 7)) * 16);
                const v8i A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
                const uint32_t ed = *reinterpret_cast<const uint32_t *>(base + SC::Slab + (2 * l16 + jb) * 4);
                acc = mfma16x16x128_e2m1_e4m3(A, B, (int)((ed >> (8 * g)) & 0xffu)) * sa + acc;
            } else {
                const uint8_t *wa = base + l16 * kIB;
                const u32x4 a0 = lds_read16(wa + (clo ^ l16) * 16), a1 = lds_read16(wa + (chi ^ l16) * 16);
                const v8i A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                const float sb = __int_as_float(meta[17 + jb]);
                if constexpr (E8M0)
                    acc = mfma16x16x128_e8m0(A, B, acc, e8m0_of(sb), e8m0_of(sa));
                else
                    acc = mfma16x16x128(A, B) * (sa * sb) + acc;
            }
        }
        // lane (row l16, group g) holds columns 4g .. 4g + 3 of its route.
        // Every lane stores (rows without a route to the spare row R): a
        // store under a lane condition would let the compiler move the MFMAs
        // under it, where lanes outside the condition keep stale scale
        // operands.  A block whose expert id is out of range adds nothing:
        // its routes' results are zero (as on the other paths, where such a
        // block's routes stay masked).
        const bool routed = l16 < BM && r >= 0 && r < R;
        if (!(e0 >= 0 && e0 < a.E)) acc = v4f{0.f, 0.f, 0.f, 0.f};    // (uniform per block)
        *reinterpret_cast<v4f *>(sY + (routed ? r : R) * kWGCols + half * kCW + 4 * g) = acc;
    };

    // ---- every valid route's intermediate row and row scales into LDS, by
    // route
    if constexpr (RQ) {
        // ---- each route's plan row from a scan of the plan (a valid route
        // sits in exactly one plan row; routes not found are masked).  The
        // first kScan x 256 entries are loaded before num_tokens_post_padded
        // is known (entries at or beyond it are dropped afterwards), so the
        // two loads overlap; the barrier between waits for LDS only.
        const int cap = a.nblocks * BM;
        int rv[kScan];
#pragma unroll
        for (int u = 0; u < kScan; ++u) {
            const int p = u * 64 * kWaves + tid;
            rv[u] = p < cap ? a.sorted[p] : -1;
        }
        for (int r = tid; r < R; r += 64 * kWaves) sRp[r] = -1;
        lds_barrier();
        const int lim = nb * BM;
#pragma unroll
        for (int u = 0; u < kScan; ++u) {
            const int p = u * 64 * kWaves + tid;
            if (p < lim && rv[u] >= 0 && rv[u] < R) sRp[rv[u]] = p;
        }
        for (int p = kScan * 64 * kWaves + tid; p < lim; p += 64 * kWaves) {
            const int r = a.sorted[p];
            if (r >= 0 && r < R) sRp[r] = p;
        }
        __syncthreads();
        // ---- the FP32 SwiGLU rows requantised into LDS by route: a wave per
        // route, lane l holds columns 4 l .. 4 l + 3, 32 lanes per 128-column
        // group (the group maximum over them), four routes' loads in flight
        const bool ue = rq.ue8m0 != 0;
        const int jb = lane >> 5;
        for (int r0 = w; r0 < R; r0 += 4 * kWaves) {
            v4f v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = r0 + u * kWaves;
                v[u] = v4f{0.f, 0.f, 0.f, 0.f};
                if (r < R && sRp[r] >= 0)
                    v[u] = *reinterpret_cast<const v4f *>(rq.h32 + (int64_t)sRp[r] * kIB + 4 * lane);
            }
            // the four routes' group maxima side by side (independent shuffles)
            float amax[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                amax[u] = fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])), fmaxf(fabsf(v[u][2]), fabsf(v[u][3])));
#pragma unroll
            for (int m = 1; m < 32; m *= 2)
#pragma unroll
                for (int u = 0; u < 4; ++u) amax[u] = wave_max_xor(amax[u], m);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = r0 + u * kWaves;
                float sc, inv;
                group_scale(amax[u], ue, sc, inv);
                const uint32_t code = pack_e4m3x4(v[u][0] * inv, v[u][1] * inv, v[u][2] * inv, v[u][3] * inv);
                if (r < R && sRp[r] >= 0) {
                    // byte 4 l of the row: chunk l / 4, stored at chunk (l / 4) ^ (r & 15)
                    *reinterpret_cast<uint32_t *>(sH + r * kIB + (((lane >> 2) ^ (r & 15)) << 4) + 4 * (lane & 3)) = code;
                    if ((lane & 31) == 0) sHs[r * kNJB + jb] = sc;
                    if (blockIdx.x == 0) {
                        const int64_t p = sRp[r];
                        *reinterpret_cast<uint32_t *>(rq.hq + p * kIB + 4 * lane) = code;
                        if ((lane & 31) == 0) rq.hs[p * kNJB + jb] = sc;
                    }
                }
            }
        }
        __syncthreads();                                // rows in; the map's reads done
    } else {
        // ---- every valid route's FP8 row and row scales copied into LDS, by
        // route: the route map of the gate/up stage gives each route's plan
        // row (-1: masked), then direct global->LDS copies, four routes (1 KB)
        // per instruction, chunk c of route r's row at LDS chunk c ^ (r & 15);
        // masked routes copy plan row 0 and stay masked
        for (int r = tid; r < R; r += 64 * kWaves) sRp[r] = rpos[r];
        __syncthreads();
        for (int r0 = 4 * w; r0 < R; r0 += 4 * kWaves) {
            const int r = r0 + (lane >> 4);
            if (r < R) {
                const int p = sRp[r];
                lds_dma16(a.hq + (int64_t)(p >= 0 ? p : 0) * kIB + ((l16 ^ (r & 15)) * 16),
                          sH + (int64_t)r0 * kIB);
            }
        }
        for (int q0 = 64 * w; q0 < R * kNJB; q0 += 64 * kWaves) {
            const int q = q0 + lane;                     // route q / kNJB, K-block q % kNJB
            if (q < R * kNJB) {
                const int p = sRp[q / kNJB];
                lds_dma4(a.hs + (int64_t)(p >= 0 ? p : 0) * kNJB + q % kNJB, sHs + q0);
            }
        }
        wait_vmcnt<0>();                                 // every wave's copies have landed
        __syncthreads();
    }

    // this wave's blocks i, slots i % NS; NS - 1 blocks in flight ahead of
    // the one being multiplied (loads complete in issue order)
    for (int q = 0; q < NS - 1; ++q)
        if (q < nw) issue(q, q);
    auto step = [&](auto st_c, int i) {
        constexpr int ST = decltype(st_c)::value;
        wait_ahead<SC::PerStage, NS - 2>(nw - 1 - i);  // blocks issued past i: at most NS - 2
        // the refill goes into the slot of block i - 1, whose operand reads
        // the previous step has consumed
        if (i + NS - 1 < nw) issue((ST + NS - 1) % NS, i + NS - 1);
        compute(ST);
    };
    for (int i = 0; i < nw; i += NS) steps_from<0, NS>(step, i, nw);
    wait_vmcnt<0>();
    __syncthreads();                                    // every wave's results are in LDS

    // ---- route sum: thread tid takes column tid % 32 of tokens tid / 32,
    // + 8, ...; routes in order, FP32, then the previous output, one rounding
    const int M = R / a.top_k;
    const int col = tid % kWGCols;
    for (int t = tid / kWGCols; t < M; t += 64 * kWaves / kWGCols) {
        float s = 0.f;
        for (int j = 0; j < a.top_k; ++j) {
            const int r = t * a.top_k + j;
            if (sRp[r] >= 0) s += a.topk_w[r] * sY[r * kWGCols + col];
        }
        uint16_t *op = out + (int64_t)t * K + cw0 + col;
        *op = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(*op) + s);
    }
}

template <int BM, bool E8M0, bool RQ, bool W4, int NW, int NS>
hipError_t launch_dc_cfg(const DownArgs &a, const int32_t *rpos, const ColsRequant &rq, uint16_t *out,
                         hipStream_t st) {
    const int64_t grid = a.K / kWGCols;
    const int smem = DCLayout<W4, NW, NS>((int)a.R).total;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e =
        raise_lds_limit(lds_set, (const void *)down_cols_kernel<BM, E8M0, RQ, W4, NW, NS>, 160 * 1024);
    if (e != hipSuccess) return e;
    down_cols_kernel<BM, E8M0, RQ, W4, NW, NS><<<(unsigned)grid, 64 * NW, smem, st>>>(a, rpos, rq, out);
    return hipGetLastError();
}

// Eight waves (two per SIMD, so one wave's LDS reads and MFMAs overlap the
// other's) with three-stage rings wherever the LDS holds them next to the
// routes' rows; else four waves with five-stage rings.
template <int BM, bool E8M0, bool RQ, bool W4>
hipError_t launch_dc(const DownArgs &a, const int32_t *rpos, const ColsRequant &rq, uint16_t *out,
                     hipStream_t st) {
    if (a.K / kWGCols == 0 || a.nblocks == 0) return hipSuccess;
    if (DCLayout<W4, 8, 3>((int)a.R).total <= 160 * 1024)
        return launch_dc_cfg<BM, E8M0, RQ, W4, 8, 3>(a, rpos, rq, out, st);
    return launch_dc_cfg<BM, E8M0, RQ, W4, kWavesMin, kStagesMin>(a, rpos, rq, out, st);
}

template <int BM>
hipError_t launch_dc_bm(const DownArgs &a, bool e8m0, const int32_t *rpos, const ColsRequant &rq,
                        uint16_t *out, hipStream_t st) {
    if (a.w2e) return launch_dc<BM, false, false, true>(a, rpos, rq, out, st);
    if (rq.h32)
        return e8m0 ? launch_dc<BM, true, true, false>(a, rpos, rq, out, st)
                    : launch_dc<BM, false, true, false>(a, rpos, rq, out, st);
    return e8m0 ? launch_dc<BM, true, false, false>(a, rpos, rq, out, st)
                : launch_dc<BM, false, false, false>(a, rpos, rq, out, st);
}

}  // namespace

bool down_cols_fits(int64_t R, int64_t I, int64_t K, int block_m) {
    return R >= 1 && R <= kMaxRoutes && I == kIB && K % kWGCols == 0 && (block_m == 8 || block_m == 16);
}

// a.w2e set: the E2M1 weights of the W4A8 variant (w2 holds E2M1 pairs
// [E, K, I / 2], w2e the K32 exponent bytes [E, K, I / 32]); they take the
// FP8 intermediate rows through rpos (no requantisation mode, no E8M0 MFMA).
hipError_t launch_down_cols(const DownArgs &a, int block_m, bool e8m0, const int32_t *rpos,
                            const ColsRequant &rq, uint16_t *out, hipStream_t st) {
    if (!down_cols_fits(a.R, a.I, a.K, block_m)) return hipErrorInvalidValue;
    if (rq.h32 && (!rq.hq || !rq.hs)) return hipErrorInvalidValue;
    if (!rq.h32 && !rpos) return hipErrorInvalidValue;
    if (a.w2e && (rq.h32 || e8m0)) return hipErrorInvalidValue;
    if (block_m == 8) return launch_dc_bm<8>(a, e8m0, rpos, rq, out, st);
    return launch_dc_bm<16>(a, e8m0, rpos, rq, out, st);
}

}  // namespace moe
