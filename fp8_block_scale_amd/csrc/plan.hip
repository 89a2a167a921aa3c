// Step 1: the moe_align_block_size routing plan (one workgroup, or three
// launches over many workgroups for large route counts).
//
// What is built (FlashInfer PR #4287, PR summary and public-contract
// section; masked int32/int64 routes from sglang-glm53-flash-sm120 PR #13,
// description and validation): valid routes grouped by expert in ascending
// expert id, ascending flat route index r inside an expert, every expert's
// segment padded with the sentinel R to a multiple of block_m, one expert id
// per block and the padded length P written on the device.
//
// How (one workgroup of NW wavefronts):
//   pass 1  each wave owns a contiguous chunk of routes and walks it 64 at a
//           time; lanes holding the same expert are found with one ballot
//           per bit of the expert id (an exact match mask), and the group's
//           lowest lane adds the group size to the wave's LDS histogram row;
//   scan    per expert: total count, round-up to block_m, exclusive prefix
//           over experts (block scan), per-wave base offsets, sentinel fill
//           and expert_ids;
//   pass 2  the waves walk their chunks again in the same order; a lane's
//           slot is its wave base + the number of lower lanes in its match
//           group, so the scatter is stable (ascending r) without atomics.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int64_t kPlanMultiMin = 4096;      // routes from which several workgroups pay off

__device__ __forceinline__ uint64_t match_mask(int key, int nbits) {
    uint64_t m = ~0ull;
    for (int b = 0; b < nbits; ++b) {
        int bit = (key >> b) & 1;
        uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

template <typename IdT>
__device__ __forceinline__ void plan_body(const IdT *__restrict__ ids, int64_t R, int E, int bm,
                                          int nwaves, int32_t *__restrict__ sorted,
                                          int32_t *__restrict__ expert_ids,
                                          int32_t *__restrict__ ntp, int *smem) {
    int *hist = smem;                     // [nwaves][E]: counts, then bases
    int *cnt = hist + nwaves * E;         // [E] per-expert totals
    int *wsum = cnt + E;                  // [32] wave totals for the scan

    const int tid = threadIdx.x;
    const int T = blockDim.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int nbits = 32 - __clz(E);      // keys 0..E fit (E = masked)
    const uint64_t lower = (1ull << lane) - 1ull;

    for (int i = tid; i < nwaves * E; i += T) hist[i] = 0;
    __syncthreads();

    // contiguous chunk per wave, a multiple of 64 routes
    int64_t chunk = (R + nwaves - 1) / nwaves;
    chunk = (chunk + 63) & ~int64_t(63);
    const int64_t beg = (int64_t)w * chunk;
    const int64_t end = beg + chunk < R ? beg + chunk : R;

    // ---- pass 1: per-wave histogram
    if (w < nwaves) {
        for (int64_t base = beg; base < end; base += 64) {
            int64_t r = base + lane;
            int key = E;
            if (r < end) {
                IdT v = ids[r];
                if (v >= 0 && v < (IdT)E) key = (int)v;
            }
            uint64_t m = match_mask(key, nbits);
            if (key < E && (m & lower) == 0) hist[w * E + key] += __popcll(m);
        }
    }
    __syncthreads();

    // ---- scan: per-expert totals, padded sizes, offsets, bases, sentinels
    const int seg = (E + T - 1) / T;
    const int e0 = tid * seg;
    const int e1 = e0 + seg < E ? e0 + seg : E;
    int local = 0;
    for (int e = e0; e < e1; ++e) {
        int c = 0;
        for (int q = 0; q < nwaves; ++q) c += hist[q * E + e];
        cnt[e] = c;
        local += (c + bm - 1) / bm * bm;
    }
    // block exclusive scan of `local`
    int incl = local;
    for (int d = 1; d < 64; d <<= 1) {
        int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int q = 0; q < T / 64; ++q) {
            int v = wsum[q];
            wsum[q] = run;
            run += v;
        }
        ntp[0] = run;                     // P
    }
    __syncthreads();
    int off = wsum[w] + incl - local;
    for (int e = e0; e < e1; ++e) {
        int c = cnt[e];
        int pad = (c + bm - 1) / bm * bm;
        int run = off;
        for (int q = 0; q < nwaves; ++q) {
            int h = hist[q * E + e];
            hist[q * E + e] = run;
            run += h;
        }
        for (int s = off + c; s < off + pad; ++s) sorted[s] = (int32_t)R;
        for (int b = off / bm; b < (off + pad) / bm; ++b) expert_ids[b] = e;
        off += pad;
    }
    __syncthreads();

    // ---- pass 2: stable scatter
    if (w < nwaves) {
        for (int64_t base = beg; base < end; base += 64) {
            int64_t r = base + lane;
            int key = E;
            if (r < end) {
                IdT v = ids[r];
                if (v >= 0 && v < (IdT)E) key = (int)v;
            }
            uint64_t m = match_mask(key, nbits);
            if (key < E) {
                int slot = hist[w * E + key] + __popcll(m & lower);
                sorted[slot] = (int32_t)r;
            }
            if (key < E && (m & lower) == 0) hist[w * E + key] += __popcll(m);
        }
    }
}

template <typename IdT>
__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(const IdT *__restrict__ ids, int64_t R, int E, int bm, int nwaves,
            int32_t *__restrict__ sorted, int32_t *__restrict__ expert_ids,
            int32_t *__restrict__ ntp) {
    extern __shared__ int smem[];
    plan_body(ids, R, E, bm, nwaves, sorted, expert_ids, ntp, smem);
}

// The one-workgroup plan and the activation quantisation in one launch:
// workgroup 0 builds the plan, the others quantise 64 groups each.
template <typename IdT, bool UE8M0>
__global__ void __launch_bounds__(kPlanThreads)
plan_quant_kernel(const IdT *__restrict__ ids, int64_t R, int E, int bm, int nwaves,
                  int32_t *__restrict__ sorted, int32_t *__restrict__ expert_ids,
                  int32_t *__restrict__ ntp, QuantJob q) {
    extern __shared__ int smem[];
    if (blockIdx.x == 0) {
        plan_body(ids, R, E, bm, nwaves, sorted, expert_ids, ntp, smem);
        return;
    }
    quant_act_group<UE8M0>(q.x, q.M, q.K, q.ld, q.xq, q.xs,
                           ((int64_t)(blockIdx.x - 1) * kPlanThreads + threadIdx.x) >> 4,
                           threadIdx.x & 15);
}

// ---------------------------------------------------------------------------
// Large route counts: the same plan from three launches over G workgroups.
// Workgroup g owns the contiguous routes [g C, (g + 1) C); its four waves own
// consecutive quarters of that range, as in the one-workgroup kernel.
//   hist     per-workgroup expert counts -> ws[g][e]
//   scan     one workgroup: per-expert totals, padded offsets, P, sentinels,
//            expert ids, and in place ws[g][e] = the offset of workgroup g's
//            first route of expert e (column prefix over g)
//   scatter  each workgroup recounts its waves, derives per-wave bases from
//            ws[g][e], and scatters stably (ascending r) as pass 2 above.
constexpr int kMT = 256;                     // threads per workgroup (4 waves)

constexpr int kMIt = 16;                     // 64-route rows a wave fetches at once

// Expert keys of routes base + 64 i + lane, i < kMIt (E for masked routes
// and for routes at or past end), fetched together.
template <typename IdT>
__device__ __forceinline__ void fetch_keys(const IdT *__restrict__ ids, int64_t base, int64_t end,
                                           int E, int lane, int (&key)[kMIt]) {
#pragma unroll
    for (int i = 0; i < kMIt; ++i) {
        const int64_t r = base + 64 * i + lane;
        key[i] = E;
        if (r < end) {
            const IdT v = ids[r];
            if (v >= 0 && v < (IdT)E) key[i] = (int)v;
        }
    }
}

template <typename IdT>
__device__ __forceinline__ void wave_count(const IdT *__restrict__ ids, int64_t beg, int64_t end,
                                           int E, int nbits, int lane, int *hrow) {
    const uint64_t lower = (1ull << lane) - 1ull;
    for (int64_t base = beg; base < end; base += 64 * kMIt) {
        int key[kMIt];
        fetch_keys(ids, base, end, E, lane, key);
#pragma unroll
        for (int i = 0; i < kMIt; ++i) {
            if (base + 64 * i >= end) break;
            const uint64_t m = match_mask(key[i], nbits);
            if (key[i] < E && (m & lower) == 0) hrow[key[i]] += __popcll(m);
        }
    }
}

template <typename IdT>
__device__ __forceinline__ void hist_body(const IdT *__restrict__ ids, int64_t R, int E,
                                          int64_t chunk, int32_t *__restrict__ ws, int *hist) {
    // hist: [4][E] in LDS
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nbits = 32 - __clz(E);
    for (int i = tid; i < 4 * E; i += kMT) hist[i] = 0;
    __syncthreads();
    const int64_t sub = chunk / 4;
    const int64_t beg = (int64_t)blockIdx.x * chunk + w * sub;
    const int64_t end = beg + sub < R ? beg + sub : R;
    wave_count(ids, beg, end, E, nbits, lane, hist + w * E);
    __syncthreads();
    for (int e = tid; e < E; e += kMT)
        ws[(int64_t)blockIdx.x * E + e] = hist[e] + hist[E + e] + hist[2 * E + e] + hist[3 * E + e];
}

template <typename IdT>
__global__ void __launch_bounds__(kMT)
plan_hist_kernel(const IdT *__restrict__ ids, int64_t R, int E, int64_t chunk,
                 int32_t *__restrict__ ws) {
    extern __shared__ int hist[];            // [4][E]
    hist_body(ids, R, E, chunk, ws, hist);
}

// The histogram pass and the activation quantisation in one launch:
// workgroups below G count routes, the others quantise 16 groups each.
template <typename IdT, bool UE8M0>
__global__ void __launch_bounds__(kMT)
plan_hist_quant_kernel(const IdT *__restrict__ ids, int64_t R, int E, int64_t chunk,
                       int32_t *__restrict__ ws, int G, QuantJob q) {
    extern __shared__ int hist[];            // [4][E]
    if ((int)blockIdx.x < G) {
        hist_body(ids, R, E, chunk, ws, hist);
        return;
    }
    quant_act_group<UE8M0>(q.x, q.M, q.K, q.ld, q.xq, q.xs,
                           ((int64_t)(blockIdx.x - G) * kMT + threadIdx.x) >> 4, threadIdx.x & 15);
}

__global__ void __launch_bounds__(1024)
plan_scan_kernel(int32_t *__restrict__ ws, int G, int E, int bm, int64_t R,
                 int32_t *__restrict__ sorted, int32_t *__restrict__ expert_ids,
                 int32_t *__restrict__ ntp) {
    extern __shared__ int sm[];              // counts [G][E], cnt [E], wsum [16]
    int *hist = sm, *cnt = sm + G * E, *wsum = cnt + E;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int T = blockDim.x;
    for (int i = tid; i < G * E; i += T) hist[i] = ws[i];
    __syncthreads();
    const int seg = (E + T - 1) / T;
    const int e0 = tid * seg;
    const int e1 = e0 + seg < E ? e0 + seg : E;
    int local = 0;
    for (int e = e0; e < e1; ++e) {
        int c = 0;
        for (int g = 0; g < G; ++g) c += hist[g * E + e];
        cnt[e] = c;
        local += (c + bm - 1) / bm * bm;
    }
    int incl = local;
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int q = 0; q < T / 64; ++q) {
            const int v = wsum[q];
            wsum[q] = run;
            run += v;
        }
        ntp[0] = run;                         // P
    }
    __syncthreads();
    int off = wsum[w] + incl - local;
    for (int e = e0; e < e1; ++e) {
        const int c = cnt[e];
        const int pad = (c + bm - 1) / bm * bm;
        int run = off;
        for (int g = 0; g < G; ++g) {
            const int h = hist[g * E + e];
            hist[g * E + e] = run;
            run += h;
        }
        for (int s = off + c; s < off + pad; ++s) sorted[s] = (int32_t)R;
        for (int b = off / bm; b < (off + pad) / bm; ++b) expert_ids[b] = e;
        off += pad;
    }
    __syncthreads();
    for (int i = tid; i < G * E; i += T) ws[i] = hist[i];
}

template <typename IdT>
__global__ void __launch_bounds__(kMT)
plan_scatter_kernel(const IdT *__restrict__ ids, int64_t R, int E, int64_t chunk,
                    const int32_t *__restrict__ ws, int32_t *__restrict__ sorted) {
    extern __shared__ int hist[];            // [4][E]: counts, then bases
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nbits = 32 - __clz(E);
    const uint64_t lower = (1ull << lane) - 1ull;
    for (int i = tid; i < 4 * E; i += kMT) hist[i] = 0;
    __syncthreads();
    const int64_t sub = chunk / 4;
    const int64_t beg = (int64_t)blockIdx.x * chunk + w * sub;
    const int64_t end = beg + sub < R ? beg + sub : R;
    wave_count(ids, beg, end, E, nbits, lane, hist + w * E);
    __syncthreads();
    for (int e = tid; e < E; e += kMT) {
        int run = ws[(int64_t)blockIdx.x * E + e];
        for (int q = 0; q < 4; ++q) {
            const int h = hist[q * E + e];
            hist[q * E + e] = run;
            run += h;
        }
    }
    __syncthreads();
    int *hrow = hist + w * E;
    for (int64_t base = beg; base < end; base += 64 * kMIt) {
        int key[kMIt];
        fetch_keys(ids, base, end, E, lane, key);
#pragma unroll
        for (int i = 0; i < kMIt; ++i) {
            if (base + 64 * i >= end) break;
            const uint64_t m = match_mask(key[i], nbits);
            if (key[i] < E) sorted[hrow[key[i]] + __popcll(m & lower)] = (int32_t)(base + 64 * i + lane);
            if (key[i] < E && (m & lower) == 0) hrow[key[i]] += __popcll(m);
        }
    }
}

template <typename IdT>
hipError_t launch_plan_multi(const IdT *ids, int64_t R, int E, int bm, int G, int32_t *ws,
                             int32_t *sorted, int32_t *expert_ids, int32_t *ntp, hipStream_t st) {
    int64_t chunk = (R + G - 1) / G;
    chunk = (chunk + 255) & ~int64_t(255);   // four waves x multiples of 64
    const size_t lds = (size_t)4 * E * sizeof(int);
    plan_hist_kernel<IdT><<<G, kMT, lds, st>>>(ids, R, E, chunk, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    plan_scan_kernel<<<1, 1024, (size_t)(G * E + E + 16) * sizeof(int), st>>>(ws, G, E, bm, R,
                                                                             sorted, expert_ids, ntp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    plan_scatter_kernel<IdT><<<G, kMT, lds, st>>>(ids, R, E, chunk, ws, sorted);
    return hipGetLastError();
}

template <typename IdT, bool UE8M0>
hipError_t launch_plan_quant_t(const IdT *ids, int64_t R, int E, int bm, int32_t *sorted,
                               int32_t *expert_ids, int32_t *ntp, int32_t *ws, int G,
                               const QuantJob &q, hipStream_t st) {
    const int64_t qgroups = q.M * (q.K >> 7);
    if (ws != nullptr && G > 0) {
        int64_t chunk = (R + G - 1) / G;
        chunk = (chunk + 255) & ~int64_t(255);   // four waves x multiples of 64
        const size_t lds = (size_t)4 * E * sizeof(int);
        const int64_t qwg = (qgroups + kMT / 16 - 1) / (kMT / 16);
        plan_hist_quant_kernel<IdT, UE8M0><<<(unsigned)(G + qwg), kMT, lds, st>>>(ids, R, E, chunk, ws, G, q);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        plan_scan_kernel<<<1, 1024, (size_t)(G * E + E + 16) * sizeof(int), st>>>(ws, G, E, bm, R, sorted,
                                                                                 expert_ids, ntp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        plan_scatter_kernel<IdT><<<G, kMT, lds, st>>>(ids, R, E, chunk, ws, sorted);
        return hipGetLastError();
    }
    const int nwaves = E <= 512 ? 16 : 8;
    const size_t lds = ((size_t)nwaves * E + E + 32) * sizeof(int);
    const int64_t qwg = (qgroups + kPlanThreads / 16 - 1) / (kPlanThreads / 16);
    plan_quant_kernel<IdT, UE8M0><<<(unsigned)(1 + qwg), kPlanThreads, lds, st>>>(ids, R, E, bm, nwaves, sorted,
                                                                                expert_ids, ntp, q);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_plan_quant(const void *ids, bool ids_i64, int64_t R, int E, int block_m,
                             int32_t *sorted, int32_t *expert_ids, int32_t *ntp, int32_t *ws,
                             int groups, const QuantJob &q, bool ue8m0, hipStream_t st) {
    if (ids_i64)
        return ue8m0 ? launch_plan_quant_t<int64_t, true>((const int64_t *)ids, R, E, block_m, sorted,
                                                          expert_ids, ntp, ws, groups, q, st)
                     : launch_plan_quant_t<int64_t, false>((const int64_t *)ids, R, E, block_m, sorted,
                                                           expert_ids, ntp, ws, groups, q, st);
    return ue8m0 ? launch_plan_quant_t<int32_t, true>((const int32_t *)ids, R, E, block_m, sorted, expert_ids,
                                                      ntp, ws, groups, q, st)
                 : launch_plan_quant_t<int32_t, false>((const int32_t *)ids, R, E, block_m, sorted,
                                                       expert_ids, ntp, ws, groups, q, st);
}

int plan_groups(int64_t R, int E) {
    if (R < kPlanMultiMin || E < 1) return 0;
    // ~1024 routes per group, at least 16 groups (R >= 4096: 256 or more
    // routes each): measured 4-9 us faster per plan than 2048 routes per
    // group at 8K-33K routes
    int64_t g = (R + 1023) / 1024;
    if (g < 16) g = 16;
    const int64_t gmax = (16384 - E - 16) / E;   // the scan holds all counts in 64 KB of LDS
    if (g > gmax) g = gmax;
    return g < 2 ? 0 : (int)g;
}

hipError_t launch_plan(const void *ids, bool ids_i64, int64_t R, int E, int block_m,
                       int32_t *sorted, int32_t *expert_ids, int32_t *ntp, int32_t *ws, int groups,
                       hipStream_t st) {
    if (ws != nullptr && groups > 0) {
        if (ids_i64)
            return launch_plan_multi((const int64_t *)ids, R, E, block_m, groups, ws, sorted,
                                     expert_ids, ntp, st);
        return launch_plan_multi((const int32_t *)ids, R, E, block_m, groups, ws, sorted,
                                 expert_ids, ntp, st);
    }
    const int T = kPlanThreads;
    const int nwaves = E <= 512 ? 16 : 8;
    size_t lds = ((size_t)nwaves * E + E + 32) * sizeof(int);
    if (ids_i64)
        plan_kernel<int64_t><<<1, T, lds, st>>>((const int64_t *)ids, R, E, block_m, nwaves,
                                               sorted, expert_ids, ntp);
    else
        plan_kernel<int32_t><<<1, T, lds, st>>>((const int32_t *)ids, R, E, block_m, nwaves,
                                               sorted, expert_ids, ntp);
    return hipGetLastError();
}

}  // namespace moe
