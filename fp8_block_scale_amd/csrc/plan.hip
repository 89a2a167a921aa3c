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
#include <climits>

#include "common.h"
#include "internal.h"
#include "layer.h"

namespace moe {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int64_t kPlanMultiMin = 4096;      // routes from which several workgroups pay off

// Waves of the one-workgroup plan that count routes: one per 64 routes, at
// most 16 (8 for E > 512, whose per-wave histogram rows take more LDS);
// fewer rows mean less LDS to clear and to add up per expert.
inline int plan_waves(int64_t R, int E) {
    const int cap = E <= 512 ? 16 : 8;
    const int64_t w = (R + 63) / 64;
    return w < 1 ? 1 : (w > cap ? cap : (int)w);
}

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

    // ---- pass 1: per-wave histogram.  The first kKeep groups of 64 routes
    // keep their keys and match masks in registers for pass 2 (no second
    // read of the ids, no second set of ballots, for chunks up to 256).
    auto key_at = [&](int64_t base) {
        const int64_t r = base + lane;
        int key = E;
        if (r < end) {
            IdT v = ids[r];
            if (v >= 0 && v < (IdT)E) key = (int)v;
        }
        return key;
    };
    constexpr int kKeep = 4;
    int kkey[kKeep];
    uint64_t kmask[kKeep];
    if (w < nwaves) {
#pragma unroll
        for (int it = 0; it < kKeep; ++it) {
            const int64_t base = beg + 64 * it;
            kkey[it] = E;
            kmask[it] = 0;
            if (base < end) {
                kkey[it] = key_at(base);
                kmask[it] = match_mask(kkey[it], nbits);
                if (kkey[it] < E && (kmask[it] & lower) == 0) hist[w * E + kkey[it]] += __popcll(kmask[it]);
            }
        }
        for (int64_t base = beg + 64 * kKeep; base < end; base += 64) {
            const int key = key_at(base);
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
        auto scatter = [&](int64_t base, int key, uint64_t m) {
            if (key < E) {
                int slot = hist[w * E + key] + __popcll(m & lower);
                sorted[slot] = (int32_t)(base + lane);
            }
            if (key < E && (m & lower) == 0) hist[w * E + key] += __popcll(m);
        };
#pragma unroll
        for (int it = 0; it < kKeep; ++it) {
            const int64_t base = beg + 64 * it;
            if (base < end) scatter(base, kkey[it], kmask[it]);
        }
        for (int64_t base = beg + 64 * kKeep; base < end; base += 64) {
            const int key = key_at(base);
            scatter(base, key, match_mask(key, nbits));
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

// plan_quant_kernel plus the clearing of a ClearJob by the workgroups past
// the quantisation's: workgroup 0 plans, 1 .. qwg quantise, the rest clear.
template <typename IdT, bool UE8M0>
__global__ void __launch_bounds__(kPlanThreads)
plan_quant_clear_kernel(const IdT *__restrict__ ids, int64_t R, int E, int bm, int nwaves,
                        int32_t *__restrict__ sorted, int32_t *__restrict__ expert_ids,
                        int32_t *__restrict__ ntp, QuantJob q, int64_t qwg, ClearJob c) {
    extern __shared__ int smem[];
    if (blockIdx.x == 0) {
        plan_body(ids, R, E, bm, nwaves, sorted, expert_ids, ntp, smem);
        return;
    }
    if ((int64_t)blockIdx.x <= qwg) {
        quant_act_group<UE8M0>(q.x, q.M, q.K, q.ld, q.xq, q.xs,
                               ((int64_t)(blockIdx.x - 1) * kPlanThreads + threadIdx.x) >> 4,
                               threadIdx.x & 15);
        return;
    }
    const size_t stride = (size_t)(gridDim.x - 1 - qwg) * kPlanThreads;
    for (size_t i = (size_t)(blockIdx.x - 1 - qwg) * kPlanThreads + threadIdx.x; i < c.nr + c.nc;
         i += stride) {
        if (i < c.nr) c.rpos[i] = 0xffffffffu;
        else c.cnt[i - c.nr] = 0u;
    }
}

template <typename IdT, bool UE8M0>
hipError_t launch_pqc_t(const IdT *ids, int64_t R, int E, int bm, int32_t *sorted,
                        int32_t *expert_ids, int32_t *ntp, const QuantJob &q, const ClearJob &c,
                        hipStream_t st) {
    const int64_t qgroups = q.M * (q.K >> 7);
    const int nwaves = plan_waves(R, E);
    const size_t lds = ((size_t)nwaves * E + E + 32) * sizeof(int);
    const int64_t qwg = (qgroups + kPlanThreads / 16 - 1) / (kPlanThreads / 16);
    const size_t n = c.nr + c.nc;
    int64_t cwg = (int64_t)((n + kPlanThreads - 1) / kPlanThreads);
    cwg = cwg > 64 ? 64 : cwg;
    plan_quant_clear_kernel<IdT, UE8M0><<<(unsigned)(1 + qwg + cwg), kPlanThreads, lds, st>>>(
        ids, R, E, bm, nwaves, sorted, expert_ids, ntp, q, qwg, c);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router fused into the plan: softmax top-k over each token's routed experts
// (the fixed router PR #4287 runs its expert kernel behind, real-model
// evaluation; its retained-measurement notes give the routed scaling and the
// shared expert of the E=257 geometry).  One wave routes one token: lane l
// holds logits l, l + 64, ...; k rounds each take the wave's largest
// remaining logit (equal logits: the lower expert index), so the chosen
// experts come out largest first; weight i = exp(l_i - l_max) / sum over the
// chosen, times the routed scaling; a shared expert (index E_routed) follows
// in slot k with weight 1.  Softmax is increasing, so choosing on the logits
// is choosing on the probabilities, without ties that rounding exp creates.

struct RouteJob {
    const float *logits;                  // [M, E_routed] FP32
    int64_t M;
    int Er, k, nshared;                   // routed experts, routed top-k, 0 or 1
    float scale;                          // routed scaling factor
    int32_t *ids;                         // [M, k + nshared] out
    float *w;                             // [M, k + nshared] out
};

// Wave-wide max / min of a uint32 with DPP: within each row of 16 lanes
// (quad swaps, half-row and row mirrors), then the four rows' results read
// into scalar registers -- the full wave must be active.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
    return v;
}
__device__ __forceinline__ uint32_t row_min_u32(uint32_t v) {
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = row_max_u32(v);
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = row_min_u32(v);
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return min(min(a, b), min(c, d));
}

// FP32 -> uint32 with the same order (finite values).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Token t's logits as order keys, lane l holding experts l, l + 64, ...,
// l + 64 (NPL - 1); key 0 marks an absent expert (every finite logit maps
// above 0; -0 and +0 map to one key).
template <int NPL>
__device__ __forceinline__ void load_keys(const RouteJob &j, int64_t t, uint32_t (&key)[NPL]) {
    const int lane = threadIdx.x & 63;
    const float *lrow = j.logits + t * j.Er;
    float v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < j.Er ? lrow[e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) key[i] = lane + 64 * i < j.Er ? ordered_bits(v[i] + 0.0f) : 0u;
}

// Routes token t, whose logit keys the calling wave holds (NPL per lane);
// its k + nshared ids also go to lds_ids[0, k + nshared).  Each round takes
// the wave's largest remaining key (one DPP max), then the lowest expert
// index holding it (one DPP min), and clears that key.
template <int NPL>
__device__ __forceinline__ void route_token(const RouteJob &j, int64_t t, uint32_t (&key)[NPL],
                                            int32_t *lds_ids) {
    const int lane = threadIdx.x & 63;
    float sel_v = 0.f;
    int sel_e = 0;
    for (int r = 0; r < j.k; ++r) {
        // this lane's best remaining key (ascending index: ties keep the lower)
        uint32_t bk = 0;
        int bi = 0;
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (key[i] > bk) {
                bk = key[i];
                bi = i;
            }
        const uint32_t top = wave_max_u32(bk);
        const int e = (int)wave_min_u32(bk == top ? (uint32_t)(lane + 64 * bi) : 0xFFFFFFFFu);
        if (lane == (e & 63)) {
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (i == (e >> 6)) key[i] = 0u;
        }
        if (lane == r) {
            sel_e = e;
            sel_v = __uint_as_float((top & 0x80000000u) ? (top & 0x7FFFFFFFu) : ~top);
        }
    }
    const float top = __shfl(sel_v, 0, 64);
    const float ex = lane < j.k ? expf(sel_v - top) : 0.f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    const int kk = j.k + j.nshared;
    int32_t *ids = j.ids + t * kk;
    float *w = j.w + t * kk;
    if (lane < j.k) {
        ids[lane] = sel_e;
        w[lane] = __fdiv_rn(ex, sum) * j.scale;
        lds_ids[lane] = sel_e;
    } else if (lane < kk) {               // the shared expert
        ids[lane] = j.Er;
        w[lane] = 1.0f;
        lds_ids[lane] = j.Er;
    }
}

// The tokens [t0, t1) (stride `step`) by the calling wave, the next token's
// logits loading while the current one is routed.
template <int NPL>
__device__ __forceinline__ void route_tokens(const RouteJob &j, int64_t t0, int64_t t1, int64_t step,
                                             int32_t *lds_base, int64_t lds_t0) {
    if (t0 >= t1) return;
    const int kk = j.k + j.nshared;
    uint32_t cur[NPL], nxt[NPL];
    load_keys<NPL>(j, t0, cur);
    for (int64_t t = t0; t < t1; t += step) {
        if (t + step < t1) load_keys<NPL>(j, t + step, nxt);
        route_token<NPL>(j, t, cur, lds_base + (t - lds_t0) * kk);
#pragma unroll
        for (int i = 0; i < NPL; ++i) cur[i] = nxt[i];
    }
}

// Router, plan and (optionally) the activation quantisation in one launch:
// workgroup 0 routes every token (wave w: tokens w, w + NW, ...) into LDS and
// global memory, then builds the plan from the LDS copy; the other
// workgroups quantise 64 groups each.
template <int NPL, bool QUANT, bool UE8M0>
__global__ void __launch_bounds__(kPlanThreads)
route_plan_kernel(RouteJob j, int bm, int nwaves, int32_t *__restrict__ sorted,
                  int32_t *__restrict__ expert_ids, int32_t *__restrict__ ntp, QuantJob q) {
    extern __shared__ int smem[];
    const int E = j.Er + j.nshared;
    if (blockIdx.x == 0) {
        int32_t *sIds = smem + nwaves * E + E + 32;       // after the plan's own LDS
        route_tokens<NPL>(j, threadIdx.x >> 6, j.M, kPlanThreads / 64, sIds, 0);
        __syncthreads();
        plan_body(static_cast<const int32_t *>(sIds), j.M * (j.k + j.nshared), E, bm, nwaves, sorted,
                  expert_ids,
                  ntp, smem);
        return;
    }
    if constexpr (QUANT)
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

// The router in the histogram launch (1024 threads): workgroup g routes
// tokens [g CT, (g + 1) CT) with its 16 waves (wave w: CT / 16 consecutive
// tokens) into global memory and LDS; then waves 0-3 count its routes from
// LDS exactly as hist_body does (a chunk of CT tokens' routes in four equal
// quarters -- the scatter launch recounts the same quarters).  Workgroups
// from G on quantise 64 groups each, if asked.
constexpr int kRT = 1024;

template <int NPL, bool QUANT, bool UE8M0>
__global__ void __launch_bounds__(kRT)
route_hist_kernel(RouteJob j, int64_t ctw, int32_t *__restrict__ ws, int G, QuantJob q) {
    extern __shared__ int sm[];              // hist [4][E], then this group's route ids
    if ((int)blockIdx.x >= G) {
        if constexpr (QUANT)
            quant_act_group<UE8M0>(q.x, q.M, q.K, q.ld, q.xq, q.xs,
                                   ((int64_t)(blockIdx.x - G) * kRT + threadIdx.x) >> 4,
                                   threadIdx.x & 15);
        return;
    }
    const int E = j.Er + j.nshared;
    const int kk = j.k + j.nshared;
    int *hist = sm;
    int32_t *sIds = sm + 4 * E;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < 4 * E; i += kRT) hist[i] = 0;
    const int64_t g0 = (int64_t)blockIdx.x * (kRT / 64) * ctw;      // the group's first token
    const int64_t t0 = g0 + w * ctw;
    const int64_t t1 = t0 + ctw < j.M ? t0 + ctw : j.M;
    route_tokens<NPL>(j, t0, t1, 1, sIds, g0);
    __syncthreads();
    if (w < 4) {
        const int64_t R = j.M * kk;
        const int64_t sub = (kRT / 64) * ctw * kk / 4;
        const int64_t base = g0 * kk;
        const int64_t beg = base + w * sub;
        const int64_t end = beg + sub < R ? beg + sub : R;
        if (beg < end)
            wave_count(static_cast<const int32_t *>(sIds), beg - base, end - base, E, 32 - __clz(E),
                       lane, hist + w * E);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRT)
        ws[(int64_t)blockIdx.x * E + e] = hist[e] + hist[E + e] + hist[2 * E + e] + hist[3 * E + e];
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
    const int nwaves = plan_waves(R, E);
    const size_t lds = ((size_t)nwaves * E + E + 32) * sizeof(int);
    const int64_t qwg = (qgroups + kPlanThreads / 16 - 1) / (kPlanThreads / 16);
    plan_quant_kernel<IdT, UE8M0><<<(unsigned)(1 + qwg), kPlanThreads, lds, st>>>(ids, R, E, bm, nwaves, sorted,
                                                                                expert_ids, ntp, q);
    return hipGetLastError();
}

template <int NPL, bool QUANT, bool UE8M0>
hipError_t launch_route_plan_t(const RouteJob &j, int bm, int32_t *sorted, int32_t *expert_ids,
                               int32_t *ntp, int32_t *ws, int G0, const QuantJob &q,
                               hipStream_t st) {
    const int E = j.Er + j.nshared;
    const int kk = j.k + j.nshared;
    const int64_t R = j.M * kk;
    const int64_t qgroups = QUANT ? q.M * (q.K >> 7) : 0;
    if (ws != nullptr && G0 > 0) {
        // groups of 16 * ctw whole tokens; no more groups than the workspace holds
        const int64_t per = kRT / 64;
        const int64_t ctw = (j.M + per * G0 - 1) / (per * G0);
        const int G = (int)((j.M + per * ctw - 1) / (per * ctw));
        const int64_t chunk = per * ctw * kk;
        const size_t lds = ((size_t)4 * E + (size_t)chunk) * sizeof(int);
        if (lds > 64 * 1024) return hipErrorInvalidValue;
        const int64_t qwg = (qgroups + kRT / 16 - 1) / (kRT / 16);
        route_hist_kernel<NPL, QUANT, UE8M0><<<(unsigned)(G + qwg), kRT, lds, st>>>(j, ctw, ws, G, q);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        plan_scan_kernel<<<1, 1024, (size_t)(G * E + E + 16) * sizeof(int), st>>>(ws, G, E, bm, R, sorted,
                                                                                 expert_ids, ntp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        plan_scatter_kernel<int32_t><<<G, kMT, (size_t)4 * E * sizeof(int), st>>>(j.ids, R, E, chunk, ws,
                                                                                   sorted);
        return hipGetLastError();
    }
    const int nwaves = plan_waves(R, E);
    const size_t lds = ((size_t)nwaves * E + E + 32 + (size_t)R) * sizeof(int);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const int64_t qwg = (qgroups + kPlanThreads / 16 - 1) / (kPlanThreads / 16);
    if (lds > 64 * 1024) {
        static std::atomic<uint64_t> lds_set{0};
        const hipError_t e = raise_lds_limit(lds_set, (const void *)route_plan_kernel<NPL, QUANT, UE8M0>,
                                             160 * 1024);
        if (e != hipSuccess) return e;
    }
    route_plan_kernel<NPL, QUANT, UE8M0><<<(unsigned)(1 + qwg), kPlanThreads, lds, st>>>(j, bm, nwaves, sorted,
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
    const int nwaves = plan_waves(R, E);
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

namespace moe {

size_t route_plan_single_lds(int64_t R, int E) {
    const int nwaves = plan_waves(R, E);
    return ((size_t)nwaves * E + E + 32 + (size_t)R) * sizeof(int);
}

template <int NPL>
hipError_t route_plan_npl(const RouteJob &j, int block_m, int32_t *sorted, int32_t *expert_ids,
                          int32_t *ntp, int32_t *ws, int groups, const QuantJob *q, bool ue8m0,
                          hipStream_t st) {
    QuantJob none{};
    if (q == nullptr)
        return launch_route_plan_t<NPL, false, false>(j, block_m, sorted, expert_ids, ntp, ws, groups, none,
                                                      st);
    return ue8m0 ? launch_route_plan_t<NPL, true, true>(j, block_m, sorted, expert_ids, ntp, ws, groups, *q, st)
                 : launch_route_plan_t<NPL, true, false>(j, block_m, sorted, expert_ids, ntp, ws, groups, *q, st);
}

hipError_t launch_route_plan(const float *logits, int64_t M, int E_routed, int top_k, int n_shared,
                             float scale, int block_m, int32_t *ids, float *w, int32_t *sorted,
                             int32_t *expert_ids, int32_t *ntp, int32_t *ws, int groups,
                             const QuantJob *q, bool ue8m0, hipStream_t st) {
    RouteJob j;
    j.logits = logits;
    j.M = M;
    j.Er = E_routed;
    j.k = top_k;
    j.nshared = n_shared;
    j.scale = scale;
    j.ids = ids;
    j.w = w;
    // logits per lane: the fewest of 2, 4, 5, 8, 16 that hold E_routed
    const int npl = E_routed <= 128 ? 2 : E_routed <= 256 ? 4 : E_routed <= 320 ? 5
                  : E_routed <= 512 ? 8 : 16;
    switch (npl) {
        case 2: return route_plan_npl<2>(j, block_m, sorted, expert_ids, ntp, ws, groups, q, ue8m0, st);
        case 4: return route_plan_npl<4>(j, block_m, sorted, expert_ids, ntp, ws, groups, q, ue8m0, st);
        case 5: return route_plan_npl<5>(j, block_m, sorted, expert_ids, ntp, ws, groups, q, ue8m0, st);
        case 8: return route_plan_npl<8>(j, block_m, sorted, expert_ids, ntp, ws, groups, q, ue8m0, st);
        default: return route_plan_npl<16>(j, block_m, sorted, expert_ids, ntp, ws, groups, q, ue8m0, st);
    }
}

hipError_t launch_plan_quant_clear(const void *ids, bool ids_i64, int64_t R, int E, int block_m,
                                   int32_t *sorted, int32_t *expert_ids, int32_t *ntp,
                                   const QuantJob &q, bool ue8m0, const ClearJob &c, hipStream_t st) {
    if (ids_i64)
        return ue8m0 ? launch_pqc_t<int64_t, true>((const int64_t *)ids, R, E, block_m, sorted, expert_ids, ntp, q, c, st)
                     : launch_pqc_t<int64_t, false>((const int64_t *)ids, R, E, block_m, sorted, expert_ids, ntp, q, c, st);
    return ue8m0 ? launch_pqc_t<int32_t, true>((const int32_t *)ids, R, E, block_m, sorted, expert_ids, ntp, q, c, st)
                 : launch_pqc_t<int32_t, false>((const int32_t *)ids, R, E, block_m, sorted, expert_ids, ntp, q, c, st);
}

}  // namespace moe
