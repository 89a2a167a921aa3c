// Host-side launchers of the libmoe_fp8 kernels (internal interface between
// the C ABI layer and the kernel translation units).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace moe {

// ---- per-device launch set-up, safe for concurrent first calls
// Raises a kernel's dynamic-LDS limit on the current device once: the
// device's bit in `done` is set after the (idempotent) attribute call
// succeeds, so threads racing on a first call may each make the call, and
// no thread launches before its own call (or an earlier one) has returned.
inline hipError_t raise_lds_limit(std::atomic<uint64_t> &done, const void *fn, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    const uint64_t bit = 1ull << dev;
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    done.fetch_or(bit, std::memory_order_release);
    return hipSuccess;
}

// Compute units of the current device (256 if the query fails), queried once
// per device; a racing first call queries twice and stores the same value.
inline int device_cu_count() {
    static std::atomic<int> cached[64];        // static storage: zero-initialised
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// ---- step 1: routing plan (plan.hip)
// Workgroups of the multi-workgroup plan for R routes (0: one-workgroup
// kernel); it needs groups * E int32 of workspace.
int plan_groups(int64_t R, int E);
// ws == nullptr or groups == 0: the one-workgroup kernel.
hipError_t launch_plan(const void *ids, bool ids_i64, int64_t R, int E, int block_m,
                       int32_t *sorted, int32_t *expert_ids, int32_t *ntp, int32_t *ws, int groups,
                       hipStream_t st);

// Activation quantisation work launched together with the plan
// (moe_plan_quant): the arguments of launch_quant_act.
struct QuantJob {
    const uint16_t *x;
    int64_t M, K, ld;
    uint8_t *xq;
    float *xs;
};
// The plan (as launch_plan) and the quantisation of q (as launch_quant_act)
// with one launch fewer: the quantisation runs in the launch that builds the
// plan (one-workgroup build) or counts its routes (multi-workgroup build).
hipError_t launch_plan_quant(const void *ids, bool ids_i64, int64_t R, int E, int block_m,
                             int32_t *sorted, int32_t *expert_ids, int32_t *ntp, int32_t *ws,
                             int groups, const QuantJob &q, bool ue8m0, hipStream_t st);
// Router + plan (+ quantisation when q != nullptr) in the plan's launches
// (plan.hip): ids/w [M, top_k + n_shared] out; ws/groups as launch_plan
// (the multi-workgroup build needs ws).  The one-workgroup build keeps every
// route id in LDS: route_plan_single_lds(R, E) bytes, at most 160 KB.
size_t route_plan_single_lds(int64_t R, int E);
hipError_t launch_route_plan(const float *logits, int64_t M, int E_routed, int top_k, int n_shared,
                             float scale, int block_m, int32_t *ids, float *w, int32_t *sorted,
                             int32_t *expert_ids, int32_t *ntp, int32_t *ws, int groups,
                             const QuantJob *q, bool ue8m0, hipStream_t st);
// ---- step 2: activation quantisation (quant.hip)
hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ld,
                            uint8_t *xq, float *xs, bool ue8m0, hipStream_t st);
hipError_t launch_e4m3_encode(const float *in, uint8_t *out, int64_t n, hipStream_t st);
// count[0] = number of scales that are not powers of two in [2^-126, 2^127]
hipError_t launch_pow2_violations(const float *scales, int64_t n, uint32_t *count, hipStream_t st);

// ---- steps 3-5 (gateup.hip, down.hip)
struct GateUpArgs {
    const uint8_t *xq;
    const float *xs;
    const uint8_t *w13;
    const float *w13s;
    const uint8_t *w13e;  // W4A8: K32 exponent bytes [E, 2I, K / 32] (w13 then holds E2M1 pairs)
    const int32_t *sorted;
    const int32_t *eids;
    const int32_t *ntp;
    uint8_t *hq;
    float *hs;
    float *part;        // split-K partial sums (nsplit > 1)
    uint32_t *cnt;      // split-K arrival counters, one per (block, j-tile)
    int64_t n_cnt;      // counter words the row-tile launch zeroes (with rpos = -1)
    int32_t *rpos;      // [R] plan row of each route (pre-filled with -1)
    int4 *tiles;        // [nblocks] row tiles {first block, blocks, expert, 0} of the persistent kernels
    int32_t *tmeta;     // [17] row-tile count, then the gate/up per-XCD work counters (1..8)
    int64_t K, I, R;
    int E, top_k;
    int nkb;            // K / 128
    int jtiles;         // I / 128
    int nblocks;        // blocks_cap
    int nsplit;         // split-K factor
    int kb_per_split;
    int inter_ue8m0;
    int w13_packed;     // w13 in the tile layout of moe_prepack_w13 (kPackedTile bytes per K-block)
    float *h32;         // FP32 SwiGLU rows [plan row, I] (the column-slice gate/up only)
};

// The packed W13 layout (moe_prepack_w13): per (expert, 128-column tile,
// K-block) one contiguous tile of 256 rows x 128 B -- the 128 gate rows, then
// the 128 up rows -- whose bytes are exactly the gate/up kernels' LDS stage
// image (row r's 16-byte chunk c at r * 128 + 16 (c ^ (r & 7))).
constexpr int kPackedTile = 256 * 128;
hipError_t launch_prepack_w13(const uint8_t *w13, int64_t E, int64_t I, int64_t K, uint8_t *out,
                              hipStream_t st);

struct DownArgs {
    const uint8_t *hq;
    const float *hs;
    const uint8_t *w2;
    const float *w2s;
    const uint8_t *w2e;   // W4A8: K32 exponent bytes [E, K, I / 32] (w2 then holds E2M1 pairs)
    const float *topk_w;
    const int32_t *sorted;
    const int32_t *eids;
    const int32_t *ntp;
    uint16_t *y16;      // FP16 [R, K]: down projection of each route / its scale
    float *ys;          // FP32 [R, K / 64]: scale of each 64 columns (router weight not applied)
    const int4 *tiles;  // row tiles listed by the gate/up stage (persistent path)
    int32_t *tmeta;
    int64_t K, I, R;
    int E, top_k;
    int njb;            // I / 128
    int ctiles;         // column tiles of 256
    int nblocks;
    int nct;            // column tiles per workgroup (small-grid kernel; set by its launcher)
};

// The single-launch expert kernel (fused.hip).  Its workgroups take tickets
// from kFusedQueues counters: queue q owns the plan blocks b = q (mod
// kFusedQueues) and hands out, in ticket order, their gate/up items, then
// their down items.  A down item waits only for gate/up items of its own
// block -- lower tickets of its own queue, held by workgroups that have
// started and never wait -- so every wait ends.  The route map is complete
// before the launch (launch_fused_prep), and all counters start at zero.
constexpr int kFusedQueues = 16;
struct FusedArgs {
    uint32_t *tickets;     // [kFusedQueues] next ticket per queue
    uint32_t *cnt_h;       // [nblocks * passes] j-tiles whose intermediate rows are written
    uint32_t *cnt_t;       // [M * ctiles] route rows of (token, 256-column tile) in y
    uint32_t *err;         // [1] set if a bounded wait gave up (never, on a valid schedule)
    uint16_t *out;         // BF16 [M, K], accumulated into
    const int32_t *rpos;   // route -> plan row (-1: masked), built before the launch
    int64_t M;
    int per_queue;         // tickets per queue (gate/up + down items of its blocks)
    int lds_ticket;        // byte offset of the ticket slot in dynamic LDS (after the items' use)
};

// fp8_mma: FP8 MFMA instead of the exact FP16-widened product path;
// e8m0: (with fp8_mma) power-of-two scales applied inside the MFMA.
// Small-grid gate/up (weight stream, split-K); kb_per_split must not exceed
// gateup_stream_kmax(block_m), and the counters hold one word per
// (j-tile, block, row pass of 64).
int gateup_stream_kmax(int block_m);
hipError_t launch_gateup(const GateUpArgs &a, int block_m, bool fp8_mma, bool e8m0,
                         hipStream_t st);
// The row-tile list of the persistent kernels alone (when only the down
// stage runs persistent); launch_gateup_pipe builds it itself.  Either way
// the same launch sets rpos[0, R) = -1 and zeroes cnt[0, n_cnt) (the work of
// launch_prep, which the stage then skips).  tile_rows: 128, or 32 for the
// down kernel's small-tile form (block_m <= 32).
hipError_t launch_tiles(const GateUpArgs &a, int block_m, int tile_rows, hipStream_t st);
// Large-grid gate/up (no split-K): 128-row tiles, three-stage LDS pipeline.
hipError_t launch_gateup_pipe(const GateUpArgs &a, int block_m, bool fp8_mma, bool e8m0,
                              hipStream_t st);
hipError_t launch_down(const DownArgs &a, int block_m, bool e8m0, hipStream_t st);
// The W4A8 variant (E2M1 weights, K32 exponent bytes in w13e / w2e) on the
// small-grid kernels: gate/up as above (exact FP16 products); the down stage
// needs I / 128 <= down_w4_max_njb(block_m).
hipError_t launch_gateup_w4(const GateUpArgs &a, int block_m, hipStream_t st);
// The W4A8 gate/up on the persistent kernel (builds the row tiles and clears
// rpos and the counters itself, as launch_gateup_pipe does).
hipError_t launch_gateup_pipe_w4(const GateUpArgs &a, int block_m, hipStream_t st);
int down_w4_max_njb(int block_m);
hipError_t launch_down_w4(const DownArgs &a, int block_m, hipStream_t st);
// The W4A8 down stage on the persistent kernel (over the gate/up stage's row
// tiles: the gate/up stage must have listed them).
hipError_t launch_down_pipe_w4(const DownArgs &a, int block_m, bool small, hipStream_t st);
// Large-grid down GEMM: persistent, over the gate/up stage's row tiles --
// of 128 rows, or (small: block_m <= 32, tiles listed by launch_tiles with
// tile_rows 32) of 32 rows with a deeper W2 ring.
hipError_t launch_down_pipe(const DownArgs &a, int block_m, bool e8m0, bool small, hipStream_t st);
// Small route counts (down_cols.hip): one workgroup per 32 output columns
// over every plan block, the route sum in the same launch (no y, no
// finalize).  down_cols_fits: I = 256, block_m 8 or 16, 1 <= R <= 192.
// Two sources of the intermediate rows:
//   rq.h32 == nullptr: the FP8 rows h_q / h_s of the gate/up stage, each
//     route's plan row read from rpos (that stage's route map);
//   rq.h32 != nullptr: the FP32 SwiGLU rows of the column-slice gate/up,
//     requantised here (128-column groups, FP32 or power-of-two rule by
//     rq.ue8m0) with the routes' plan rows found by scanning the plan;
//     workgroup 0 also stores the codes and scales to rq.hq / rq.hs.
struct ColsRequant {
    const float *h32;
    uint8_t *hq;
    float *hs;
    int ue8m0;
};
bool down_cols_fits(int64_t R, int64_t I, int64_t K, int block_m);
hipError_t launch_down_cols(const DownArgs &a, int block_m, bool e8m0, const int32_t *rpos,
                            const ColsRequant &rq, uint16_t *out, hipStream_t st);
// The gate/up split over slices of 8 or 16 intermediate columns
// (gateup_slices.hip): one workgroup per (plan block, slice), K split over its
// eight waves and added in LDS; writes FP32 SwiGLU rows to a.h32 (rows that
// hold no route untouched), nothing else -- no route map, no counters.
// block_m 8 or 16, I % 16 == 0.
hipError_t launch_gateup_slices(const GateUpArgs &a, int block_m, int slice, hipStream_t st);
// The single-launch path (fused.hip): steps 3-5 over the arguments of both
// stages.  Needs I / 128 <= fused_max_njb(block_m).
int fused_max_njb(int block_m);
// counter words the single-launch path needs (the queue tickets and the
// error flag, then cnt_h, then cnt_t)
size_t fused_counter_words(int64_t nblocks, int block_m, int64_t M, int64_t ctiles);
// Its set-up launch (one workgroup): cnt[0, n_cnt) = 0, rpos[0, R) = -1, then
// rpos[sorted[p]] = p for the plan's valid rows.
hipError_t launch_fused_prep(uint32_t *cnt, size_t n_cnt, int32_t *rpos, int64_t R,
                             const int32_t *sorted, const int32_t *ntp, int64_t sorted_cap,
                             hipStream_t st);
hipError_t launch_fused(const GateUpArgs &ga, const DownArgs &da, const FusedArgs &f, int block_m,
                        bool fp8_mma, bool e8m0, hipStream_t st);
// rpos[0, n_rpos) = -1 and cnt[0, n_cnt) = 0 in one launch.
hipError_t launch_prep(uint32_t *rpos, size_t n_rpos, uint32_t *cnt, size_t n_cnt, hipStream_t st);
hipError_t launch_fill(uint32_t *p, size_t n_words, uint32_t value, hipStream_t st);
inline hipError_t launch_fill_zero(uint32_t *p, size_t n_words, hipStream_t st) {
    return launch_fill(p, n_words, 0u, st);
}
// out[t, :] = bf16(out[t, :] + sum_{j < top_k, rpos[t*top_k+j] >= 0} y[t*top_k+j, :])
hipError_t launch_finalize(uint16_t *out, const uint16_t *y16, const float *ys, const float *topk_w,
                           const int32_t *rpos, int64_t M, int64_t K, int top_k, hipStream_t st);

}  // namespace moe
