// C ABI of libmoe_fp8.so: argument validation, workspace layout and the
// launch sequence of each entry point (declared in include/moe_fp8.h).
#include <atomic>
#include <cmath>
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/moe_fp8.h"
#include "internal.h"
#include "layer.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

moe_status hip_check(hipError_t e, const char *what) {
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kMaxE = 1024;

int64_t plan_sorted_cap(int64_t M, int32_t top_k, int32_t E, int32_t bm) {
    int64_t R = M * top_k;
    int64_t n = R + (E < R ? E : R) * (int64_t)(bm - 1);
    return (n + bm - 1) / bm * bm;
}

bool valid_block_m(int32_t bm) { return bm == 8 || bm == 16 || bm == 32 || bm == 64 || bm == 128; }

// Kernel families and the gate/up work split.  The persistent kernels walk
// 128-row tiles of one expert (the row-tile list, built in the gate/up
// stage, is shared by both stages) and reuse each weight tile across all of
// its rows; the per-block kernels stream an expert's weights once per plan
// block (per 64-row pass), which wins while experts hold few rows each.
// The small-grid gate/up splits K over enough workgroups to cover the chip.
struct SplitChoice {
    int nsplit;
    int kb_per_split;
    bool gu_persistent;
    bool dn_persistent;
    bool dn_small;       // the persistent down on row tiles of 32 rows (deeper W2 ring)
    bool dn_cols;        // the down stage split over output columns, route sum included
    bool gu_cols;        // the gate/up split over column slices (FP32 rows; needs dn_cols)
    int gu_slice;        // its slice width: 8 or 16 intermediate columns
    bool fused;          // steps 3-5 in one launch (moe_fp8_experts only)
};

constexpr int64_t kPersistentTiles = 512;   // (block, j-tile) pairs
constexpr double kStreamFill = 192.0;       // workgroups the stream kernel's split aims at
// The column-slice gate/up by default only for short K with few routes:
// measured at the tiny shape (K = 256, 8 routes) steps 3-5 took 9.8 against
// 12.6 us (no clearing launch, no split-K), but at the decode shape (K =
// 7168) 22.8 against 21.9 us at M = 1 and 37.6 against 28.1 at M = 2: its
// gate/up streams no faster than the split-K kernel there, and requantising
// the FP32 rows in the down stage costs ~2 us.
constexpr int64_t kSlicesMaxRoutes = 32;
constexpr int64_t kSlicesMaxK = 1024;

SplitChoice choose_split(int64_t R, int32_t E, int64_t blocks_cap, int64_t jtiles, int64_t K,
                         int64_t I, int32_t bm, uint32_t flags, bool w4) {
    const int64_t nkb = K / 128;
    const int64_t tiles = blocks_cap * jtiles;
    const int64_t forced = (flags & MOE_F_SPLITK_MASK) >> MOE_F_SPLITK_SHIFT;
    const uint32_t gu_path = (flags & MOE_F_GATEUP_PATH_MASK) >> MOE_F_GATEUP_PATH_SHIFT;
    const uint32_t dn_path = (flags & MOE_F_DOWN_PATH_MASK) >> MOE_F_DOWN_PATH_SHIFT;
    const bool fits = K <= 32768 && I <= 32768;
    const bool big = tiles >= kPersistentTiles && fits;
    // Measured on the page-1, skew and zipf workloads: the per-block gate/up
    // is faster up to ~3/4 of a 64-row pass of routes per expert on average.
    const int64_t pass_rows = bm < 64 ? bm : 64;
    const bool dense = 4 * R > 3 * pass_rows * (int64_t)E;
    const uint32_t fuse = (flags & MOE_F_FUSE_MASK) >> MOE_F_FUSE_SHIFT;
    // Plan blocks expected to hold routes under uniform routing: the experts
    // hit, E (1 - (1 - 1/E)^R), or R / block_m if more, at most the capacity.
    const double hit = (double)E * -std::expm1((double)R * std::log1p(-1.0 / (double)E));
    double blocks = hit > (double)R / bm ? hit : (double)R / bm;
    if (blocks > (double)blocks_cap) blocks = (double)blocks_cap;
    // The persistent down kernel streams W2 without a break across its items;
    // with FP8 weights it wins once the (block, 256-column) items outnumber
    // the CUs twice over (measured at the decode shape: M=4, 8, 16 faster,
    // M=1 with 252 items slower).  With E2M1 weights (half the bytes per
    // item) the per-block down kernel stayed 2-4% faster at M=4-16.
    const bool dn_many = !w4 && blocks * (double)((K + 255) / 256) >= 512.0 && fits;
    SplitChoice c;
    c.gu_persistent = gu_path == MOE_PATH_PERSISTENT ||
                      (gu_path == MOE_PATH_AUTO && forced == 0 && big && dense);
    c.dn_persistent = dn_path == MOE_PATH_PERSISTENT || (dn_path == MOE_PATH_AUTO && (big || dn_many));
    // The single launch only on request: measured on MI355X it is slower than
    // the two stages at every size tried (decode M=1: 34 against 27 us; M=16:
    // 155 against 120 us): every workgroup pays the larger item's LDS, so
    // neither item kind keeps its own occupancy and ring depth.
    if (fuse == MOE_FUSE_ON) c.gu_persistent = c.dn_persistent = false;   // (forced paths: rejected)
    c.fused = fuse == MOE_FUSE_ON;
    // Without the persistent gate/up (whose row tiles hold up to 128 rows) the
    // down stage's row tiles are cut at 32 rows when blocks allow: experts
    // then hold a block or two each, and the 32-row tile leaves LDS for four
    // W2 stages in flight instead of three.
    c.dn_small = c.dn_persistent && !c.gu_persistent && bm <= 32;
    // The column-split down with its own route sum (no per-route buffer, no
    // route-sum launch) wherever it applies: measured at the decode shape
    // faster than the per-block and the persistent down at M = 1 .. 16 (down
    // stage 7.4 / 10.3 / 14.2 / 22.2 / 36.7 us at M = 1, 2, 4, 8, 16).
    c.dn_cols = fuse != MOE_FUSE_ON && moe::down_cols_fits(R, I, K, bm) &&
                (dn_path == MOE_PATH_COLUMNS || dn_path == MOE_PATH_AUTO);
    if (c.dn_cols) c.dn_persistent = c.dn_small = false;
    // The column-slice gate/up leaves FP32 rows that only the column-split
    // down reads (requantising them as it loads them); it multiplies exactly
    // (FP16-widened codes) and needs no clearing launch and no counters.
    const bool slices_ok = c.dn_cols && !w4 && forced == 0 &&
                           !(flags & (MOE_F_FP8_GATEUP | MOE_F_W13_PACKED));
    c.gu_cols = slices_ok && (gu_path == MOE_PATH_COLUMNS ||
                              (gu_path == MOE_PATH_AUTO && R <= kSlicesMaxRoutes && K <= kSlicesMaxK));
    if (c.gu_cols) c.gu_persistent = false;
    c.gu_slice = 16;
    if (c.gu_persistent || c.gu_cols) {
        c.nsplit = 1;
        c.kb_per_split = (int)nkb;
        return c;
    }
    const int64_t npass = bm > 64 ? bm / 64 : 1;
    int64_t s = forced;
    if (s == 0) {
        // Workgroups that will have work: the plan blocks expected above, not
        // the capacity's one block per route.  The smallest split that fills
        // 3/4 of the chip in one round: a partial second round costs nearly
        // a whole one (decode M=4: 37 us at 288 workgroups against 26 us at
        // 216).
        double units = blocks * (double)jtiles * (double)npass;
        if (units < 1.0) units = 1.0;
        s = (int64_t)std::ceil(kStreamFill / units);
    }
    const int64_t kmax = moe::gateup_stream_kmax(bm);
    if (s < (nkb + kmax - 1) / kmax) s = (nkb + kmax - 1) / kmax;
    if (s > nkb) s = nkb;
    if (s < 1) s = 1;
    const int64_t kps = (nkb + s - 1) / s;
    s = (nkb + kps - 1) / kps;        // no empty splits
    c.nsplit = (int)s;
    c.kb_per_split = (int)kps;
    return c;
}

struct WsLayout {
    size_t hq, hs, y, ys, rpos, tiles, cnt, part, h32, total;
    size_t splitk_words;              // split-K counters
    size_t cnt_words;                 // all counters (split-K, then the single launch's), zeroed per call
    SplitChoice sp;
};

WsLayout ws_layout(int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k, int32_t block_m,
                   int64_t sorted_cap, uint32_t flags, bool w4 = false) {
    WsLayout l;
    int64_t blocks_cap = sorted_cap / block_m;
    int64_t jtiles = I / 128;
    l.sp = choose_split(M * top_k, E, blocks_cap, jtiles, K, I, block_m, flags, w4);
    size_t off = 0;
    l.hq = off;
    off = align256(off + (size_t)sorted_cap * I);
    l.hs = off;
    off = align256(off + (size_t)sorted_cap * (I / 128) * 4);
    const size_t R = (size_t)M * top_k;
    l.y = off;                           // FP16 [R, K], then FP32 scales [R, K / 64]
    off = align256(off + R * K * 2);
    l.ys = off;
    off = align256(off + R * (size_t)(K / 64) * 4);
    l.rpos = off;
    off = align256(off + R * 4);
    l.tiles = off;                       // row tiles [blocks_cap] int4, then 17 ints of tile meta
    off = align256(off + (size_t)blocks_cap * 16 + 17 * 4);
    l.cnt = off;
    size_t ntiles = (size_t)blocks_cap * jtiles;
    l.splitk_words = l.sp.nsplit > 1 ? ntiles * (block_m > 64 ? block_m / 64 : 1) : 0;
    l.cnt_words = l.splitk_words;
    if (l.sp.fused) l.cnt_words += moe::fused_counter_words(blocks_cap, block_m, M, (K + 255) / 256);
    off = align256(off + l.cnt_words * 4);
    l.part = off;
    if (l.sp.nsplit > 1) off = align256(off + ntiles * l.sp.nsplit * block_m * 256 * 4);
    l.h32 = off;                         // FP32 SwiGLU rows [sorted_cap, I] (column-slice gate/up)
    if (l.sp.gu_cols) off = align256(off + (size_t)sorted_cap * I * 4);
    l.total = off;
    return l;
}

moe_status check_experts_shape(int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                               int32_t block_m, int64_t sorted_cap) {
    if (M < 0 || K <= 0 || I <= 0 || E < 1 || top_k < 1)
        return fail(MOE_ERR_SHAPE, "need M >= 0, K > 0, I > 0, E >= 1, top_k >= 1");
    if (K % 128 != 0 || I % 128 != 0)
        return fail(MOE_ERR_SHAPE, "K (%lld) and I (%lld) must be multiples of 128",
                    (long long)K, (long long)I);
    if (!valid_block_m(block_m))
        return fail(MOE_ERR_UNSUPPORTED, "block_m %d not in {8, 16, 32, 64, 128}", block_m);
    if (sorted_cap < 0 || sorted_cap % block_m != 0)
        return fail(MOE_ERR_SHAPE, "sorted_cap must be a non-negative multiple of block_m");
    if (M * top_k >= (int64_t)1 << 31)
        return fail(MOE_ERR_SHAPE, "M * top_k must fit in int32");
    const int64_t blocks = sorted_cap / block_m;
    const int64_t grid_up = blocks * (I / 128) * (K / 128);   // worst split-K factor
    const int64_t grid_dn = blocks * ((K + 255) / 256);
    if (grid_up >= ((int64_t)1 << 31) || grid_dn >= ((int64_t)1 << 31))
        return fail(MOE_ERR_SHAPE, "plan too large for one launch grid");
    return MOE_OK;
}

}  // namespace

MOE_API const char *moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: size out of range or inconsistent";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: misaligned pointer or leading dimension";
        case MOE_ERR_CAPACITY: return "MOE_ERR_CAPACITY: plan buffers or workspace too small";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: not implemented for these arguments";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
    }
    return "unknown moe_status";
}

MOE_API const char *moe_last_hip_error(void) { return g_err; }
MOE_API const char *moe_last_error(void) { return g_err; }

// ------------------------------------------------------------------ plan

MOE_API moe_status moe_plan_capacity(int64_t M, int32_t top_k, int32_t E, int32_t block_m,
                                     int64_t *sorted_cap, int64_t *blocks_cap) {
    if (!sorted_cap || !blocks_cap) return fail(MOE_ERR_NULL, "output pointer is NULL");
    if (M < 0 || top_k < 1 || E < 1 || block_m < 1)
        return fail(MOE_ERR_SHAPE, "need M >= 0, top_k >= 1, E >= 1, block_m >= 1");
    if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E = %d exceeds %d", E, kMaxE);
    if (block_m > 256) return fail(MOE_ERR_UNSUPPORTED, "block_m = %d exceeds 256", block_m);
    if (M * top_k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "M * top_k must fit in int32");
    *sorted_cap = plan_sorted_cap(M, top_k, E, block_m);
    *blocks_cap = *sorted_cap / block_m;
    return MOE_OK;
}

MOE_API size_t moe_plan_workspace_size(int64_t M, int32_t top_k, int32_t E, int32_t) {
    if (M <= 0 || top_k <= 0 || E <= 0) return 0;
    return (size_t)moe::plan_groups(M * top_k, E) * (size_t)E * sizeof(int32_t);
}

namespace {

// Validation of moe_plan's arguments; *groups = workgroups of the
// multi-workgroup build when the workspace holds it, else 0.
moe_status check_plan(const void *topk_ids, int32_t ids_dtype, int64_t M, int32_t top_k, int32_t E,
                      int32_t block_m, const int32_t *sorted_token_ids, int64_t sorted_cap,
                      const int32_t *expert_ids, int64_t blocks_cap,
                      const int32_t *num_tokens_post_padded, const void *workspace,
                      size_t workspace_bytes, int *groups) {
    int64_t need_sorted, need_blocks;
    moe_status st = moe_plan_capacity(M, top_k, E, block_m, &need_sorted, &need_blocks);
    if (st != MOE_OK) return st;
    if (ids_dtype != MOE_IDS_I32 && ids_dtype != MOE_IDS_I64)
        return fail(MOE_ERR_SHAPE, "ids_dtype %d is neither MOE_IDS_I32 nor MOE_IDS_I64", ids_dtype);
    if (!num_tokens_post_padded) return fail(MOE_ERR_NULL, "num_tokens_post_padded is NULL");
    if (M > 0 && (!topk_ids || !sorted_token_ids || !expert_ids))
        return fail(MOE_ERR_NULL, "topk_ids, sorted_token_ids and expert_ids are required");
    if (sorted_cap < need_sorted || blocks_cap < need_blocks)
        return fail(MOE_ERR_CAPACITY, "plan buffers [%lld, %lld] below capacity [%lld, %lld]",
                    (long long)sorted_cap, (long long)blocks_cap, (long long)need_sorted,
                    (long long)need_blocks);
    if (sorted_cap < blocks_cap * block_m)
        return fail(MOE_ERR_CAPACITY, "sorted_cap must be >= blocks_cap * block_m");
    // the multi-workgroup build when the caller's workspace holds it
    const int g = M > 0 ? moe::plan_groups(M * top_k, E) : 0;
    const bool multi = g > 0 && workspace != nullptr && ((uintptr_t)workspace & 3u) == 0 &&
                       workspace_bytes >= (size_t)g * (size_t)E * sizeof(int32_t);
    *groups = multi ? g : 0;
    return MOE_OK;
}

moe_status check_quant(const void *x_bf16, int64_t M, int64_t K, int64_t ld_x, const uint8_t *x_q,
                       const float *x_s, int32_t scale_mode) {
    if (M < 0 || K <= 0 || K % 128 != 0)
        return fail(MOE_ERR_SHAPE, "need M >= 0 and K a positive multiple of 128");
    if (ld_x < K) return fail(MOE_ERR_SHAPE, "ld_x (%lld) < K (%lld)", (long long)ld_x, (long long)K);
    if (scale_mode != MOE_SCALE_FP32 && scale_mode != MOE_SCALE_UE8M0)
        return fail(MOE_ERR_SHAPE, "unknown scale_mode %d", scale_mode);
    if (M == 0) return MOE_OK;
    if (!x_bf16 || !x_q || !x_s) return fail(MOE_ERR_NULL, "x_bf16, x_q and x_s are required");
    if (!aligned16(x_bf16) || ld_x % 8 != 0 || !aligned16(x_q))
        return fail(MOE_ERR_ALIGN, "x_bf16 and x_q must be 16-byte aligned and ld_x a multiple of 8");
    if (((uintptr_t)x_s & 3u) != 0) return fail(MOE_ERR_ALIGN, "x_s must be 4-byte aligned");
    return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_plan(const void *topk_ids, int32_t ids_dtype, int64_t M, int32_t top_k,
                            int32_t E, int32_t block_m, int32_t *sorted_token_ids,
                            int64_t sorted_cap, int32_t *expert_ids, int64_t blocks_cap,
                            int32_t *num_tokens_post_padded, void *workspace,
                            size_t workspace_bytes, void *stream) {
    int groups = 0;
    moe_status st = check_plan(topk_ids, ids_dtype, M, top_k, E, block_m, sorted_token_ids, sorted_cap,
                               expert_ids, blocks_cap, num_tokens_post_padded, workspace,
                               workspace_bytes, &groups);
    if (st != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (M == 0) {
        // a fill kernel, not a memset node, so the call stays graph-capturable
        return hip_check(moe::launch_fill_zero((uint32_t *)num_tokens_post_padded, 1, s),
                         "moe_plan: clear num_tokens_post_padded");
    }
    return hip_check(moe::launch_plan(topk_ids, ids_dtype == MOE_IDS_I64, M * top_k, E, block_m,
                                      sorted_token_ids, expert_ids, num_tokens_post_padded,
                                      groups > 0 ? (int32_t *)workspace : nullptr, groups, s),
                     "moe_plan: launch");
}

MOE_API moe_status moe_plan_quant(const void *topk_ids, int32_t ids_dtype, int64_t M, int32_t top_k,
                                  int32_t E, int32_t block_m, int32_t *sorted_token_ids,
                                  int64_t sorted_cap, int32_t *expert_ids, int64_t blocks_cap,
                                  int32_t *num_tokens_post_padded, void *workspace,
                                  size_t workspace_bytes, const void *x_bf16, int64_t K,
                                  int64_t ld_x, uint8_t *x_q, float *x_s, int32_t scale_mode,
                                  void *stream) {
    int groups = 0;
    moe_status st = check_plan(topk_ids, ids_dtype, M, top_k, E, block_m, sorted_token_ids, sorted_cap,
                               expert_ids, blocks_cap, num_tokens_post_padded, workspace,
                               workspace_bytes, &groups);
    if (st != MOE_OK) return st;
    st = check_quant(x_bf16, M, K, ld_x, x_q, x_s, scale_mode);
    if (st != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (M == 0)
        return hip_check(moe::launch_fill_zero((uint32_t *)num_tokens_post_padded, 1, s),
                         "moe_plan_quant: clear num_tokens_post_padded");
    moe::QuantJob q;
    q.x = (const uint16_t *)x_bf16;
    q.M = M;
    q.K = K;
    q.ld = ld_x;
    q.xq = x_q;
    q.xs = x_s;
    return hip_check(moe::launch_plan_quant(topk_ids, ids_dtype == MOE_IDS_I64, M * top_k, E, block_m,
                                            sorted_token_ids, expert_ids, num_tokens_post_padded,
                                            groups > 0 ? (int32_t *)workspace : nullptr, groups, q,
                                            scale_mode == MOE_SCALE_UE8M0, s),
                     "moe_plan_quant: launch");
}

MOE_API moe_status moe_route_plan(const float *router_logits, int64_t M, int32_t E_routed,
                                  int32_t top_k, int32_t n_shared, float routed_scaling,
                                  int32_t block_m, int32_t *topk_ids, float *topk_weights,
                                  int32_t *sorted_token_ids, int64_t sorted_cap,
                                  int32_t *expert_ids, int64_t blocks_cap,
                                  int32_t *num_tokens_post_padded, void *workspace,
                                  size_t workspace_bytes, const void *x_bf16, int64_t K,
                                  int64_t ld_x, uint8_t *x_q, float *x_s, int32_t scale_mode,
                                  void *stream) {
    if (E_routed < 1 || top_k < 1 || top_k > 32 || top_k > E_routed)
        return fail(MOE_ERR_SHAPE, "need 1 <= top_k <= min(E_routed, 32) (top_k %d, E_routed %d)",
                    top_k, E_routed);
    if (n_shared != 0 && n_shared != 1) return fail(MOE_ERR_SHAPE, "n_shared must be 0 or 1");
    if (E_routed + n_shared > kMaxE)
        return fail(MOE_ERR_SHAPE, "E_routed + n_shared = %d exceeds %d", E_routed + n_shared, kMaxE);
    if (!std::isfinite(routed_scaling)) return fail(MOE_ERR_SHAPE, "routed_scaling must be finite");
    const int32_t E = E_routed + n_shared, kk = top_k + n_shared;
    int groups = 0;
    moe_status st = check_plan(topk_ids, MOE_IDS_I32, M, kk, E, block_m, sorted_token_ids, sorted_cap,
                               expert_ids, blocks_cap, num_tokens_post_padded, workspace,
                               workspace_bytes, &groups);
    if (st != MOE_OK) return st;
    const bool quant = x_bf16 != nullptr;
    if (quant) {
        st = check_quant(x_bf16, M, K, ld_x, x_q, x_s, scale_mode);
        if (st != MOE_OK) return st;
    }
    hipStream_t s = (hipStream_t)stream;
    if (M == 0)
        return hip_check(moe::launch_fill_zero((uint32_t *)num_tokens_post_padded, 1, s),
                         "moe_route_plan: clear num_tokens_post_padded");
    if (!router_logits || !topk_weights)
        return fail(MOE_ERR_NULL, "router_logits and topk_weights are required");
    if (((uintptr_t)router_logits & 3u) || ((uintptr_t)topk_weights & 3u) || ((uintptr_t)topk_ids & 3u))
        return fail(MOE_ERR_ALIGN, "router_logits, topk_ids and topk_weights must be 4-byte aligned");
    if (groups == 0 && moe::route_plan_single_lds(M * kk, E) > 160 * 1024)
        return fail(MOE_ERR_CAPACITY,
                    "%lld routes need the plan workspace (moe_plan_workspace_size bytes)",
                    (long long)(M * kk));
    moe::QuantJob q;
    if (quant) {
        q.x = (const uint16_t *)x_bf16;
        q.M = M;
        q.K = K;
        q.ld = ld_x;
        q.xq = x_q;
        q.xs = x_s;
    }
    return hip_check(moe::launch_route_plan(router_logits, M, E_routed, top_k, n_shared, routed_scaling,
                                            block_m, topk_ids, topk_weights, sorted_token_ids,
                                            expert_ids, num_tokens_post_padded,
                                            groups > 0 ? (int32_t *)workspace : nullptr, groups,
                                            quant ? &q : nullptr, scale_mode == MOE_SCALE_UE8M0, s),
                     "moe_route_plan: launch");
}

// ------------------------------------------------------------- quant act

MOE_API moe_status moe_quant_act(const void *x_bf16, int64_t M, int64_t K, int64_t ld_x,
                                 uint8_t *x_q, float *x_s, int32_t scale_mode, void *stream) {
    const moe_status st = check_quant(x_bf16, M, K, ld_x, x_q, x_s, scale_mode);
    if (st != MOE_OK || M == 0) return st;
    return hip_check(moe::launch_quant_act((const uint16_t *)x_bf16, M, K, ld_x, x_q, x_s,
                                           scale_mode == MOE_SCALE_UE8M0, (hipStream_t)stream),
                     "moe_quant_act: launch");
}

MOE_API moe_status moe_debug_e4m3_encode(const float *in, uint8_t *out, int64_t n, void *stream) {
    if (n < 0) return fail(MOE_ERR_SHAPE, "n < 0");
    if (n == 0) return MOE_OK;
    if (!in || !out) return fail(MOE_ERR_NULL, "in and out are required");
    return hip_check(moe::launch_e4m3_encode(in, out, n, (hipStream_t)stream),
                     "moe_debug_e4m3_encode: launch");
}

MOE_API moe_status moe_debug_count_non_pow2(const float *scales, int64_t n, uint32_t *count,
                                            void *stream) {
    if (n < 0) return fail(MOE_ERR_SHAPE, "n < 0");
    if (!count || (n > 0 && !scales)) return fail(MOE_ERR_NULL, "scales and count are required");
    return hip_check(moe::launch_pow2_violations(scales, n, count, (hipStream_t)stream),
                     "moe_debug_count_non_pow2: launch");
}

// --------------------------------------------------------------- experts

MOE_API size_t moe_fp8_experts_workspace_size(int64_t M, int64_t K, int64_t I, int32_t E,
                                              int32_t top_k, int32_t block_m, int64_t sorted_cap,
                                              uint32_t flags) {
    if (check_experts_shape(M, K, I, E, top_k, block_m, sorted_cap) != MOE_OK) return 0;
    return ws_layout(M, K, I, E, top_k, block_m, sorted_cap, flags).total;
}

MOE_API moe_status moe_fp8_experts_workspace_layout(int64_t M, int64_t K, int64_t I, int32_t E,
                                                    int32_t top_k, int32_t block_m,
                                                    int64_t sorted_cap, uint32_t flags,
                                                    size_t *h_q_offset, size_t *h_s_offset) {
    moe_status st = check_experts_shape(M, K, I, E, top_k, block_m, sorted_cap);
    if (st != MOE_OK) return st;
    if (!h_q_offset || !h_s_offset) return fail(MOE_ERR_NULL, "output pointer is NULL");
    WsLayout l = ws_layout(M, K, I, E, top_k, block_m, sorted_cap, flags);
    *h_q_offset = l.hq;
    *h_s_offset = l.hs;
    return MOE_OK;
}

namespace {

moe_status check_flags(uint32_t flags, int64_t K, int64_t I, int32_t block_m, int64_t R) {
    const uint32_t known = MOE_F_INTER_UE8M0 | MOE_F_MMA_E8M0 | MOE_F_FP8_GATEUP | MOE_F_SPLITK_MASK |
                           MOE_F_GATEUP_PATH_MASK | MOE_F_DOWN_PATH_MASK | MOE_F_FUSE_MASK |
                           MOE_F_W13_PACKED;
    if (flags & ~known) return fail(MOE_ERR_SHAPE, "unknown flag bits 0x%x", flags & ~known);
    const uint32_t gp = (flags & MOE_F_GATEUP_PATH_MASK) >> MOE_F_GATEUP_PATH_SHIFT;
    const uint32_t dp = (flags & MOE_F_DOWN_PATH_MASK) >> MOE_F_DOWN_PATH_SHIFT;
    if (gp > MOE_PATH_COLUMNS || dp > MOE_PATH_COLUMNS)
        return fail(MOE_ERR_SHAPE, "kernel path override must be 0, 1, 2 or 3");
    if ((dp == MOE_PATH_COLUMNS || gp == MOE_PATH_COLUMNS) && R > 0 &&
        !moe::down_cols_fits(R, I, K, block_m))
        return fail(MOE_ERR_UNSUPPORTED,
                    "the column-split kernels need I = 256, block_m 8 or 16 and M * top_k <= 192");
    if (gp == MOE_PATH_COLUMNS &&
        (dp == MOE_PATH_STREAM || dp == MOE_PATH_PERSISTENT || (flags & MOE_F_SPLITK_MASK) ||
         (flags & (MOE_F_FP8_GATEUP | MOE_F_W13_PACKED))))
        return fail(MOE_ERR_SHAPE, "the column-slice gate/up runs with the column-split down, "
                                   "exact products, unpacked W13 and no split-K factor");
    if ((gp == MOE_PATH_PERSISTENT || dp == MOE_PATH_PERSISTENT) && (K > 32768 || I > 32768))
        return fail(MOE_ERR_UNSUPPORTED, "the persistent kernels need K, I <= 32768");
    if (gp == MOE_PATH_PERSISTENT && (flags & MOE_F_SPLITK_MASK))
        return fail(MOE_ERR_SHAPE, "a forced split-K factor needs the per-block gate/up kernel");
    if ((flags & MOE_F_MMA_E8M0) && !(flags & MOE_F_INTER_UE8M0))
        return fail(MOE_ERR_SHAPE, "MOE_F_MMA_E8M0 requires MOE_F_INTER_UE8M0");
    const uint32_t fu = (flags & MOE_F_FUSE_MASK) >> MOE_F_FUSE_SHIFT;
    if (fu > MOE_FUSE_ON) return fail(MOE_ERR_SHAPE, "fuse choice must be 0, 1 or 2");
    if (fu == MOE_FUSE_ON && (gp == MOE_PATH_PERSISTENT || gp == MOE_PATH_COLUMNS ||
                              dp == MOE_PATH_PERSISTENT || dp == MOE_PATH_COLUMNS))
        return fail(MOE_ERR_SHAPE, "MOE_FUSE_ON runs the per-block kernel family: no other path");
    if (fu == MOE_FUSE_ON && I / 128 > moe::fused_max_njb(block_m))
        return fail(MOE_ERR_UNSUPPORTED, "MOE_FUSE_ON needs I / 128 <= %d at block_m %d",
                    moe::fused_max_njb(block_m), block_m);
    return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_fp8_experts_schedule(int64_t M, int64_t K, int64_t I, int32_t E,
                                            int32_t top_k, int32_t block_m, int64_t sorted_cap,
                                            uint32_t flags, int32_t *info) {
    moe_status st = check_experts_shape(M, K, I, E, top_k, block_m, sorted_cap);
    if (st != MOE_OK) return st;
    if (!info) return fail(MOE_ERR_NULL, "output pointer is NULL");
    st = check_flags(flags, K, I, block_m, M * top_k);
    if (st != MOE_OK) return st;
    const WsLayout l = ws_layout(M, K, I, E, top_k, block_m, sorted_cap, flags);
    info[0] = l.sp.gu_cols ? 2 : (l.sp.gu_persistent ? 1 : 0);
    info[1] = l.sp.dn_cols ? 2 : (l.sp.dn_persistent ? 1 : 0);
    info[2] = l.sp.nsplit;
    info[3] = l.sp.kb_per_split;
    info[4] = l.sp.fused ? 1 : 0;
    return MOE_OK;
}

namespace {

// Validation shared by the expert-stage entry points.
moe_status check_stage(int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k, int32_t block_m,
                       int64_t sorted_cap, uint32_t flags, const void *workspace,
                       size_t workspace_bytes, WsLayout *l) {
    moe_status st = check_experts_shape(M, K, I, E, top_k, block_m, sorted_cap);
    if (st != MOE_OK) return st;
    st = check_flags(flags, K, I, block_m, M * top_k);
    if (st != MOE_OK) return st;
    *l = ws_layout(M, K, I, E, top_k, block_m, sorted_cap, flags);
    if (M == 0 || sorted_cap == 0) return MOE_OK;
    if (!workspace) return fail(MOE_ERR_NULL, "workspace is required");
    if (((uintptr_t)workspace & 255u) != 0) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < l->total)
        return fail(MOE_ERR_CAPACITY, "workspace %zu bytes < required %zu", workspace_bytes, l->total);
    return MOE_OK;
}

}  // namespace

namespace {

moe::GateUpArgs gateup_args(const uint8_t *x_q, const float *x_s, const uint8_t *w13,
                            const float *w13_s, const int32_t *sorted_token_ids,
                            const int32_t *expert_ids, const int32_t *num_tokens_post_padded,
                            int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                            int32_t block_m, int64_t sorted_cap, uint32_t flags, uint8_t *ws,
                            const WsLayout &l) {
    moe::GateUpArgs ga;
    ga.xq = x_q;
    ga.xs = x_s;
    ga.w13 = w13;
    ga.w13s = w13_s;
    ga.w13e = nullptr;
    ga.sorted = sorted_token_ids;
    ga.eids = expert_ids;
    ga.ntp = num_tokens_post_padded;
    ga.hq = ws + l.hq;
    ga.hs = (float *)(ws + l.hs);
    ga.part = (float *)(ws + l.part);
    ga.cnt = (uint32_t *)(ws + l.cnt);
    ga.n_cnt = (int64_t)l.cnt_words;
    ga.rpos = (int32_t *)(ws + l.rpos);
    ga.tiles = (int4 *)(ws + l.tiles);
    ga.tmeta = (int32_t *)(ws + l.tiles + (size_t)(sorted_cap / block_m) * 16);
    ga.K = K;
    ga.I = I;
    ga.R = M * top_k;
    ga.E = E;
    ga.top_k = top_k;
    ga.nkb = (int)(K / 128);
    ga.jtiles = (int)(I / 128);
    ga.nblocks = (int)(sorted_cap / block_m);
    ga.nsplit = l.sp.nsplit;
    ga.kb_per_split = l.sp.kb_per_split;
    ga.inter_ue8m0 = (flags & MOE_F_INTER_UE8M0) ? 1 : 0;
    ga.w13_packed = (flags & MOE_F_W13_PACKED) ? 1 : 0;
    ga.h32 = l.sp.gu_cols ? (float *)(ws + l.h32) : nullptr;
    return ga;
}

moe::DownArgs down_args(const uint8_t *w2, const float *w2_s, const float *topk_weights,
                        const int32_t *sorted_token_ids, const int32_t *expert_ids,
                        const int32_t *num_tokens_post_padded, int64_t M, int64_t K, int64_t I,
                        int32_t E, int32_t top_k, int32_t block_m, int64_t sorted_cap, uint8_t *ws,
                        const WsLayout &l) {
    moe::DownArgs da;
    da.hq = ws + l.hq;
    da.hs = (const float *)(ws + l.hs);
    da.w2 = w2;
    da.w2s = w2_s;
    da.w2e = nullptr;
    da.topk_w = topk_weights;
    da.sorted = sorted_token_ids;
    da.eids = expert_ids;
    da.ntp = num_tokens_post_padded;
    da.y16 = (uint16_t *)(ws + l.y);
    da.ys = (float *)(ws + l.ys);
    da.K = K;
    da.I = I;
    da.R = M * top_k;
    da.E = E;
    da.top_k = top_k;
    da.njb = (int)(I / 128);
    da.ctiles = (int)((K + 255) / 256);
    da.nblocks = (int)(sorted_cap / block_m);
    da.tiles = (const int4 *)(ws + l.tiles);
    da.tmeta = (int32_t *)(ws + l.tiles + (size_t)(sorted_cap / block_m) * 16);
    return da;
}

}  // namespace

namespace {

// prep_done: the route map and the split-K counters were cleared by the
// plan's launch (moe_fp8_layer)
moe_status gate_up_stage(const uint8_t *x_q, const float *x_s, const uint8_t *w13,
                         const float *w13_s, const int32_t *sorted_token_ids,
                         const int32_t *expert_ids, const int32_t *num_tokens_post_padded,
                         int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                         int32_t block_m, int64_t sorted_cap, uint32_t flags,
                         void *workspace, size_t workspace_bytes, void *stream, bool prep_done) {
    WsLayout l;
    moe_status st = check_stage(M, K, I, E, top_k, block_m, sorted_cap, flags, workspace,
                                workspace_bytes, &l);
    if (st != MOE_OK || M == 0 || sorted_cap == 0) return st;
    if (!x_q || !x_s || !w13 || !w13_s || !sorted_token_ids || !expert_ids || !num_tokens_post_padded)
        return fail(MOE_ERR_NULL, "x_q, x_s, w13, w13_s and the plan are required");
    if (!aligned16(x_q) || !aligned16(w13))
        return fail(MOE_ERR_ALIGN, "x_q and w13 must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    uint8_t *ws = (uint8_t *)workspace;
    if (l.sp.gu_cols) {                        // no route map, no counters
        const moe::GateUpArgs ga = gateup_args(x_q, x_s, w13, w13_s, sorted_token_ids, expert_ids,
                                               num_tokens_post_padded, M, K, I, E, top_k, block_m,
                                               sorted_cap, flags, ws, l);
        return hip_check(moe::launch_gateup_slices(ga, block_m, l.sp.gu_slice, s), "moe_fp8_gate_up: launch");
    }
    // the route map and the split-K counters are cleared by the row-tile
    // launch when a persistent kernel runs, else by a launch of their own
    if (!l.sp.gu_persistent && !l.sp.dn_persistent && !prep_done) {
        st = hip_check(moe::launch_prep((uint32_t *)(ws + l.rpos), (size_t)M * top_k,
                                        (uint32_t *)(ws + l.cnt), l.cnt_words, s),
                       "moe_fp8_gate_up: clear route map and counters");
        if (st != MOE_OK) return st;
    }
    const moe::GateUpArgs ga = gateup_args(x_q, x_s, w13, w13_s, sorted_token_ids, expert_ids,
                                           num_tokens_post_padded, M, K, I, E, top_k, block_m,
                                           sorted_cap, flags, ws, l);
    const bool fp8 = (flags & MOE_F_FP8_GATEUP) != 0, e8 = (flags & MOE_F_MMA_E8M0) != 0;
    if (l.sp.gu_persistent)
        return hip_check(moe::launch_gateup_pipe(ga, block_m, fp8, e8, s), "moe_fp8_gate_up: launch");
    if (l.sp.dn_persistent) {                  // the down stage's row tiles
        st = hip_check(moe::launch_tiles(ga, block_m, l.sp.dn_small ? 32 : 128, s),
                       "moe_fp8_gate_up: row tiles");
        if (st != MOE_OK) return st;
    }
    return hip_check(moe::launch_gateup(ga, block_m, fp8, e8, s), "moe_fp8_gate_up: launch");
}

}  // namespace

MOE_API moe_status moe_fp8_gate_up(const uint8_t *x_q, const float *x_s, const uint8_t *w13,
                                   const float *w13_s, const int32_t *sorted_token_ids,
                                   const int32_t *expert_ids, const int32_t *num_tokens_post_padded,
                                   int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                                   int32_t block_m, int64_t sorted_cap, uint32_t flags,
                                   void *workspace, size_t workspace_bytes, void *stream) {
    return gate_up_stage(x_q, x_s, w13, w13_s, sorted_token_ids, expert_ids, num_tokens_post_padded,
                         M, K, I, E, top_k, block_m, sorted_cap, flags, workspace, workspace_bytes,
                         stream, false);
}

MOE_API moe_status moe_fp8_down_reduce(const uint8_t *w2, const float *w2_s,
                                       const float *topk_weights, const int32_t *sorted_token_ids,
                                       const int32_t *expert_ids,
                                       const int32_t *num_tokens_post_padded, int64_t M, int64_t K,
                                       int64_t I, int32_t E, int32_t top_k, int32_t block_m,
                                       int64_t sorted_cap, uint32_t flags, void *out_bf16,
                                       void *workspace, size_t workspace_bytes, void *stream) {
    WsLayout l;
    moe_status st = check_stage(M, K, I, E, top_k, block_m, sorted_cap, flags, workspace,
                                workspace_bytes, &l);
    if (st != MOE_OK || M == 0 || sorted_cap == 0) return st;
    if (!w2 || !w2_s || !topk_weights || !sorted_token_ids || !expert_ids ||
        !num_tokens_post_padded || !out_bf16)
        return fail(MOE_ERR_NULL, "w2, w2_s, topk_weights, the plan and out are required");
    if (!aligned16(w2) || !aligned16(out_bf16))
        return fail(MOE_ERR_ALIGN, "w2 and out must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    uint8_t *ws = (uint8_t *)workspace;
    const moe::DownArgs da = down_args(w2, w2_s, topk_weights, sorted_token_ids, expert_ids,
                                       num_tokens_post_padded, M, K, I, E, top_k, block_m,
                                       sorted_cap, ws, l);
    const bool e8 = (flags & MOE_F_MMA_E8M0) != 0;
    if (l.sp.dn_cols) {                        // the route sum is part of this launch
        moe::ColsRequant rq;
        rq.h32 = l.sp.gu_cols ? (const float *)(ws + l.h32) : nullptr;
        rq.hq = ws + l.hq;
        rq.hs = (float *)(ws + l.hs);
        rq.ue8m0 = (flags & MOE_F_INTER_UE8M0) ? 1 : 0;
        return hip_check(moe::launch_down_cols(da, block_m, e8, (const int32_t *)(ws + l.rpos), rq,
                                               (uint16_t *)out_bf16, s),
                         "moe_fp8_down_reduce: down launch");
    }
    st = hip_check(l.sp.dn_persistent ? moe::launch_down_pipe(da, block_m, e8, l.sp.dn_small, s)
                                                   : moe::launch_down(da, block_m, e8, s),
                   "moe_fp8_down_reduce: down launch");
    if (st != MOE_OK) return st;
    return hip_check(moe::launch_finalize((uint16_t *)out_bf16, (const uint16_t *)(ws + l.y),
                                          (const float *)(ws + l.ys), topk_weights,
                                          (const int32_t *)(ws + l.rpos), M, K, top_k, s),
                     "moe_fp8_down_reduce: finalize launch");
}

MOE_API moe_status moe_fp8_experts(const uint8_t *x_q, const float *x_s, const uint8_t *w13,
                                   const float *w13_s, const uint8_t *w2, const float *w2_s,
                                   const float *topk_weights, const int32_t *sorted_token_ids,
                                   const int32_t *expert_ids, const int32_t *num_tokens_post_padded,
                                   int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                                   int32_t block_m, int64_t sorted_cap, uint32_t flags,
                                   void *out_bf16, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    // validate everything before enqueuing anything
    WsLayout l;
    moe_status st = check_stage(M, K, I, E, top_k, block_m, sorted_cap, flags, workspace,
                                workspace_bytes, &l);
    if (st != MOE_OK || M == 0 || sorted_cap == 0) return st;
    if (!x_q || !x_s || !w13 || !w13_s || !w2 || !w2_s || !topk_weights || !sorted_token_ids ||
        !expert_ids || !num_tokens_post_padded || !out_bf16)
        return fail(MOE_ERR_NULL, "all tensor arguments and the workspace are required");
    if (!aligned16(x_q) || !aligned16(w13) || !aligned16(w2) || !aligned16(out_bf16))
        return fail(MOE_ERR_ALIGN, "x_q, w13, w2 and out must be 16-byte aligned");
    if (l.sp.fused) {
        hipStream_t s = (hipStream_t)stream;
        uint8_t *ws = (uint8_t *)workspace;
        const moe::GateUpArgs ga = gateup_args(x_q, x_s, w13, w13_s, sorted_token_ids, expert_ids,
                                               num_tokens_post_padded, M, K, I, E, top_k, block_m,
                                               sorted_cap, flags, ws, l);
        const moe::DownArgs da = down_args(w2, w2_s, topk_weights, sorted_token_ids, expert_ids,
                                           num_tokens_post_padded, M, K, I, E, top_k, block_m,
                                           sorted_cap, ws, l);
        uint32_t *c = (uint32_t *)(ws + l.cnt) + l.splitk_words;
        const int64_t npass = block_m > 64 ? block_m / 64 : 1;
        moe::FusedArgs f;
        f.tickets = c;
        f.err = c + moe::kFusedQueues;
        f.cnt_h = c + moe::kFusedQueues + 4;
        f.cnt_t = f.cnt_h + (sorted_cap / block_m) * npass;
        f.out = (uint16_t *)out_bf16;
        f.rpos = (const int32_t *)(ws + l.rpos);
        f.M = M;
        f.per_queue = f.lds_ticket = 0;
        st = hip_check(moe::launch_fused_prep((uint32_t *)(ws + l.cnt), l.cnt_words,
                                              (int32_t *)(ws + l.rpos), M * top_k, sorted_token_ids,
                                              num_tokens_post_padded, sorted_cap, s),
                       "moe_fp8_experts: single-launch set-up");
        if (st != MOE_OK) return st;
        const bool fp8 = (flags & MOE_F_FP8_GATEUP) != 0, e8 = (flags & MOE_F_MMA_E8M0) != 0;
        return hip_check(moe::launch_fused(ga, da, f, block_m, fp8, e8, s),
                         "moe_fp8_experts: single-launch kernel");
    }
    st = moe_fp8_gate_up(x_q, x_s, w13, w13_s, sorted_token_ids, expert_ids, num_tokens_post_padded,
                         M, K, I, E, top_k, block_m, sorted_cap, flags, workspace, workspace_bytes,
                         stream);
    if (st != MOE_OK) return st;
    return moe_fp8_down_reduce(w2, w2_s, topk_weights, sorted_token_ids, expert_ids,
                               num_tokens_post_padded, M, K, I, E, top_k, block_m, sorted_cap,
                               flags, out_bf16, workspace, workspace_bytes, stream);
}

MOE_API moe_status moe_fp8_layer(const void *x_bf16, int64_t ld_x, int32_t scale_mode,
                                 const void *topk_ids, int32_t ids_dtype, const float *topk_weights,
                                 const uint8_t *w13, const float *w13_s, const uint8_t *w2,
                                 const float *w2_s, int64_t M, int64_t K, int64_t I, int32_t E,
                                 int32_t top_k, int32_t block_m, int32_t *sorted_token_ids,
                                 int64_t sorted_cap, int32_t *expert_ids, int64_t blocks_cap,
                                 int32_t *num_tokens_post_padded, uint8_t *x_q, float *x_s,
                                 void *plan_workspace, size_t plan_workspace_bytes, uint32_t flags,
                                 void *out_bf16, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    // validate both halves before enqueuing anything
    int groups = 0;
    moe_status st = check_plan(topk_ids, ids_dtype, M, top_k, E, block_m, sorted_token_ids, sorted_cap,
                               expert_ids, blocks_cap, num_tokens_post_padded, plan_workspace,
                               plan_workspace_bytes, &groups);
    if (st != MOE_OK) return st;
    st = check_quant(x_bf16, M, K, ld_x, x_q, x_s, scale_mode);
    if (st != MOE_OK) return st;
    WsLayout l;
    st = check_stage(M, K, I, E, top_k, block_m, sorted_cap, flags, workspace, workspace_bytes, &l);
    if (st != MOE_OK) return st;
    if (M > 0 && sorted_cap > 0) {
        if (!w13 || !w13_s || !w2 || !w2_s || !topk_weights || !out_bf16)
            return fail(MOE_ERR_NULL, "all tensor arguments and the workspace are required");
        if (!aligned16(x_q) || !aligned16(w13) || !aligned16(w2) || !aligned16(out_bf16))
            return fail(MOE_ERR_ALIGN, "x_q, w13, w2 and out must be 16-byte aligned");
    }
    // the clearing launch of the per-block gate/up folds into the plan's
    // one-workgroup launch; every other schedule runs the two calls as they are
    const bool fold = M > 0 && sorted_cap > 0 && groups == 0 && !l.sp.fused && !l.sp.gu_persistent &&
                      !l.sp.dn_persistent && !l.sp.gu_cols;
    if (!fold) {
        st = moe_plan_quant(topk_ids, ids_dtype, M, top_k, E, block_m, sorted_token_ids, sorted_cap,
                            expert_ids, blocks_cap, num_tokens_post_padded, plan_workspace,
                            plan_workspace_bytes, x_bf16, K, ld_x, x_q, x_s, scale_mode, stream);
        if (st != MOE_OK) return st;
        return moe_fp8_experts(x_q, x_s, w13, w13_s, w2, w2_s, topk_weights, sorted_token_ids,
                               expert_ids, num_tokens_post_padded, M, K, I, E, top_k, block_m,
                               sorted_cap, flags, out_bf16, workspace, workspace_bytes, stream);
    }
    uint8_t *ws = (uint8_t *)workspace;
    moe::QuantJob q;
    q.x = (const uint16_t *)x_bf16;
    q.M = M;
    q.K = K;
    q.ld = ld_x;
    q.xq = x_q;
    q.xs = x_s;
    moe::ClearJob c;
    c.rpos = (uint32_t *)(ws + l.rpos);
    c.nr = (size_t)M * top_k;
    c.cnt = (uint32_t *)(ws + l.cnt);
    c.nc = l.cnt_words;
    st = hip_check(moe::launch_plan_quant_clear(topk_ids, ids_dtype == MOE_IDS_I64, M * top_k, E, block_m,
                                                sorted_token_ids, expert_ids, num_tokens_post_padded, q,
                                                scale_mode == MOE_SCALE_UE8M0, c, (hipStream_t)stream),
                   "moe_fp8_layer: plan launch");
    if (st != MOE_OK) return st;
    st = gate_up_stage(x_q, x_s, w13, w13_s, sorted_token_ids, expert_ids, num_tokens_post_padded, M, K,
                       I, E, top_k, block_m, sorted_cap, flags, workspace, workspace_bytes, stream, true);
    if (st != MOE_OK) return st;
    return moe_fp8_down_reduce(w2, w2_s, topk_weights, sorted_token_ids, expert_ids,
                               num_tokens_post_padded, M, K, I, E, top_k, block_m, sorted_cap, flags,
                               out_bf16, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------- weight prepack

MOE_API size_t moe_prepack_w13_size(int64_t E, int64_t I, int64_t K) {
    if (E < 1 || I <= 0 || K <= 0 || I % 128 || K % 128) return 0;
    return (size_t)E * 2 * I * K;
}

MOE_API moe_status moe_prepack_w13(const uint8_t *w13, int64_t E, int64_t I, int64_t K,
                                   uint8_t *w13_packed, void *stream) {
    if (E < 1 || I <= 0 || K <= 0)
        return fail(MOE_ERR_SHAPE, "need E >= 1, I > 0, K > 0");
    if (I % 128 || K % 128)
        return fail(MOE_ERR_SHAPE, "I (%lld) and K (%lld) must be multiples of 128", (long long)I,
                    (long long)K);
    if (!w13 || !w13_packed) return fail(MOE_ERR_NULL, "w13 and w13_packed are required");
    if (!aligned16(w13) || !aligned16(w13_packed))
        return fail(MOE_ERR_ALIGN, "w13 and w13_packed must be 16-byte aligned");
    const uintptr_t a0 = (uintptr_t)w13, b0 = (uintptr_t)w13_packed;
    const uintptr_t n = (uintptr_t)moe_prepack_w13_size(E, I, K);
    if (a0 < b0 + n && b0 < a0 + n) return fail(MOE_ERR_SHAPE, "w13 and w13_packed overlap");
    return hip_check(moe::launch_prepack_w13(w13, E, I, K, w13_packed, (hipStream_t)stream),
                     "moe_prepack_w13: launch");
}

// ------------------------------------------------------- W4A8 variant

namespace {

// The W4A8 variant schedules like moe_fp8_experts (two stages, each on the
// per-block or the persistent kernel family).
uint32_t w4_flags(uint32_t flags) { return flags; }

moe_status check_w4(int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k, int32_t block_m,
                    int64_t sorted_cap, uint32_t flags) {
    moe_status st = check_experts_shape(M, K, I, E, top_k, block_m, sorted_cap);
    if (st != MOE_OK) return st;
    if (flags & (MOE_F_MMA_E8M0 | MOE_F_FP8_GATEUP | MOE_F_W13_PACKED))
        return fail(MOE_ERR_UNSUPPORTED,
                    "W4A8: MOE_F_MMA_E8M0, MOE_F_FP8_GATEUP and MOE_F_W13_PACKED do not apply");
    if (((flags & MOE_F_FUSE_MASK) >> MOE_F_FUSE_SHIFT) == MOE_FUSE_ON)
        return fail(MOE_ERR_UNSUPPORTED, "W4A8 runs as two stages (no MOE_FUSE_ON)");
    if (((flags & MOE_F_GATEUP_PATH_MASK) >> MOE_F_GATEUP_PATH_SHIFT) == MOE_PATH_COLUMNS)
        return fail(MOE_ERR_UNSUPPORTED, "W4A8: the column-slice gate/up takes FP8 weights only");
    st = check_flags(w4_flags(flags), K, I, block_m, M * top_k);
    if (st != MOE_OK) return st;
    // the per-block down kernel keeps a block's intermediate rows in LDS
    const WsLayout l = ws_layout(M, K, I, E, top_k, block_m, sorted_cap, w4_flags(flags), true);
    if (!l.sp.dn_persistent && !l.sp.dn_cols && I / 128 > moe::down_w4_max_njb(block_m))
        return fail(MOE_ERR_UNSUPPORTED,
                    "W4A8 on the per-block down kernel needs I / 128 <= %d at block_m %d",
                    moe::down_w4_max_njb(block_m), block_m);
    return MOE_OK;
}

}  // namespace

MOE_API size_t moe_w4a8_experts_workspace_size(int64_t M, int64_t K, int64_t I, int32_t E,
                                               int32_t top_k, int32_t block_m, int64_t sorted_cap,
                                               uint32_t flags) {
    if (check_w4(M, K, I, E, top_k, block_m, sorted_cap, flags) != MOE_OK) return 0;
    return ws_layout(M, K, I, E, top_k, block_m, sorted_cap, w4_flags(flags), true).total;
}

MOE_API moe_status moe_w4a8_experts(const uint8_t *x_q, const float *x_s, const uint8_t *w13,
                                    const uint8_t *w13_e, const uint8_t *w2, const uint8_t *w2_e,
                                    const float *topk_weights, const int32_t *sorted_token_ids,
                                    const int32_t *expert_ids,
                                    const int32_t *num_tokens_post_padded, int64_t M, int64_t K,
                                    int64_t I, int32_t E, int32_t top_k, int32_t block_m,
                                    int64_t sorted_cap, uint32_t flags, void *out_bf16,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    moe_status st = check_w4(M, K, I, E, top_k, block_m, sorted_cap, flags);
    if (st != MOE_OK) return st;
    const uint32_t fl = w4_flags(flags);
    const WsLayout l = ws_layout(M, K, I, E, top_k, block_m, sorted_cap, fl, true);
    if (M == 0 || sorted_cap == 0) return MOE_OK;
    if (!workspace) return fail(MOE_ERR_NULL, "workspace is required");
    if (((uintptr_t)workspace & 255u) != 0) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < l.total)
        return fail(MOE_ERR_CAPACITY, "workspace %zu bytes < required %zu", workspace_bytes, l.total);
    if (!x_q || !x_s || !w13 || !w13_e || !w2 || !w2_e || !topk_weights || !sorted_token_ids ||
        !expert_ids || !num_tokens_post_padded || !out_bf16)
        return fail(MOE_ERR_NULL, "all tensor arguments and the workspace are required");
    if (!aligned16(x_q) || !aligned16(w13) || !aligned16(w2) || !aligned16(out_bf16))
        return fail(MOE_ERR_ALIGN, "x_q, w13, w2 and out must be 16-byte aligned");
    if (((uintptr_t)w13_e & 3u) || ((uintptr_t)w2_e & 3u))
        return fail(MOE_ERR_ALIGN, "w13_e and w2_e must be 4-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    uint8_t *ws = (uint8_t *)workspace;
    moe::GateUpArgs ga = gateup_args(x_q, x_s, w13, nullptr, sorted_token_ids, expert_ids,
                                     num_tokens_post_padded, M, K, I, E, top_k, block_m, sorted_cap,
                                     fl, ws, l);
    ga.w13e = w13_e;
    // the row-tile launch (persistent gate/up, or alone for a persistent
    // down stage) also clears the route map and the counters
    if (l.sp.gu_persistent) {
        st = hip_check(moe::launch_gateup_pipe_w4(ga, block_m, s), "moe_w4a8_experts: gate/up launch");
    } else {
        st = l.sp.dn_persistent
                 ? hip_check(moe::launch_tiles(ga, block_m, l.sp.dn_small ? 32 : 128, s),
                             "moe_w4a8_experts: row tiles")
                 : hip_check(moe::launch_prep((uint32_t *)(ws + l.rpos), (size_t)M * top_k,
                                              (uint32_t *)(ws + l.cnt), l.cnt_words, s),
                             "moe_w4a8_experts: clear route map and counters");
        if (st != MOE_OK) return st;
        st = hip_check(moe::launch_gateup_w4(ga, block_m, s), "moe_w4a8_experts: gate/up launch");
    }
    if (st != MOE_OK) return st;
    moe::DownArgs da = down_args(w2, nullptr, topk_weights, sorted_token_ids, expert_ids,
                                 num_tokens_post_padded, M, K, I, E, top_k, block_m, sorted_cap, ws, l);
    da.w2e = w2_e;
    if (l.sp.dn_cols) {                        // the route sum is part of this launch
        moe::ColsRequant rq;
        rq.h32 = nullptr;
        rq.hq = nullptr;
        rq.hs = nullptr;
        rq.ue8m0 = 0;
        return hip_check(moe::launch_down_cols(da, block_m, false, (const int32_t *)(ws + l.rpos), rq,
                                               (uint16_t *)out_bf16, s),
                         "moe_w4a8_experts: down launch");
    }
    st = hip_check(l.sp.dn_persistent ? moe::launch_down_pipe_w4(da, block_m, l.sp.dn_small, s)
                                      : moe::launch_down_w4(da, block_m, s),
                   "moe_w4a8_experts: down launch");
    if (st != MOE_OK) return st;
    return hip_check(moe::launch_finalize((uint16_t *)out_bf16, (const uint16_t *)(ws + l.y),
                                          (const float *)(ws + l.ys), topk_weights,
                                          (const int32_t *)(ws + l.rpos), M, K, top_k, s),
                     "moe_w4a8_experts: finalize launch");
}

// ------------------------------------------------- no-allocation variant

// The static workspace of moe_fp8_experts_noalloc: one copy per device,
// allocated with the code object.  Host code never passes `scratch` itself
// (on the host it is only a stand-in symbol): it takes the device address
// that hipGetSymbolAddress reports for the current device, looked up once per
// device and kept in g_scratch.
static __device__ __attribute__((aligned(256))) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<uintptr_t> g_scratch[64];   // device address of `scratch`, per device (0: not yet)

moe_status scratch_of_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_check(e, "moe_fp8_experts_noalloc: hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the 64 supported", dev);
    uintptr_t p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == 0) {
        void *q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_check(e, "moe_fp8_experts_noalloc: hipGetSymbolAddress");
        if (q == nullptr || ((uintptr_t)q & 255u) != 0)
            return fail(MOE_ERR_HIP, "moe_fp8_experts_noalloc: scratch address %p unusable", q);
        p = (uintptr_t)q;
        g_scratch[dev].store(p, std::memory_order_release);   // a racing lookup stores the same
    }
    *out = (void *)p;
    return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_fp8_experts_noalloc(const uint8_t *x_q, const float *x_s, const uint8_t *w13,
                                           const float *w13_s, const uint8_t *w2, const float *w2_s,
                                           const float *topk_weights,
                                           const int32_t *sorted_token_ids,
                                           const int32_t *expert_ids,
                                           const int32_t *num_tokens_post_padded, int64_t M,
                                           int64_t K, int64_t I, int32_t E, int32_t top_k,
                                           int32_t block_m, int64_t sorted_cap, uint32_t flags,
                                           void *out_bf16, void *stream) {
    moe_status st = check_experts_shape(M, K, I, E, top_k, block_m, sorted_cap);
    if (st != MOE_OK) return st;
    st = check_flags(flags, K, I, block_m, M * top_k);
    if (st != MOE_OK) return st;
    const size_t need = ws_layout(M, K, I, E, top_k, block_m, sorted_cap, flags).total;
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_CAPACITY,
                    "moe_fp8_experts_noalloc: these sizes need %zu bytes of workspace, above the "
                    "%zu-byte static scratch; use moe_fp8_experts with a caller workspace",
                    need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    if (M == 0 || sorted_cap == 0) return MOE_OK;
    void *ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != MOE_OK) return st;
    return moe_fp8_experts(x_q, x_s, w13, w13_s, w2, w2_s, topk_weights, sorted_token_ids, expert_ids,
                           num_tokens_post_padded, M, K, I, E, top_k, block_m, sorted_cap, flags,
                           out_bf16, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}
