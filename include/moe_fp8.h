/*
 * moe_fp8.h -- C ABI of libmoe_fp8.so: the routed FP8 W8A8 block-scale
 * mixture-of-experts expert path for AMD Instinct MI355X (gfx950).
 *
 * The path, as the method's pages define it:
 *   1. moe_plan        -- the moe_align_block_size routing plan
 *                         (FlashInfer PR #4287, PR summary; host bound on the
 *                         plan buffers in its review and public-contract
 *                         section; masked int32/int64 routes from
 *                         sglang-glm53-flash-sm120 PR #13, description and
 *                         validation).
 *   2. moe_quant_act   -- 1x128 FP8 (E4M3) activation quantisation with one
 *                         FP32 scale per token and 128-column group
 *                         (PR #4287, public-contract section).
 *   3-5. moe_fp8_experts -- gate/up grouped GEMM with FP32 128x128 weight
 *                         block scales applied per K-block, SwiGLU, FP8
 *                         requantisation of the SwiGLU output per row and
 *                         128-column group, down GEMM, weighting by the
 *                         router probability and reduce-add into the
 *                         caller's BF16 output (PR #4287, PR summary and
 *                         public-contract section; power-of-two scales from
 *                         SGLang PR #43556, motivation and modifications).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument, unless said otherwise, is DEVICE memory owned
 *     by the caller.  The library allocates nothing and frees nothing.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work; buffers must stay alive until the stream has
 *     executed it.  No call synchronises the host or copies device data to
 *     the host.
 *   - Host-checkable problems (NULL pointers, shapes, alignment, capacity,
 *     workspace size) return a status and enqueue nothing.  Launch failures
 *     return MOE_ERR_HIP and moe_last_hip_error() holds the HIP message.
 *   - Host-side state: none that affects results.  Each launcher raises its
 *     kernel's dynamic-LDS limit once per device and the device's CU count
 *     is queried once; both are kept in atomics, so concurrent first calls
 *     from several host threads are safe.
 *   - Data conditions are not errors: ids outside [0, E) are masked routes;
 *     zero scales contribute zero.
 *   - All tensors are dense row-major with the shapes given; sizes are in
 *     elements unless named *_bytes.
 *
 * Notation: M tokens, K hidden size, I intermediate size (W13 has 2I rows:
 * rows [0, I) are the gate projection, rows [I, 2I) the up projection),
 * E experts, top_k routes per token, R = M * top_k routes, flat route index
 * r = t * top_k + j.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                    */
    MOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent        */
    MOE_ERR_ALIGN = 3,       /* a pointer or leading dimension is misaligned  */
    MOE_ERR_CAPACITY = 4,    /* plan buffers or workspace too small           */
    MOE_ERR_UNSUPPORTED = 5, /* valid request the library does not implement  */
    MOE_ERR_HIP = 6          /* a HIP runtime call failed                     */
} moe_status;

enum { MOE_IDS_I32 = 0, MOE_IDS_I64 = 1 };

/* Group scale rules of the quantisers.
 *   MOE_SCALE_FP32 : s = max(amax / 448, FLT_MIN) (IEEE FP32 division),
 *                    code = E4M3_RNE_SAT(v * (1 / s)).
 *   MOE_SCALE_UE8M0: s = 2^e with e the least integer such that
 *                    448 * 2^e >= amax, floored at -126; code = E4M3(v * 2^-e).
 * The FLT_MIN floor keeps an all-zero group at code 0 instead of 0 * inf
 * (PR #4287, review of the zero-activation scale and public contract). */
enum { MOE_SCALE_FP32 = 0, MOE_SCALE_UE8M0 = 1 };

/* moe_fp8_experts flags. */
enum {
    /* requantise the SwiGLU output with MOE_SCALE_UE8M0 scales */
    MOE_F_INTER_UE8M0 = 1u,
    /* apply the block scales as powers of two inside the multiply instead
     * of FP32 multiplies per K-block (SGLang PR #43556, motivation): in the
     * down GEMM as E8M0 scale operands of the FP8 MFMA; in the exact gate/up
     * GEMM folded into the FP16 widening (codes times their scale's ratio to
     * the largest over K, exact) with the sums accumulated across K-blocks
     * in the MFMA and scaled once at the end; with MOE_F_FP8_GATEUP as E8M0
     * operands of the FP8 MFMA.  Requires MOE_F_INTER_UE8M0, and the caller
     * guarantees that x_s, w13_s and w2_s hold only powers of two in
     * [2^-126, 2^126] (no zeros): a non-power-of-two scale is silently
     * truncated to its exponent (moe_debug_count_non_pow2 checks). */
    MOE_F_MMA_E8M0 = 2u,
    /* EXPERIMENTAL, outside the parity contract: run the gate/up GEMM on
     * the FP8 MFMA (v_mfma_f32_16x16x128_f8f6f4) instead of the default
     * exact path (codes widened to FP16, exact products, FP32 accumulation).
     * Faster, but the FP8 MFMA keeps only ~15 bits below the largest product
     * of each instruction, so about 1e-3 of the requantised SwiGLU codes
     * move (some by more than one step) relative to an exactly accumulated
     * reference -- ten times the 1e-4 intermediate-code budget the default
     * path meets.  The output stays within the output tolerance on the
     * tested workloads, but no bar is promised. */
    MOE_F_FP8_GATEUP = 4u
};
/* Bits 8..15 of `flags` optionally force the gate/up split-K factor
 * (0 = automatic).  A tuning and test override; the same value must be
 * given to moe_fp8_experts_workspace_size. */
#define MOE_F_SPLITK_SHIFT 8
#define MOE_F_SPLITK_MASK  0xFF00u
/* Bits 16..17 and 18..19 optionally force the kernel family of the gate/up
 * and of the down stage: MOE_PATH_AUTO (0), MOE_PATH_STREAM (1: per plan
 * block, the weights streamed once per block), MOE_PATH_PERSISTENT (2:
 * persistent workgroups over row tiles of one expert; needs K, I <= 32768
 * and, for the gate/up, no forced split-K) or MOE_PATH_COLUMNS (3; needs
 * I = 256, block_m 8 or 16 and M * top_k <= 192, else MOE_ERR_UNSUPPORTED).
 * For the down stage, MOE_PATH_COLUMNS is one workgroup per 32 output
 * columns over every plan block, the route sum in the same launch.  For the
 * gate/up it is one workgroup per (plan block, 16 intermediate columns)
 * with K split inside the workgroup: it writes FP32
 * SwiGLU rows that the column-split down requantises as it reads them, so
 * it needs that down stage (down path AUTO or COLUMNS), exact products (no
 * MOE_F_FP8_GATEUP), unpacked W13 and no forced split-K, else
 * MOE_ERR_SHAPE; on that path h_q / h_s are written by moe_fp8_down_reduce.
 * The W4A8 entry point takes the column-split down (E2M1 weights) but not
 * the column-slice gate/up.
 * A tuning and test override; the same value must be given to
 * moe_fp8_experts_workspace_size.  Other values: MOE_ERR_SHAPE. */
#define MOE_F_GATEUP_PATH_SHIFT 16
#define MOE_F_GATEUP_PATH_MASK  0x30000u
#define MOE_F_DOWN_PATH_SHIFT   18
#define MOE_F_DOWN_PATH_MASK    0xC0000u
enum { MOE_PATH_AUTO = 0, MOE_PATH_STREAM = 1, MOE_PATH_PERSISTENT = 2, MOE_PATH_COLUMNS = 3 };
/* Bits 20..21 choose how moe_fp8_experts launches steps 3-5:
 *   MOE_FUSE_AUTO (0) the library's choice: currently always two stages
 *                     (the single launch measured slower on MI355X at every
 *                     size tried);
 *   MOE_FUSE_OFF  (1) the gate/up and the down stage as separate launches,
 *                     exactly moe_fp8_gate_up then moe_fp8_down_reduce;
 *   MOE_FUSE_ON   (2) one launch for gate/up, SwiGLU + requantisation, down
 *                     and the route sum (after a small set-up fill), as in
 *                     PR #4287's single fused expert kernel (PR summary);
 *                     needs the per-block family for both stages and
 *                     I / 128 <= 512 / min(block_m, 64), else
 *                     MOE_ERR_UNSUPPORTED.
 * The single launch computes what the two stages compute, item for item:
 * the output is bit-identical.  The stage calls always run separately. */
#define MOE_F_FUSE_SHIFT 20
#define MOE_F_FUSE_MASK  0x300000u
enum { MOE_FUSE_AUTO = 0, MOE_FUSE_OFF = 1, MOE_FUSE_ON = 2 };
/* Bit 22: w13 holds the packed layout written by moe_prepack_w13 (the same
 * bytes, reordered); w13_s keeps its layout.  Every gate/up kernel family
 * reads it.  Not accepted by moe_w4a8_experts (MOE_ERR_UNSUPPORTED). */
#define MOE_F_W13_PACKED 0x400000u

/* ---------------------------------------------------------------- plan -- */

/* Worst-case plan sizes for any routing:
 *   sorted_cap = roundup(R + min(E, R) * (block_m - 1), block_m),
 *   blocks_cap = sorted_cap / block_m.
 * M >= 0, 1 <= top_k, 1 <= E <= 1024, 1 <= block_m <= 256. */
moe_status moe_plan_capacity(int64_t M, int32_t top_k, int32_t E, int32_t block_m,
                             int64_t *sorted_cap, int64_t *blocks_cap);

/* Device workspace for the fast moe_plan build (bytes, 4-byte aligned; 0
 * for small route counts).  moe_plan also accepts a NULL or smaller
 * workspace and then builds the same plan with one workgroup. */
size_t moe_plan_workspace_size(int64_t M, int32_t top_k, int32_t E, int32_t block_m);

/* Build the routing plan on the device.
 *   topk_ids      [M, top_k] int32 (ids_dtype = MOE_IDS_I32) or int64
 *                 (MOE_IDS_I64); ids outside [0, E) are masked routes.
 *   sorted_token_ids [sorted_cap] int32 out: routes grouped by expert in
 *                 ascending expert id, ascending r inside an expert, each
 *                 expert's segment padded with the sentinel R to a multiple
 *                 of block_m.
 *   expert_ids    [blocks_cap] int32 out: the expert of each block.
 *   num_tokens_post_padded [1] int32 out: P, the padded length.
 *   Entries at or beyond P (resp. P / block_m) are left untouched.
 * Errors: MOE_ERR_CAPACITY if sorted_cap or blocks_cap is below
 * moe_plan_capacity, or sorted_cap < blocks_cap * block_m. */
moe_status moe_plan(const void *topk_ids, int32_t ids_dtype, int64_t M, int32_t top_k,
                    int32_t E, int32_t block_m,
                    int32_t *sorted_token_ids, int64_t sorted_cap,
                    int32_t *expert_ids, int64_t blocks_cap,
                    int32_t *num_tokens_post_padded,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Router and plan in one call, in the plan's own launches (none added):
 * softmax top-k over each token's routed-expert logits, the chosen weights
 * renormalised and multiplied by routed_scaling, optionally one shared
 * expert, then the plan of moe_plan over those routes -- the fused router
 * that PR #4287's real-model evaluation runs in front of its expert kernel
 * (routed scaling 1.0 without a shared expert in one geometry, 2.5 with one
 * shared expert in the E=257 geometry, its retained-measurement notes).
 *   router_logits [M, E_routed] FP32 (finite), 4-byte aligned.
 *   Chosen experts: the top_k largest logits (equal logits: the lower expert
 *   index), listed largest first; weight of a chosen expert
 *   exp(l_i - l_max) / sum over the chosen, times routed_scaling (softmax
 *   over all experts, top-k, renormalised: the full denominator cancels).
 *   n_shared = 1 appends expert E_routed as route slot top_k with weight 1.
 *   topk_ids [M, top_k + n_shared] int32 out, topk_weights the same FP32 out
 *   (ready for moe_fp8_experts).
 *   The plan is moe_plan's for E = E_routed + n_shared experts and
 *   top_k + n_shared routes per token (its capacity and workspace queries
 *   take those sizes).
 *   x_bf16 != NULL also runs moe_quant_act's quantisation in the same
 *   launch (x_bf16, K, ld_x, x_q, x_s, scale_mode as there); x_bf16 == NULL
 *   skips it (the other five are then ignored).
 * Errors: those of moe_plan (and moe_quant_act); MOE_ERR_SHAPE unless
 * 1 <= top_k <= min(E_routed, 32), n_shared in {0, 1} and
 * E_routed + n_shared <= 1024; MOE_ERR_CAPACITY if the routes need the
 * plan workspace (moe_plan_workspace_size, for 4096 routes and up) and it
 * is missing or too small while they do not fit one workgroup. */
moe_status moe_route_plan(const float *router_logits, int64_t M, int32_t E_routed, int32_t top_k,
                          int32_t n_shared, float routed_scaling, int32_t block_m,
                          int32_t *topk_ids, float *topk_weights,
                          int32_t *sorted_token_ids, int64_t sorted_cap,
                          int32_t *expert_ids, int64_t blocks_cap,
                          int32_t *num_tokens_post_padded,
                          void *workspace, size_t workspace_bytes,
                          const void *x_bf16, int64_t K, int64_t ld_x,
                          uint8_t *x_q, float *x_s, int32_t scale_mode, void *stream);

/* ----------------------------------------------------------- quant act -- */

/* Quantise BF16 activations per token and 128-column group.
 *   x_bf16 [M, ld_x] BF16 (first K columns used); K % 128 == 0,
 *          ld_x >= K, ld_x % 8 == 0, x_bf16 16-byte aligned.
 *   x_q    [M, K] E4M3 codes out (16-byte aligned).
 *   x_s    [M, K/128] FP32 scales out.
 *   scale_mode MOE_SCALE_FP32 or MOE_SCALE_UE8M0. */
moe_status moe_quant_act(const void *x_bf16, int64_t M, int64_t K, int64_t ld_x,
                         uint8_t *x_q, float *x_s, int32_t scale_mode, void *stream);

/* moe_plan and moe_quant_act in one call, with one kernel launch fewer (the
 * quantisation runs inside the plan's first launch).  Arguments, outputs and
 * errors are those of the two calls (validated in full before anything is
 * enqueued); the results are bit-identical to calling them in turn. */
moe_status moe_plan_quant(const void *topk_ids, int32_t ids_dtype, int64_t M, int32_t top_k,
                          int32_t E, int32_t block_m,
                          int32_t *sorted_token_ids, int64_t sorted_cap,
                          int32_t *expert_ids, int64_t blocks_cap,
                          int32_t *num_tokens_post_padded,
                          void *workspace, size_t workspace_bytes,
                          const void *x_bf16, int64_t K, int64_t ld_x,
                          uint8_t *x_q, float *x_s, int32_t scale_mode, void *stream);

/* --------------------------------------------------------------- experts -- */

/* Device workspace moe_fp8_experts needs, in bytes (flags as passed to the
 * call).  Holds the intermediate FP8 rows and their scales, each route's
 * down projection [M * top_k, K] (FP16 with an FP32 scale per 64 columns),
 * the route -> plan-row map and, for small grids, split-K partial sums.  The
 * reduction over a token's routes reads them in route order: results do not
 * depend on scheduling. */
size_t moe_fp8_experts_workspace_size(int64_t M, int64_t K, int64_t I, int32_t E,
                                      int32_t top_k, int32_t block_m, int64_t sorted_cap,
                                      uint32_t flags);

/* Byte offsets inside that workspace of the intermediate codes
 * h_q [sorted_cap, I] (E4M3, indexed by plan row) and their scales
 * h_s [sorted_cap, I/128] (FP32); valid after a call of moe_fp8_experts (or
 * of both stages), for inspection. */
moe_status moe_fp8_experts_workspace_layout(int64_t M, int64_t K, int64_t I, int32_t E,
                                            int32_t top_k, int32_t block_m,
                                            int64_t sorted_cap, uint32_t flags,
                                            size_t *h_q_offset, size_t *h_s_offset);

/* The launch schedule moe_fp8_experts would use for these sizes and flags
 * (host only, nothing enqueued): info[0] = the gate/up stage's kernel (0 per
 * plan block, 1 persistent, 2 split over intermediate-column slices), info[1] = the down stage's kernel (0 per plan block,
 * 1 persistent, 2 split over output columns with the route sum), info[2] = the
 * gate/up split-K factor, info[3] = K-blocks (of 128) per split, info[4] =
 * 1 if steps 3-5 run as the single launch.  info is host memory of 5
 * int32.  Errors: as moe_fp8_experts_workspace_size's
 * shape checks (MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED), MOE_ERR_NULL. */
moe_status moe_fp8_experts_schedule(int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                                    int32_t block_m, int64_t sorted_cap, uint32_t flags,
                                    int32_t *info);

/* Steps 3-5 over a plan built by moe_plan (or any plan of that form):
 *   out[t, :] += sum over valid routes r of token t of
 *                topk_weights[r] * down(requant(SwiGLU(gate_up(x_q[t]))))
 * with FP32 accumulation and one BF16 rounding of out.
 *   x_q [M, K] E4M3, x_s [M, K/128] FP32          (from moe_quant_act)
 *   w13 [E, 2I, K] E4M3, w13_s [E, 2I/128, K/128] FP32
 *   w2  [E, K, I]  E4M3, w2_s  [E, K/128, I/128]  FP32
 *   topk_weights [M, top_k] FP32 (any routed scaling already folded in)
 *   sorted_token_ids [sorted_cap], expert_ids (at least P / block_m
 *   entries: a buffer of moe_plan_capacity's blocks_cap suffices),
 *   num_tokens_post_padded [1]: the plan (device); blocks at or beyond P
 *   exit untouched and their expert ids are never read, so worst-case
 *   buffers are fine.
 *   out_bf16 [M, K] BF16, read and written (accumulated into).
 * Constraints: K % 128 == 0, I % 128 == 0, block_m in {8, 16, 32, 64, 128},
 * sorted_cap % block_m == 0, weights and x_q 16-byte aligned.
 * Errors: MOE_ERR_CAPACITY if workspace_bytes is below
 * moe_fp8_experts_workspace_size; MOE_ERR_SHAPE if MOE_F_MMA_E8M0 is set
 * without MOE_F_INTER_UE8M0. */
moe_status moe_fp8_experts(const uint8_t *x_q, const float *x_s,
                           const uint8_t *w13, const float *w13_s,
                           const uint8_t *w2, const float *w2_s,
                           const float *topk_weights,
                           const int32_t *sorted_token_ids, const int32_t *expert_ids,
                           const int32_t *num_tokens_post_padded,
                           int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                           int32_t block_m, int64_t sorted_cap, uint32_t flags,
                           void *out_bf16, void *workspace, size_t workspace_bytes,
                           void *stream);

/* The two stages of moe_fp8_experts, for callers that schedule them
 * separately (moe_fp8_experts = moe_fp8_gate_up then moe_fp8_down_reduce on
 * one stream, same workspace and flags):
 *   moe_fp8_gate_up      steps 3-4: writes the requantised SwiGLU rows h_q and
 *                        their scales h_s into the workspace (with the
 *                        column-slice gate/up: the FP32 SwiGLU rows, which
 *                        the down stage requantises);
 *   moe_fp8_down_reduce  step 5: reads them (and the work list the gate/up
 *                        stage leaves in the workspace), adds the weighted
 *                        down projections into out_bf16.
 * Arguments, constraints and errors as for moe_fp8_experts. */
moe_status moe_fp8_gate_up(const uint8_t *x_q, const float *x_s,
                           const uint8_t *w13, const float *w13_s,
                           const int32_t *sorted_token_ids, const int32_t *expert_ids,
                           const int32_t *num_tokens_post_padded,
                           int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                           int32_t block_m, int64_t sorted_cap, uint32_t flags,
                           void *workspace, size_t workspace_bytes, void *stream);

moe_status moe_fp8_down_reduce(const uint8_t *w2, const float *w2_s,
                               const float *topk_weights,
                               const int32_t *sorted_token_ids, const int32_t *expert_ids,
                               const int32_t *num_tokens_post_padded,
                               int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                               int32_t block_m, int64_t sorted_cap, uint32_t flags,
                               void *out_bf16, void *workspace, size_t workspace_bytes,
                               void *stream);

/* All five steps in one call: moe_plan_quant then moe_fp8_experts (arguments,
 * constraints and errors those of the two calls, validated in full before
 * anything is enqueued; outputs bit-identical to the two calls).  When the
 * plan runs as one workgroup (no plan workspace, or fewer routes than the
 * several-workgroup build takes) and the gate/up stage runs the per-block
 * kernel, the route map and split-K counters that stage would clear in a
 * launch of its own are cleared inside the plan's launch: one launch fewer
 * per layer at decode sizes.  x_q / x_s receive the activation codes and
 * scales, sorted_token_ids / expert_ids / num_tokens_post_padded the plan,
 * as from moe_plan_quant. */
moe_status moe_fp8_layer(const void *x_bf16, int64_t ld_x, int32_t scale_mode,
                         const void *topk_ids, int32_t ids_dtype, const float *topk_weights,
                         const uint8_t *w13, const float *w13_s,
                         const uint8_t *w2, const float *w2_s,
                         int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                         int32_t block_m, int32_t *sorted_token_ids, int64_t sorted_cap,
                         int32_t *expert_ids, int64_t blocks_cap,
                         int32_t *num_tokens_post_padded, uint8_t *x_q, float *x_s,
                         void *plan_workspace, size_t plan_workspace_bytes, uint32_t flags,
                         void *out_bf16, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------ weight prepack -- */

/* Offline reordering of W13 into the order the gate/up kernels consume it,
 * the analogue of the private eight-row gate/up interleave of FlashInfer PR
 * #4287 (public contract and review fixes section): for expert e, 128-column
 * tile jt < I/128 and K-block kb < K/128, one contiguous 32 KiB tile at byte
 * ((e * (I/128) + jt) * (K/128) + kb) * 32768 holds 256 rows of 128 bytes --
 * rows 0-127 are gate rows jt*128 + r of w13, rows 128-255 up rows
 * I + jt*128 + r - 128 -- with 16-byte chunk c of row r (bytes
 * kb*128 + 16c .. of the row) stored at r * 128 + 16 * (c ^ (r & 7)).  That is
 * the gate/up kernels' LDS stage image, so each of their load instructions
 * reads 1 KiB of consecutive bytes instead of 128-byte pieces of 256 rows K
 * bytes apart.  Pass MOE_F_W13_PACKED with the result; w13_s is unchanged.
 *   w13        [E, 2I, K] E4M3 (device), unchanged
 *   w13_packed moe_prepack_w13_size(E, I, K) bytes (= E * 2I * K; device),
 *              written; must not overlap w13
 * Both 16-byte aligned; I % 128 == 0, K % 128 == 0.  Asynchronous on
 * `stream`.  Errors: MOE_ERR_SHAPE (sizes, overlap), MOE_ERR_NULL,
 * MOE_ERR_ALIGN, MOE_ERR_HIP.  moe_prepack_w13_size returns 0 for sizes it
 * rejects. */
size_t moe_prepack_w13_size(int64_t E, int64_t I, int64_t K);
moe_status moe_prepack_w13(const uint8_t *w13, int64_t E, int64_t I, int64_t K,
                           uint8_t *w13_packed, void *stream);

/* ------------------------------------------------------- W4A8 variant -- */

/* Steps 3-5 with E2M1 (FP4) expert weights: FP8 activations against E2M1
 * weights with one power-of-two scale per 32 elements along K, the weight
 * scales applied in FP32 (sglang-glm53-flash-sm120 PR #13, description of
 * its FP8-activation path for E2M1-K32 weights).  Everything else -- the
 * plan, the activation and intermediate FP8 quantisation, SwiGLU, the route
 * sum into out_bf16 -- is that of moe_fp8_experts.
 *   w13   [E, 2I, K/2] uint8: E2M1 codes, two per byte, the even K index in
 *         the low nibble (sign bit 3, exponent bits 2-1 with bias 1, mantissa
 *         bit 0: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6);
 *   w13_e [E, 2I, K/32] uint8: the K32 scales as E8M0 bytes, scale =
 *         2^(byte - 127); 255 (E8M0 NaN) is not accepted and gives
 *         undefined results;
 *   w2 [E, K, I/2], w2_e [E, K, I/32]: the same for the down projection.
 * Gate/up products are exact (FP16 MFMA on widened codes, FP32 sums) while
 * the four K32 exponents of a weight row within each 128-wide K-block span
 * at most 23; beyond that the smaller groups' products round to FP16.
 * Each stage runs the per-block or the persistent kernel family, and the
 * down stage also the column split, chosen (or forced by flag bits 16-19)
 * as for moe_fp8_experts.  Constraints: those of moe_fp8_experts; w13 / w2
 * 16-byte and w13_e / w2_e 4-byte aligned; when the down stage runs the
 * per-block kernel, I / 128 <= 512 / min(max(block_m, 16), 64).  Flags
 * MOE_F_INTER_UE8M0, a forced split-K and the path bits apply;
 * MOE_F_MMA_E8M0, MOE_F_FP8_GATEUP, MOE_FUSE_ON, MOE_F_W13_PACKED and the
 * column-slice gate/up give MOE_ERR_UNSUPPORTED.  The workspace is sized by
 * moe_w4a8_experts_workspace_size (0 if the arguments are rejected); the
 * intermediate rows sit where moe_fp8_experts_workspace_layout says. */
size_t moe_w4a8_experts_workspace_size(int64_t M, int64_t K, int64_t I, int32_t E,
                                       int32_t top_k, int32_t block_m, int64_t sorted_cap,
                                       uint32_t flags);

moe_status moe_w4a8_experts(const uint8_t *x_q, const float *x_s,
                            const uint8_t *w13, const uint8_t *w13_e,
                            const uint8_t *w2, const uint8_t *w2_e,
                            const float *topk_weights,
                            const int32_t *sorted_token_ids, const int32_t *expert_ids,
                            const int32_t *num_tokens_post_padded,
                            int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                            int32_t block_m, int64_t sorted_cap, uint32_t flags,
                            void *out_bf16, void *workspace, size_t workspace_bytes,
                            void *stream);

/* ------------------------------------------------- no-allocation variant -- */

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_fp8_experts with its workspace taken from a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  Arguments, results and errors are those of
 * moe_fp8_experts (the caller still passes every input and the output);
 * sizes whose moe_fp8_experts_workspace_size exceeds the array return
 * MOE_ERR_CAPACITY before anything is enqueued (the decode shapes fit; the
 * page-1 shape at M=4096 does not).  No call allocates or frees memory: the
 * first call on a device looks up the array's device address once.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents; calls that overlap on one GPU (concurrent streams or host
 * threads) race on it and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_fp8_experts_noalloc(const uint8_t *x_q, const float *x_s,
                                   const uint8_t *w13, const float *w13_s,
                                   const uint8_t *w2, const float *w2_s,
                                   const float *topk_weights,
                                   const int32_t *sorted_token_ids, const int32_t *expert_ids,
                                   const int32_t *num_tokens_post_padded,
                                   int64_t M, int64_t K, int64_t I, int32_t E, int32_t top_k,
                                   int32_t block_m, int64_t sorted_cap, uint32_t flags,
                                   void *out_bf16, void *stream);

/* ------------------------------------------------------------ utilities -- */

const char *moe_status_str(moe_status s);
/* Text of the last MOE_ERR_HIP / validation failure on this thread (a
 * thread-local buffer, valid until this thread's next library call). */
const char *moe_last_hip_error(void);
/* The same text under its earlier name. */
const char *moe_last_error(void);

/* Test hook: convert n FP32 values to E4M3 codes with the exact device
 * routine the quantisers use (clamp to +-448, round to nearest even).
 * in/out are device pointers; n >= 0. */
moe_status moe_debug_e4m3_encode(const float *in, uint8_t *out, int64_t n, void *stream);

/* Debug check of the MOE_F_MMA_E8M0 precondition (SGLang PR #43556,
 * Motivation: scales that are not powers of two, fed to an E8M0-scaled MFMA,
 * give wrong results without any error).  Writes to count[0] (device memory,
 * one uint32, overwritten) the number of the n FP32 values at `scales` that
 * are not positive powers of two in [2^-126, 2^127]; 0 means x_s, w13_s or
 * w2_s may be used with MOE_F_MMA_E8M0.  Asynchronous on `stream`. */
moe_status moe_debug_count_non_pow2(const float *scales, int64_t n, uint32_t *count,
                                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H */
