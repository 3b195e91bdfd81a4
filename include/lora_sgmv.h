/*
 * lora_sgmv.h — C ABI of the MI355X (gfx950) segment-routed multi-adapter
 * LoRA delta:  y[t] += B[slot(t)] · (A[slot(t)] · x[t]).
 *
 * The delta is computed in two steps over a batch whose requests are sorted
 * by adapter slot: an SGMV "shrink" (x -> rank-space intermediate u) and a
 * boundary-aware "expand" (u -> the output slices of a fused q/k/v projection,
 * or of o_proj).  Both are driven by the routing triple (lora_ids,
 * grouped_offsets, end).
 *
 * Sources (by page title and section):
 *   [MAX-lora]  "MAX 的 max.pipelines.lora 模块解析" — LoRAConfig table;
 *               LoRAModel "加载时的处理管线" (validate, pre-scale, pad, fuse
 *               QKV, cast); "运行时工作流与调度交互" (base-only routing);
 *               LoRAStatus table.
 *   [MAX-V3]    Modular API page "LoRAManagerV3" — sort_lora_batch(),
 *               get_lora_graph_inputs(), bind_inputs() errors.
 *   [vLLM]      "vLLM LoRA 实现深度解析" — §1 (forward, scaling, rsLoRA,
 *               pre-multiplied scaling), §5.3 (activate_adapter, reset_lora),
 *               §6 (lora_shrink / lora_expand), §9 (stacked buffer layout).
 *
 * Conventions for every entry point
 *   - Return value: a lora_status_t code (0 = success).  No call throws,
 *     aborts or prints.  Arguments are checked before any work or launch; on
 *     an error nothing is written and nothing is launched.
 *   - Memory: the caller owns every buffer.  The library allocates no memory
 *     and keeps no pointer after a call returns.  Host calls take host
 *     pointers; device calls take device pointers (HBM) and run
 *     asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 *   - Layout: row-major, no padding between elements of a row; a row stride
 *     (ld*) in elements where stated.  bf16 data is passed as 16-bit patterns.
 *   - Thread safety: host calls are re-entrant.  Device calls that share a
 *     workspace must be ordered on one stream.
 */
#ifndef LORA_SGMV_H
#define LORA_SGMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 9

/* Status codes, modelled on the page's LoRAStatus enum ([MAX-lora] LoRAStatus
 * table: SUCCESS, LOAD_INVALID_ADAPTER, UNSPECIFIED_ERROR, ...) and on the
 * ValueError cases the pages name (bad rank/bias/target, no free slot, input
 * count mismatch). */
typedef int32_t lora_status_t;
enum {
    LORA_OK = 0,                    /* success */
    LORA_ERR_INVALID_ARGUMENT = 1,  /* null pointer, bad size/stride/dtype/family/path, bad offsets, misalignment */
    LORA_ERR_INVALID_ADAPTER = 2,   /* rank < 1 or > max_lora_rank, bias not "none", unknown target */
    LORA_ERR_SLOT_OUT_OF_RANGE = 3, /* slot id outside [-1, max_num_loras) */
    LORA_ERR_CAPACITY = 4,          /* a caller buffer (workspace, output) is too small */
    LORA_ERR_DEVICE = 5,            /* the HIP runtime reported an error for a launch */
    LORA_ERR_UNSPECIFIED = 6,       /* anything else */
    LORA_ERR_NO_FREE_SLOT = 7,      /* every slot holds an adapter that may not be evicted ([vLLM] §5.3 "No free lora slots") */
    LORA_ERR_NOT_ACTIVE = 8         /* the adapter holds no slot (LoRAStatus UNLOAD_NAME_NONEXISTENT) */
};

/* Element type of x, y and the adapter stacks.  Accumulation is always fp32. */
enum { LORA_DTYPE_F32 = 0, LORA_DTYPE_BF16 = 1 };

/* Projection families.  QKV: input width hidden, three output slices of
 * widths (n_heads*head_dim, n_kv_heads*head_dim, n_kv_heads*head_dim).
 * O: input width n_heads*head_dim, one output slice of width hidden.
 * ([MAX-lora] LoRATargetModule: fused self_attn.qkv = (q,k,v)_proj; o_proj.)
 * GATE_UP: input width hidden, two output slices of width intermediate_size
 * (gate_proj, up_proj fused like q/k/v); DOWN: input width
 * intermediate_size, one output slice of width hidden (down_proj).  The MLP
 * families need intermediate_size > 0 ([MAX-lora] 目标模块白名单: the MLP
 * projections gate_proj/up_proj/down_proj, a TODO there; [vLLM] §5.4 packed
 * modules). */
enum { LORA_FAMILY_QKV = 0, LORA_FAMILY_O = 1, LORA_FAMILY_GATE_UP = 2, LORA_FAMILY_DOWN = 3 };

/* Adapter target bits (q_proj, k_proj, v_proj, o_proj). */
enum { LORA_TARGET_Q = 1, LORA_TARGET_K = 2, LORA_TARGET_V = 4, LORA_TARGET_O = 8 };

/* Kernel path selection for the device calls.  AUTO picks per token tile:
 * wavefront-reduction VALU code for short (decode-shaped) tiles, MFMA for
 * longer bf16 tiles; for lora_sgmv_delta, when the host copy of the routing
 * shows only short groups, the one-kernel path below, or, for an input width
 * above 4096 or an output wide enough for more than two of its workgroups per
 * compute unit, its shrink half with K split over workgroups (partial sums in
 * the workspace) followed by its expand half.  VALU / MFMA force one
 * path (MFMA needs bf16; for the expand also a rank that is a multiple of 16
 * and at most 64 and slice widths that are multiples of 32).  FUSED (only
 * lora_sgmv_delta) forces the one-kernel path: shrink and expand of tiles of
 * at most 16 tokens in one launch, each workgroup recomputing the rank-space
 * values of its slice; it needs bf16, a rank of 16 or 32 and slice widths
 * that are multiples of 32, and uses no workspace. */
enum { LORA_PATH_AUTO = 0, LORA_PATH_VALU = 1, LORA_PATH_MFMA = 2, LORA_PATH_FUSED = 3 };

/* Model and LoRA capacity dimensions.  max_lora_rank (R) and max_num_loras (L)
 * correspond to LoRAConfig.max_lora_rank / max_num_loras ([MAX-lora] LoRAConfig
 * table; page defaults 16 and 1).  Constraints checked by every call:
 * all fields > 0 except intermediate_size; hidden, n_heads*head_dim,
 * n_kv_heads*head_dim and intermediate_size multiples of 8 and at most 2^20;
 * max_lora_rank a multiple of 8 and <= 128; dtype one of LORA_DTYPE_*;
 * intermediate_size 0 when the model's MLP is not targeted. */
typedef struct lora_dims {
    int32_t hidden;
    int32_t n_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t max_lora_rank;
    int32_t max_num_loras;
    int32_t dtype;
    int32_t intermediate_size;
} lora_dims_t;

/* Library ABI version (LORA_ABI_VERSION of the build). */
int32_t lora_abi_version(void);

/* Static, NUL-terminated name of a status code ("LORA_OK", ...). */
const char* lora_status_string(lora_status_t status);

/* Shape of a projection family: input width, slice count (1..4), the slice
 * widths (slice_widths needs room for 4 entries) and the total output width.
 * The packed stacks of the family are A [L][rows_t][in_features] in the
 * tiled layout below and B [L][out_features][R] row-major.
 *
 * A layout.  Logically A of one slot is [n_slices*R][in_features] (the rank
 * rows of q, k, v stacked, [MAX-lora] QKV 融合).  On the device the rows are
 * grouped in blocks of 16 (rows_t = n_slices*R rounded up to 16; the rows
 * added are zero) and each block is stored as 8-element pieces along K,
 * piece-major then row:
 *   A[row][k]  at element  ((row/16) * (K/8) + k/8) * 128 + (row%16) * 8 + k%8
 * with K = in_features.  This puts the 16 rows x 32 K values that one matrix
 * instruction consumes in one contiguous 1 KB run.  A slot holds
 * rows_t * in_features elements. */
lora_status_t lora_family_shape(const lora_dims_t* dims, int32_t family, int32_t* in_features,
                                int32_t* n_slices, int32_t* slice_widths, int32_t* out_features);

/* ---------------------------------------------------------------------------
 * lora_pack_adapter — host, synchronous.
 *
 * Turns one adapter's per-projection PEFT matrices of one layer into one slot
 * of the layer's stacks, in the page's order ([MAX-lora] 加载时的处理管线;
 * [vLLM] §1 pre-multiplied scaling, §5.3 reset_lora, §5.4 packed qkv):
 *   1. validate: bias_none != 0, 1 <= rank <= max_lora_rank, target_mask
 *      within Q|K|V|O  (else LORA_ERR_INVALID_ADAPTER);
 *   2. scale = lora_alpha / rank, or lora_alpha / sqrt(rank) when use_rslora;
 *      B <- fp32(B * fp32(scale)) (one fp32 multiply per element);
 *   3. zero-pad A [rank, in] -> [R, in] and B [out, rank] -> [out, R];
 *   4. fuse q/k/v: A_qkv = [A_q; A_k; A_v] (rank dim), B_qkv = [B_q; B_k; B_v]
 *      (output dim);
 *   5. cast to dims->dtype with round-to-nearest-even (bf16) or keep fp32.
 * A projection not in target_mask gets all-zero blocks (its delta is zero).
 *
 * Inputs: A_p [rank][in_p] and B_p [out_p][rank] fp32, row-major, for the
 * targeted projections (NULL allowed for the others); in_q = in_k = in_v =
 * hidden, in_o = n_heads*head_dim; out_q = n_heads*head_dim, out_k = out_v =
 * n_kv_heads*head_dim, out_o = hidden.
 * Outputs (host memory, dims->dtype): A_qkv [3R][hidden] and A_o [R][nq] in
 * the tiled A layout (see lora_family_shape: round16(3R) * hidden and
 * round16(R) * nq elements), B_qkv [nq+2nkv][R] and B_o [hidden][R]
 * row-major — one slot each; the caller copies them into slot s of the
 * device stacks.
 */
lora_status_t lora_pack_adapter(const lora_dims_t* dims, int32_t rank, float lora_alpha,
                                int32_t use_rslora, int32_t bias_none, uint32_t target_mask,
                                const float* A_q, const float* B_q, const float* A_k,
                                const float* B_k, const float* A_v, const float* B_v,
                                const float* A_o, const float* B_o, void* A_qkv_out,
                                void* B_qkv_out, void* A_o_out, void* B_o_out);

/* Host, synchronous: pack one adapter's projections of one family into one
 * slot's A and B — the steps of lora_pack_adapter (validate, scale B by
 * alpha/r or alpha/sqrt(r), zero-pad to max_lora_rank, concatenate the
 * slices, round to the stack dtype) for any family, the MLP ones included.
 * Slice s (in the family's slice order, e.g. gate then up) takes A_slices[s]
 * [rank][in_features] and B_slices[s] [width_s][rank] (fp32, PEFT layout)
 * when bit s of slice_mask is set, and is a zero block otherwise ([vLLM]
 * §5.3 reset_lora).  A_out: the tiled A layout, round16(n_slices*R) rows;
 * B_out: [out_features][R].  Errors: INVALID_ARGUMENT (dims, family, NULL
 * pointers for a set bit), INVALID_ADAPTER (bias not none, rank outside
 * [1, max_lora_rank], mask bits past the family's slices). */
lora_status_t lora_pack_family(const lora_dims_t* dims, int32_t family, int32_t rank, float lora_alpha,
                               int32_t use_rslora, int32_t bias_none, uint32_t slice_mask,
                               const float* const* A_slices, const float* const* B_slices, void* A_out,
                               void* B_out);

/* Host, synchronous: pack one adapter's LoRA bias of one family into one
 * slot of a bias stack [L][out_features].  [vLLM] §5.3 activate_adapter
 * writes the bias into the slot next to A and B, and only B carries the
 * scaling (§5.3 optimize); [MAX-lora] LoRAType BIAS names it a bias attached
 * to B.  The bias is therefore stored as given: bias_out = round(b) in the
 * stack dtype; slice s (bias_slices[s], width_s fp32) is zero when bit s of
 * slice_mask is clear (the slot's reset_lora for a module without one).
 * Errors: INVALID_ARGUMENT (dims, family, NULL output or a NULL slice for a
 * set bit), INVALID_ADAPTER (mask bits past the family's slices). */
lora_status_t lora_pack_bias(const lora_dims_t* dims, int32_t family, uint32_t slice_mask,
                             const float* const* bias_slices, void* bias_out);

/* ---------------------------------------------------------------------------
 * lora_build_routing — host, synchronous.
 *
 * [MAX-V3] sort_lora_batch(): requests of one adapter adjacent, ordered by
 * slot id, base requests (slot -1) last; order within a slot is arrival order
 * (stable).  [MAX-V3] get_lora_graph_inputs(): consecutive same-slot requests
 * form a group; grouping stops at the first base request; `end` is the
 * number of LoRA-routed tokens.  Requests with zero tokens keep their place
 * (a group may be empty).
 *
 * Inputs:  request_slot[num_requests] in [-1, max_num_loras);
 *          row_offsets[num_requests+1], row_offsets[0] == 0, non-decreasing,
 *          request i owns tokens [row_offsets[i], row_offsets[i+1]).
 * Outputs: perm[num_requests] (sorted position -> arrival index),
 *          sorted_row_offsets[num_requests+1],
 *          lora_ids[G] (capacity max_num_loras), grouped_offsets[G+1]
 *          (capacity max_num_loras+1; [0] = 0, [G] = end; token offsets in the
 *          sorted batch), *num_groups = G, *end.
 * Errors:  LORA_ERR_SLOT_OUT_OF_RANGE for a bad slot; LORA_ERR_INVALID_ARGUMENT
 *          for bad offsets, null pointers or end >= 2^31.
 * A base-only or empty batch gives G = 0, end = 0; the device calls then do
 * nothing.
 */
lora_status_t lora_build_routing(int32_t num_requests, const int32_t* request_slot,
                                 const int64_t* row_offsets, int32_t max_num_loras,
                                 int32_t* perm, int64_t* sorted_row_offsets, int32_t* lora_ids,
                                 int32_t* grouped_offsets, int32_t* num_groups, int64_t* end);

/* ---------------------------------------------------------------------------
 * lora_build_token_routing — host, synchronous.
 *
 * Per-token routing ([vLLM] §6 多 LoRA 并发路由机制): token_lora_mapping
 * gives every token of the batch its GPU slot (-1: no adapter), in the
 * caller's token order, and the batch is not reordered in memory.  Tokens
 * are ordered by slot, stably, base tokens last (the kernels' view, as
 * token_indices_sorted_by_lora_ids orders them for locality); consecutive
 * tokens of one slot form a group.  This is lora_build_routing with one
 * request per token.
 *
 * Inputs:  token_slot[num_tokens] in [-1, max_num_loras).
 * Outputs: token_indices_sorted[num_tokens] (sorted position -> token row),
 *          lora_ids[G] (capacity max_num_loras), grouped_offsets[G+1]
 *          (capacity max_num_loras+1), *num_groups = G, *end = the number
 *          of tokens with a slot.  Pass token_indices_sorted (its first end
 *          entries, on the device) as lora_routing_t.token_rows.
 * Errors:  LORA_ERR_SLOT_OUT_OF_RANGE for a bad slot; LORA_ERR_INVALID_ARGUMENT
 *          for null pointers or num_tokens outside [0, 2^31).
 */
lora_status_t lora_build_token_routing(int32_t num_tokens, const int32_t* token_slot, int32_t max_num_loras,
                                       int32_t* token_indices_sorted, int32_t* lora_ids,
                                       int32_t* grouped_offsets, int32_t* num_groups, int64_t* end);

/* Workspace bytes that lora_sgmv_shrink and lora_sgmv_delta need for a
 * family, for any batch with at most max_tokens LoRA-routed tokens.  The
 * workspace holds fp32 partial sums of u (one slab per K split of the shrink);
 * its contents on entry do not matter and it needs no initialisation.
 * Errors: LORA_ERR_INVALID_ARGUMENT for bad dims, family or max_tokens. */
lora_status_t lora_sgmv_workspace_bytes(const lora_dims_t* dims, int32_t family,
                                        int64_t max_tokens, size_t* bytes);

/* ---------------------------------------------------------------------------
 * The routing triple of one batch, as lora_build_routing produces it and as
 * [MAX-V3] get_lora_graph_inputs() hands it to the kernels: lora_ids and
 * grouped_offsets in device memory, `end` on the host.
 *
 * lora_ids         device int32[num_groups]: slot of each group.
 * grouped_offsets  device int32[num_groups + 1]: token offsets of the groups
 *                  in the sorted batch ([0] = 0, [num_groups] = end).
 * num_groups       G, 0 <= G <= max_num_loras.
 * end              LoRA-routed tokens, 0 <= end < 2^31.
 * host_lora_ids, host_grouped_offsets
 *                  optional host copies of the same two arrays (both or
 *                  neither; NULL = none).  When given and G <=
 *                  LORA_MAX_HOST_GROUPS, the device calls check them and pass
 *                  them to the kernels as launch arguments, so no kernel reads
 *                  the device arrays (which may then be NULL) before its first
 *                  data load.  They are read at call time: launches recorded
 *                  into a HIP graph keep the routing of the recording call.
 * token_rows, num_rows
 *                  per-token routing (lora_build_token_routing): NULL = the
 *                  rows of x, u and y are in sorted order (row t is sorted
 *                  position t).  Otherwise token_rows is a device
 *                  int32[end]: sorted position t reads row token_rows[t] of
 *                  x and updates that row of y, where x and y hold num_rows
 *                  rows in the caller's order; u stays in sorted order.  The
 *                  entries must be distinct (two positions on one y row
 *                  race); an entry outside [0, num_rows) reads zeros and
 *                  writes nothing.  Requires end <= num_rows and
 *                  (num_rows + 1) * row stride * element size <= 2^31 bytes
 *                  for x and y (else LORA_ERR_INVALID_ARGUMENT, before any
 *                  launch).  Rows not listed are neither read nor written.
 * A base-only or empty batch (G = 0 or end = 0) makes every device call a
 * no-op (the base-only routing of [MAX-lora] 运行时工作流与调度交互 — all tokens
 * on slot 0 holding all-zero adapters — is also valid and leaves y as is).
 * Malformed device arrays cannot make a kernel access rows outside [0, end)
 * or memory outside the stacks (indices are clamped, bad slot ids skipped),
 * but the results are then unspecified.
 */
#define LORA_MAX_HOST_GROUPS 64
typedef struct lora_routing {
    const int32_t* lora_ids;
    const int32_t* grouped_offsets;
    int32_t num_groups;
    int64_t end;
    const int32_t* host_lora_ids;
    const int32_t* host_grouped_offsets;
    const int32_t* token_rows;
    int64_t num_rows;
} lora_routing_t;

/* ---------------------------------------------------------------------------
 * lora_sgmv_shrink — device, asynchronous on `stream`.
 *
 * [vLLM] §6 lora_shrink (A·x, hidden -> rank) over the segments of the
 * routing triple:
 *   u[t][c] = sum_k A[lora_ids[g]][c][k] * x[t][k]
 *   for t in [grouped_offsets[g], grouped_offsets[g+1]), g < num_groups,
 *   c < n_slices*R, accumulated in fp32.
 *
 * x        [>= end rows][in_features] in dims->dtype, row stride ldx elements;
 *          rows >= end are not read.
 * A_stack  [L][round16(n_slices*R)][in_features] in dims->dtype, tiled layout
 *          (see lora_family_shape; lora_pack_adapter writes it).
 * routing  see lora_routing_t.
 * u        fp32 [end][n_slices*R] (device).
 * workspace: device scratch, >= lora_sgmv_workspace_bytes(dims, family, end)
 *          bytes (NULL allowed when that is 0); used when K is split over
 *          several workgroups, whose partial sums are then added in a fixed
 *          order (results are deterministic).
 * path     LORA_PATH_*.
 * Alignment: x, A_stack, u and workspace 16-byte aligned; ldx*element size a
 * multiple of 16 and at most 2^24 bytes.
 */
lora_status_t lora_sgmv_shrink(const lora_dims_t* dims, int32_t family, const void* x, int64_t ldx,
                               const void* A_stack, const lora_routing_t* routing, float* u,
                               void* workspace, size_t workspace_bytes, int32_t path, void* stream);

/* ---------------------------------------------------------------------------
 * lora_sgmv_expand — device, asynchronous on `stream`.
 *
 * [vLLM] §6 lora_expand (B·u, rank -> hidden), boundary-aware ([MAX-V3]
 * get_lora_graph_inputs: `end` bounds the rows the expand touches):
 *   y[t][off_s + o] = round(y[t][off_s + o] + sum_j B[lora_ids[g]][off_s + o][j] * u[t][s*R + j])
 *   for t < end in segment g, slice s with offset off_s, fp32 accumulation and
 *   one rounding to dims->dtype (round to nearest even).  Rows >= end are
 *   neither read nor written.
 *
 * u        fp32 [end][n_slices*R] (device), as lora_sgmv_shrink wrote it.
 * B_stack  [L][out_features][R] in dims->dtype.
 * bias_stack  NULL, or [L][out_features] in dims->dtype (lora_pack_bias): the
 *          slot's bias is added to the rows of its segments inside the same
 *          fp32 accumulation as B.u ([MAX-lora] LoRAType BIAS; [vLLM] §5.3
 *          set_lora's bias, §8 --enable-lora-bias).  16-byte aligned.
 * routing  see lora_routing_t.
 * y        [>= end rows][out_features] in dims->dtype, row stride ldy, updated in place.
 * Alignment: u, B_stack and y 16-byte aligned; ldy*element size a multiple of 16
 * and at most 2^24 bytes.  u must not alias y.
 */
lora_status_t lora_sgmv_expand(const lora_dims_t* dims, int32_t family, const float* u,
                               const void* B_stack, const void* bias_stack, const lora_routing_t* routing,
                               void* y, int64_t ldy, int32_t path, void* stream);

/* Tuning choices of lora_sgmv_delta.  None changes what is computed, only
 * which kernels compute it (and so the fp32 summation order); a NULL pointer
 * means the library's defaults, which are the measured best.  A negative
 * value (0 for fused_feature_tile) selects the default of that field.
 *   long_delta          AUTO on a batch with longer groups: the one-kernel
 *                       delta for long groups (workgroups of at most 64
 *                       tokens doing the shrink and the expand; bf16, ranks
 *                       16 to 64 with n_slices*R <= 64, slice widths
 *                       multiples of 64, host routing copy): -1 when the
 *                       batch fills the chip without splitting K (prefill-
 *                       sized batches) and either n_slices*R <= 16 or the
 *                       call has no workspace of lora_sgmv_workspace_bytes
 *                       (wider u otherwise takes the shrink and the expand
 *                       in two launches, measured faster there), 0 never,
 *                       1 whenever it applies.
 *   fused_max_tokens    AUTO takes the one-kernel path when no group has more
 *                       tokens than this (default 32; 0: never).
 *   splitk_short        on that path, the split-K form for an input width
 *                       above 4096 or a wide output: -1 automatic, 0 never,
 *                       1 whenever it applies (needs the workspace).
 *   fused_feature_tile  widest feature tile of the one-kernel path: 0
 *                       automatic, else a power of two in [32, 512]
 *                       (else LORA_ERR_INVALID_ARGUMENT).
 *   fused_k_rotation    staggered K ranges of the one-kernel path's waves:
 *                       -1 default (on), 0 off, 1 on.
 *   fold_slabs          two-kernel path: add the shrink's K-split partial
 *                       sums in a separate pass before the expand: -1 or 0
 *                       never (the expand adds them), 1 always. */
typedef struct lora_options {
    int32_t long_delta;
    int32_t fused_max_tokens;
    int32_t splitk_short;
    int32_t fused_feature_tile;
    int32_t fused_k_rotation;
    int32_t fold_slabs;
} lora_options_t;

/* ---------------------------------------------------------------------------
 * lora_sgmv_delta — device, asynchronous on `stream`.
 *
 * The whole delta of one family in one call: the shrink followed by the
 * boundary-aware expand ([vLLM] §6 lora_shrink then lora_expand; [MAX-V3]
 * get_lora_graph_inputs for the routing and `end`), with the rank-space
 * intermediate kept in `workspace` as fp32 partial sums that the expand adds
 * in a fixed order:
 *   y[t][off_s + o] = round(y[t][off_s + o]
 *                     + sum_j B[slot][off_s + o][j] * sum_k A[slot][s*R + j][k] * x[t][k])
 * for t < end, fp32 accumulation, one rounding to dims->dtype.  Rows >= end
 * are neither read nor written.  Arguments as for lora_sgmv_shrink and
 * lora_sgmv_expand (bias_stack as there); workspace >= lora_sgmv_workspace_bytes(dims, family, end)
 * bytes, 16-byte aligned; it must not alias x, y or the stacks.
 * path: any LORA_PATH_*; with the one-kernel paths (FUSED, or AUTO on short
 * groups when the split-K form above is not taken, or AUTO's one-kernel
 * delta for long groups, see lora_options_t) the workspace is not touched
 * and may be NULL (AUTO then never takes the split-K form), and y must not
 * alias x or the stacks.  On the other paths a NULL workspace is
 * LORA_ERR_INVALID_ARGUMENT and a short one LORA_ERR_CAPACITY.
 * options: NULL or the tuning choices above.
 */
lora_status_t lora_sgmv_delta(const lora_dims_t* dims, int32_t family, const void* x, int64_t ldx,
                              const void* A_stack, const void* B_stack, const void* bias_stack,
                              const lora_routing_t* routing, void* y, int64_t ldy, void* workspace,
                              size_t workspace_bytes, int32_t path, const lora_options_t* options,
                              void* stream);

/* ---------------------------------------------------------------------------
 * lora_sgmv_delta_noalloc — device, asynchronous on `stream`.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * lora_sgmv_delta with the same arguments minus the workspace, whose partial
 * sums go to a scratch array of lora_sgmv_noalloc_scratch_bytes() bytes
 * (64 MiB) that the library holds in each device's memory while it is loaded.
 * The call allocates and frees nothing.  A batch whose two-kernel path needs
 * more partial-sum space than the scratch holds gets LORA_ERR_CAPACITY
 * before any launch (lora_sgmv_workspace_bytes gives the need); the
 * one-kernel path needs none.  Every call on one device shares that
 * device's scratch, which keeps the last call's contents (every element a
 * call reads it has written first, so no clearing is needed): calls that
 * may overlap on one device (different streams, or host threads) race and
 * must be ordered by the caller.  LORA_ERR_DEVICE if the scratch's device
 * address cannot be obtained.
 */
size_t lora_sgmv_noalloc_scratch_bytes(void);
lora_status_t lora_sgmv_delta_noalloc(const lora_dims_t* dims, int32_t family, const void* x, int64_t ldx,
                                      const void* A_stack, const void* B_stack, const void* bias_stack,
                                      const lora_routing_t* routing, void* y, int64_t ldy, int32_t path,
                                      const lora_options_t* options, void* stream);

/* ---------------------------------------------------------------------------
 * Adapter slot cache — host, synchronous.
 *
 * Which adapter (a caller-chosen integer id >= 0, like vLLM's lora_int_id)
 * occupies which of the num_slots slots of the device stacks
 * ([vLLM] §9 lora_index_to_id; [MAX-V3] "LRU slot" of activate_adapter):
 *   - activating an adapter that holds a slot keeps the slot and makes the
 *     adapter the most recently used ([vLLM] §5.3 early return, §7 touch);
 *   - a new adapter takes the lowest free slot ([vLLM] §5.3 first free slot);
 *   - with no free slot, policy LORA_CACHE_LRU evicts the least recently used
 *     adapter that is not pinned and reuses its slot ([MAX-V3]
 *     activate_adapter; [vLLM] §7 remove_oldest, then activate), policy
 *     LORA_CACHE_NO_EVICT fails with LORA_ERR_NO_FREE_SLOT ([vLLM] §5.3);
 *   - unloading frees the slot ([MAX-V3] unload_adapter); a pinned adapter is
 *     never evicted ([vLLM] §7 pin_adapter).
 * A slot that needs_load must be filled (lora_write_slot) before a batch
 * routes tokens to it.  The cache owns its host memory (lora_cache_destroy
 * frees it); calls on one cache must not run concurrently.  On an error the
 * cache is unchanged.
 */
typedef struct lora_slot_cache lora_slot_cache_t;
enum { LORA_CACHE_LRU = 0, LORA_CACHE_NO_EVICT = 1 };

/* num_slots in [1, 2^20] (normally max_num_loras).  Errors: INVALID_ARGUMENT. */
lora_status_t lora_cache_create(int32_t num_slots, int32_t policy, lora_slot_cache_t** cache);
void lora_cache_destroy(lora_slot_cache_t* cache);

/* Activate one adapter: *slot = its slot, *needs_load = 1 when the slot must
 * be (re)written, *evicted_id = the adapter it replaced (-1 if none).
 * Errors: INVALID_ARGUMENT (NULL, id < 0), NO_FREE_SLOT. */
lora_status_t lora_cache_activate(lora_slot_cache_t* cache, int64_t adapter_id, int32_t* slot,
                                  int32_t* needs_load, int64_t* evicted_id);

/* Activate the adapters of one batch ([vLLM] §4 set_active_adapters: every
 * adapter of the batch active before the forward): adapter_ids[i] of request
 * i (-1 = base model) becomes request_slot[i] (-1 for base), ready for
 * lora_build_routing.  The batch's adapters that hold a slot are touched
 * first, then the others are activated in first-appearance order; a batch
 * never evicts its own adapters.  The slots that need loading and their
 * adapters are listed in load_slots / load_ids (capacity num_requests),
 * *num_loads of them.  Errors: INVALID_ARGUMENT, NO_FREE_SLOT (the batch
 * needs more slots than the unpinned and free ones). */
lora_status_t lora_cache_activate_batch(lora_slot_cache_t* cache, int32_t num_requests,
                                        const int64_t* adapter_ids, int32_t* request_slot,
                                        int32_t* load_slots, int64_t* load_ids, int32_t* num_loads);

/* Free the adapter's slot (*slot = the slot it held).  Errors:
 * INVALID_ARGUMENT, NOT_ACTIVE. */
lora_status_t lora_cache_unload(lora_slot_cache_t* cache, int64_t adapter_id, int32_t* slot);

/* pinned != 0: activate the adapter (as lora_cache_activate) and pin it;
 * pinned == 0: unpin an active adapter (NOT_ACTIVE otherwise). */
lora_status_t lora_cache_pin(lora_slot_cache_t* cache, int64_t adapter_id, int32_t pinned, int32_t* slot,
                             int32_t* needs_load, int64_t* evicted_id);

/* *slot = the adapter's slot, or -1 if it holds none ([MAX-V3] is_active_lora). */
lora_status_t lora_cache_lookup(const lora_slot_cache_t* cache, int64_t adapter_id, int32_t* slot);

/* slot_ids[s] = adapter in slot s or -1 ([vLLM] §9 lora_index_to_id);
 * pinned[s] (optional) = 1 if pinned.  Errors: INVALID_ARGUMENT, CAPACITY
 * (capacity < num_slots). */
lora_status_t lora_cache_slot_table(const lora_slot_cache_t* cache, int32_t capacity, int64_t* slot_ids,
                                    uint8_t* pinned);

/* ---------------------------------------------------------------------------
 * lora_write_slot / lora_reset_slot — device, asynchronous on `stream`.
 *
 * Write one adapter of one layer, as lora_pack_adapter laid it out in host
 * memory, into slot `slot` of the layer's four device stacks ([vLLM] §5.3
 * set_lora; [MAX-lora] 加载时的处理管线, last step), with host-to-device
 * copies; or zero the slot ([vLLM] §5.3 reset_lora) with a fill kernel.
 * Stacks: A_qkv [L][round16(3R)][hidden] and A_o [L][round16(R)][n_heads*head_dim]
 * in the tiled layout, B_qkv [L][q+2kv][R], B_o [L][hidden][R], dims->dtype.
 * The host buffers must stay valid until the copies have run (pinned memory
 * makes them asynchronous).  Errors: INVALID_ARGUMENT (NULL, slot outside
 * [0, max_num_loras)), DEVICE.
 */
lora_status_t lora_write_slot(const lora_dims_t* dims, int32_t slot, const void* A_qkv, const void* B_qkv,
                              const void* A_o, const void* B_o, void* A_qkv_stack, void* B_qkv_stack,
                              void* A_o_stack, void* B_o_stack, void* stream);
lora_status_t lora_reset_slot(const lora_dims_t* dims, int32_t slot, void* A_qkv_stack, void* B_qkv_stack,
                              void* A_o_stack, void* B_o_stack, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_SGMV_H */
