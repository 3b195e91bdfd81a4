/*
 * CPU oracle for the segment-routed multi-adapter LoRA delta.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  It shares no code,
 * header, table or helper with the GPU library: it is a plain, slow,
 * single-threaded restatement of what the three source pages define, with
 * fp64 accumulation and no blocking, fusion or reordering.
 *
 * Sources (cited by page title and section):
 *   [MAX-lora]  "MAX 的 max.pipelines.lora 模块解析" (xdnf.cn article), sections
 *               "LoRAModel：单个适配器的权重加载器 / 加载时的处理管线" and
 *               "运行时工作流与调度交互".
 *   [MAX-V3]    Modular API page "LoRAManagerV3", entries sort_lora_batch()
 *               and get_lora_graph_inputs().
 *   [vLLM]      "vLLM LoRA 实现深度解析" (gitcode/CSDN article), sections
 *               1 (LoRA 数学原理, rsLoRA 变体, 推理优化：预合并 scaling),
 *               5.3 (activate_adapter / reset_lora), 5.4 (packed qkv) and
 *               9 (内存布局).
 *
 * Every entry point returns 0 on success or a positive error code:
 *   1 = bad argument, 2 = invalid adapter, 3 = slot id out of range.
 *
 * Parity status: every function here is pinned by tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_BAD_ARG 1
#define OR_BAD_ADAPTER 2
#define OR_BAD_SLOT 3

#define OR_DTYPE_F32 0
#define OR_DTYPE_BF16 1

/* ------------------------------------------------------------------------ */
/* Scaling factor.  [vLLM] §1: scaling = alpha / r, or alpha / sqrt(r) when the
 * adapter was trained with rsLoRA. */
double oracle_scaling(double alpha, int32_t r, int32_t use_rslora)
{
    if (use_rslora)
        return alpha / sqrt((double)r);
    return alpha / (double)r;
}

/* ------------------------------------------------------------------------ */
/* Round a binary32 value to the nearest bfloat16 (8-bit significand), ties to
 * even, written from the definition: pick the closer of the two bf16
 * neighbours that bracket the value.  Infinity counts as the neighbour above
 * the largest finite bf16 (at 2^128), as IEEE overflow rounding prescribes. */
static double bf16_magnitude(uint16_t h)
{
    uint32_t bits = ((uint32_t)(h & 0x7FFFu)) << 16;
    float f;
    if ((h & 0x7FFFu) == 0x7F80u)
        return ldexp(1.0, 128);
    memcpy(&f, &bits, 4);
    return (double)f;
}

uint16_t oracle_bf16_round(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    if (isnan(f))
        return (uint16_t)((bits >> 16) | 0x0040u); /* quiet NaN, sign kept */
    if (isinf(f))
        return (uint16_t)(bits >> 16);
    uint16_t down = (uint16_t)(bits >> 16);     /* same sign, magnitude truncated */
    uint16_t up = (uint16_t)(down + 1u);        /* next magnitude of that sign */
    double v = fabs((double)f);
    double gap_down = v - bf16_magnitude(down);
    double gap_up = bf16_magnitude(up) - v;
    if (gap_down < gap_up)
        return down;
    if (gap_up < gap_down)
        return up;
    return (down & 1u) ? up : down;
}

void oracle_bf16_round_array(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_round(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Pack one adapter of one layer into the slot layout the kernels read.
 *
 * [MAX-lora] 加载时的处理管线 lists the steps in this order: validate
 * (bias must be "none", rank not above max_lora_rank), pre-multiply the scale
 * into lora_B, zero-pad [rank,in] -> [max_rank,in] and [out,rank] ->
 * [out,max_rank], concatenate q/k/v (A along the rank dim, B along the output
 * dim), cast to the base dtype.  Only q/k/v/o projections are accepted.  A
 * projection the adapter does not target gets an all-zero block, as the
 * [vLLM] §5.3 reset_lora step zeroes a slot's layer without LoRA.
 *
 * Projection order in A_in/B_in: q, k, v, o.  A_in[p] is [r, in_p] and
 * B_in[p] is [out_p, r], row-major fp32 (PEFT lora_A / lora_B).
 * Outputs (row-major, dtype `dtype`):
 *   A_qkv [3R, hidden], B_qkv [nq + 2 nkv, R], A_o [R, nq], B_o [hidden, R].
 */
int oracle_pack_adapter(int32_t hidden, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                        int32_t max_rank, int32_t dtype,
                        int32_t r, double alpha, int32_t use_rslora, int32_t bias_none,
                        uint32_t target_mask,
                        const float* const* A_in, const float* const* B_in,
                        void* A_qkv, void* B_qkv, void* A_o, void* B_o)
{
    if (hidden <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || max_rank <= 0)
        return OR_BAD_ARG;
    if (dtype != OR_DTYPE_F32 && dtype != OR_DTYPE_BF16)
        return OR_BAD_ARG;
    if (!A_qkv || !B_qkv || !A_o || !B_o || !A_in || !B_in)
        return OR_BAD_ARG;

    /* step 1: validation */
    if (!bias_none)
        return OR_BAD_ADAPTER;
    if (r < 1 || r > max_rank)
        return OR_BAD_ADAPTER;
    if (target_mask & ~0xFu)
        return OR_BAD_ADAPTER;
    for (int p = 0; p < 4; ++p)
        if ((target_mask >> p) & 1u)
            if (!A_in[p] || !B_in[p])
                return OR_BAD_ARG;

    const int64_t R = max_rank;
    const int64_t nq = (int64_t)n_heads * head_dim, nkv = (int64_t)n_kv_heads * head_dim;
    const int64_t in_dim[4] = {hidden, hidden, hidden, nq};
    const int64_t out_dim[4] = {nq, nkv, nkv, hidden};

    /* step 2: pre-multiply the scale into B, in fp32 (one rounding) */
    const float scale = (float)oracle_scaling(alpha, r, use_rslora);
    float* B_scaled[4] = {0, 0, 0, 0};
    for (int p = 0; p < 4; ++p) {
        if (!((target_mask >> p) & 1u))
            continue;
        int64_t n = out_dim[p] * r;
        B_scaled[p] = (float*)malloc(sizeof(float) * (size_t)n);
        for (int64_t i = 0; i < n; ++i)
            B_scaled[p][i] = B_in[p][i] * scale;
    }

    /* step 3: zero-pad to max_rank (absent projections stay all zero) */
    float* A_pad[4];
    float* B_pad[4];
    for (int p = 0; p < 4; ++p) {
        A_pad[p] = (float*)calloc((size_t)(R * in_dim[p]), sizeof(float));
        B_pad[p] = (float*)calloc((size_t)(out_dim[p] * R), sizeof(float));
        if (!((target_mask >> p) & 1u))
            continue;
        for (int64_t i = 0; i < r; ++i)
            for (int64_t k = 0; k < in_dim[p]; ++k)
                A_pad[p][i * in_dim[p] + k] = A_in[p][i * in_dim[p] + k];
        for (int64_t o = 0; o < out_dim[p]; ++o)
            for (int64_t j = 0; j < r; ++j)
                B_pad[p][o * R + j] = B_scaled[p][o * r + j];
    }

    /* step 4: fuse q/k/v — A stacked along the rank dim, B along the output dim */
    const int64_t n_qkv = nq + 2 * nkv;
    float* A_cat = (float*)malloc(sizeof(float) * (size_t)(3 * R * hidden));
    float* B_cat = (float*)malloc(sizeof(float) * (size_t)(n_qkv * R));
    int64_t arow = 0, brow = 0;
    for (int p = 0; p < 3; ++p) {
        memcpy(A_cat + arow * hidden, A_pad[p], sizeof(float) * (size_t)(R * hidden));
        arow += R;
        memcpy(B_cat + brow * R, B_pad[p], sizeof(float) * (size_t)(out_dim[p] * R));
        brow += out_dim[p];
    }

    /* step 5: cast to the stack dtype */
    const float* src[4] = {A_cat, B_cat, A_pad[3], B_pad[3]};
    void* dst[4] = {A_qkv, B_qkv, A_o, B_o};
    const int64_t count[4] = {3 * R * hidden, n_qkv * R, R * nq, hidden * R};
    for (int t = 0; t < 4; ++t) {
        if (dtype == OR_DTYPE_F32)
            memcpy(dst[t], src[t], sizeof(float) * (size_t)count[t]);
        else
            oracle_bf16_round_array(src[t], (uint16_t*)dst[t], count[t]);
    }

    for (int p = 0; p < 4; ++p) {
        free(B_scaled[p]);
        free(A_pad[p]);
        free(B_pad[p]);
    }
    free(A_cat);
    free(B_cat);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Packing of any projection family (the MLP ones included): the same five
 * steps as oracle_pack_adapter — validate, pre-multiply the scale into B in
 * fp32, zero-pad to max_rank, concatenate the slices (A along the rank dim,
 * B along the output dim), cast — for n_slices slices of widths[s] over
 * input width in_f.  Slice s is present when bit s of slice_mask is set
 * ([MAX-lora] 加载时的处理管线 for the steps; [vLLM] §5.4 packed modules for
 * fusing projections that share an input, as gate_proj/up_proj do).
 * Outputs (row-major, dtype `dtype`): A [n_slices R][in_f], B [sum widths][R].
 */
int oracle_pack_family(int32_t in_f, int32_t n_slices, const int32_t* widths, int32_t max_rank, int32_t dtype,
                       int32_t r, double alpha, int32_t use_rslora, int32_t bias_none, uint32_t slice_mask,
                       const float* const* A_in, const float* const* B_in, void* A_out, void* B_out)
{
    if (in_f <= 0 || n_slices <= 0 || n_slices > 4 || !widths || max_rank <= 0)
        return OR_BAD_ARG;
    if (dtype != OR_DTYPE_F32 && dtype != OR_DTYPE_BF16)
        return OR_BAD_ARG;
    if (!A_out || !B_out || !A_in || !B_in)
        return OR_BAD_ARG;
    /* step 1: validation */
    if (!bias_none || r < 1 || r > max_rank || (slice_mask >> n_slices))
        return OR_BAD_ADAPTER;
    for (int s = 0; s < n_slices; ++s)
        if (((slice_mask >> s) & 1u) && (!A_in[s] || !B_in[s]))
            return OR_BAD_ARG;
    const int64_t R = max_rank;
    int64_t n_out = 0;
    for (int s = 0; s < n_slices; ++s)
        n_out += widths[s];
    const float scale = (float)oracle_scaling(alpha, r, use_rslora);
    float* A_cat = (float*)calloc((size_t)(n_slices * R * in_f), sizeof(float));
    float* B_cat = (float*)calloc((size_t)(n_out * R), sizeof(float));
    int64_t brow = 0;
    for (int s = 0; s < n_slices; ++s) {
        if ((slice_mask >> s) & 1u) {
            /* steps 3 and 4: rows [s R, s R + r) of A, columns [0, r) of B */
            for (int64_t i = 0; i < r; ++i)
                for (int64_t k = 0; k < in_f; ++k)
                    A_cat[(s * R + i) * in_f + k] = A_in[s][i * in_f + k];
            /* step 2: B times the scale in fp32 */
            for (int64_t o = 0; o < widths[s]; ++o)
                for (int64_t j = 0; j < r; ++j)
                    B_cat[(brow + o) * R + j] = B_in[s][o * r + j] * scale;
        }
        brow += widths[s];
    }
    /* step 5: cast */
    if (dtype == OR_DTYPE_F32) {
        memcpy(A_out, A_cat, sizeof(float) * (size_t)(n_slices * R * in_f));
        memcpy(B_out, B_cat, sizeof(float) * (size_t)(n_out * R));
    } else {
        oracle_bf16_round_array(A_cat, (uint16_t*)A_out, n_slices * R * in_f);
        oracle_bf16_round_array(B_cat, (uint16_t*)B_out, n_out * R);
    }
    free(A_cat);
    free(B_cat);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Batch routing.
 *
 * [MAX-V3] sort_lora_batch(): same-adapter requests adjacent, ordered by
 * adapter id, base requests (id -1) last.  The order among requests of one
 * adapter is not stated; this keeps arrival order (a stable sort).
 * [MAX-V3] get_lora_graph_inputs(): group consecutive same-adapter requests
 * and stop at the first base group; `end` is the number of LoRA-routed tokens.
 *
 * Inputs: slot[n_req] in [-1, L); row_offsets[n_req+1], starting at 0 and
 * non-decreasing (request i owns tokens [row_offsets[i], row_offsets[i+1])).
 * Outputs: perm[n_req] (sorted position -> arrival index),
 * sorted_offsets[n_req+1], lora_ids[G], grouped_offsets[G+1] (token offsets
 * in sorted order, [0] = 0, [G] = end), *n_groups = G, *end.
 * lora_ids and grouped_offsets need room for L and L+1 entries.
 */
int oracle_route(int32_t n_req, const int32_t* slot, const int64_t* row_offsets, int32_t L,
                 int32_t* perm, int64_t* sorted_offsets, int32_t* lora_ids,
                 int32_t* grouped_offsets, int32_t* n_groups, int64_t* end)
{
    if (n_req < 0 || L < 1 || !row_offsets || !perm || !sorted_offsets || !lora_ids ||
        !grouped_offsets || !n_groups || !end)
        return OR_BAD_ARG;
    if (n_req > 0 && !slot)
        return OR_BAD_ARG;
    if (row_offsets[0] != 0)
        return OR_BAD_ARG;
    for (int32_t i = 0; i < n_req; ++i)
        if (row_offsets[i + 1] < row_offsets[i])
            return OR_BAD_ARG;
    for (int32_t i = 0; i < n_req; ++i)
        if (slot[i] < -1 || slot[i] >= L)
            return OR_BAD_SLOT;

    /* sort key: the slot id, with base (-1) after every adapter */
    /* stable insertion sort of arrival indices by key */
    for (int32_t i = 0; i < n_req; ++i) {
        int32_t cur = i;
        int64_t key = slot[cur] == -1 ? (int64_t)L : slot[cur];
        int32_t j = i - 1;
        while (j >= 0) {
            int64_t kj = slot[perm[j]] == -1 ? (int64_t)L : slot[perm[j]];
            if (kj <= key)
                break;
            perm[j + 1] = perm[j];
            --j;
        }
        perm[j + 1] = cur;
    }

    sorted_offsets[0] = 0;
    for (int32_t i = 0; i < n_req; ++i) {
        int32_t a = perm[i];
        sorted_offsets[i + 1] = sorted_offsets[i] + (row_offsets[a + 1] - row_offsets[a]);
    }

    /* group consecutive same-slot requests; stop at the first base request */
    int32_t G = 0;
    int64_t tok = 0;
    grouped_offsets[0] = 0;
    for (int32_t i = 0; i < n_req; ++i) {
        int32_t s = slot[perm[i]];
        if (s == -1)
            break;
        if (G == 0 || lora_ids[G - 1] != s) {
            lora_ids[G] = s;
            grouped_offsets[G] = (int32_t)tok;
            ++G;
        }
        tok = sorted_offsets[i + 1];
        if (tok > 2147483647LL)
            return OR_BAD_ARG;
        grouped_offsets[G] = (int32_t)tok;
    }
    *n_groups = G;
    *end = tok;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* The delta of one adapter for a run of tokens, straight from the LoRA forward
 * ([vLLM] §1: h = W0 x + scaling * B A x, with the scale already folded into
 * B by packing), for a projection family whose output is split into n_slices
 * slices.  Slice s has width widths[s]; its rows of B start after the widths
 * of the slices before it, and it contracts with u columns [s R, s R + R)
 * ([MAX-lora] QKV fusion: A stacked along the rank dim, B along the output dim).
 *
 *   u[t][c]          = sum_k A[c][k] * x[t][k]                 c < n_slices R
 *   y_out[t][off+o]  = y_in[t][off+o] + sum_j B[off+o][j] * u[t][s R + j]
 *
 * All arrays are fp64, row-major: x [n_tok, in_f], A [n_slices R, in_f],
 * B [sum(widths), R], y_in / y_out [n_tok, sum(widths)], u [n_tok, n_slices R].
 */
int oracle_delta(int32_t n_tok, int32_t in_f, int32_t n_slices, const int32_t* widths, int32_t R,
                 const double* x, const double* A, const double* B, const double* y_in,
                 double* u, double* y_out)
{
    if (n_tok < 0 || in_f <= 0 || n_slices <= 0 || R <= 0 || !widths)
        return OR_BAD_ARG;
    int64_t n_out = 0;
    for (int32_t s = 0; s < n_slices; ++s)
        n_out += widths[s];
    const int64_t C = (int64_t)n_slices * R;

    for (int64_t t = 0; t < n_tok; ++t) {
        for (int64_t c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int64_t k = 0; k < in_f; ++k)
                acc += A[c * in_f + k] * x[t * in_f + k];
            u[t * C + c] = acc;
        }
        int64_t off = 0;
        for (int32_t s = 0; s < n_slices; ++s) {
            for (int64_t o = 0; o < widths[s]; ++o) {
                double acc = 0.0;
                for (int64_t j = 0; j < R; ++j)
                    acc += B[(off + o) * R + j] * u[t * C + (int64_t)s * R + j];
                y_out[t * n_out + off + o] = y_in[t * n_out + off + o] + acc;
            }
            off += widths[s];
        }
    }
    return OR_OK;
}
