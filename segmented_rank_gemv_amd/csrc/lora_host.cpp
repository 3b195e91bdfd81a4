// Host part of the library: status strings, argument checks, projection
// family shapes, launch plans, adapter packing and batch routing.
//
// Packing follows the load pipeline of the MAX page ("MAX 的
// max.pipelines.lora 模块解析", LoRAModel 加载时的处理管线): validate, pre-scale
// B, zero-pad to max_lora_rank, fuse q/k/v, cast.  Scaling follows the vLLM
// page ("vLLM LoRA 实现深度解析", §1: alpha/r, rsLoRA alpha/sqrt(r), folded into
// B).  Routing follows the LoRAManagerV3 API page (sort_lora_batch,
// get_lora_graph_inputs).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "lora_internal.h"

namespace lora {

lora_status_t check_dims(const lora_dims_t* d)
{
    if (!d)
        return LORA_ERR_INVALID_ARGUMENT;
    if (d->hidden <= 0 || d->n_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 ||
        d->max_lora_rank <= 0 || d->max_num_loras <= 0)
        return LORA_ERR_INVALID_ARGUMENT;
    if (d->dtype != LORA_DTYPE_F32 && d->dtype != LORA_DTYPE_BF16)
        return LORA_ERR_INVALID_ARGUMENT;
    const int64_t nq = (int64_t)d->n_heads * d->head_dim;
    const int64_t nkv = (int64_t)d->n_kv_heads * d->head_dim;
    if (nq > kMaxWidth || nkv > kMaxWidth || d->hidden > kMaxWidth)
        return LORA_ERR_INVALID_ARGUMENT;
    if (d->hidden % 8 || nq % 8 || nkv % 8)
        return LORA_ERR_INVALID_ARGUMENT;
    if (d->max_lora_rank % 8 || d->max_lora_rank > kMaxRank)
        return LORA_ERR_INVALID_ARGUMENT;
    if (d->intermediate_size < 0 || d->intermediate_size % 8 || d->intermediate_size > kMaxWidth)
        return LORA_ERR_INVALID_ARGUMENT;
    return LORA_OK;
}

lora_status_t family_shape(const lora_dims_t* d, int32_t family, FamilyShape* fs)
{
    lora_status_t st = check_dims(d);
    if (st != LORA_OK)
        return st;
    const int nq = d->n_heads * d->head_dim;
    const int nkv = d->n_kv_heads * d->head_dim;
    FamilyShape f;
    memset(&f, 0, sizeof(f));
    if (family == LORA_FAMILY_QKV) {
        f.in_f = d->hidden;
        f.n_s = 3;
        f.widths[0] = nq;
        f.widths[1] = nkv;
        f.widths[2] = nkv;
    } else if (family == LORA_FAMILY_O) {
        f.in_f = nq;
        f.n_s = 1;
        f.widths[0] = d->hidden;
    } else if (family == LORA_FAMILY_GATE_UP && d->intermediate_size > 0) {
        f.in_f = d->hidden;
        f.n_s = 2;
        f.widths[0] = d->intermediate_size;
        f.widths[1] = d->intermediate_size;
    } else if (family == LORA_FAMILY_DOWN && d->intermediate_size > 0) {
        f.in_f = d->intermediate_size;
        f.n_s = 1;
        f.widths[0] = d->hidden;
    } else {
        return LORA_ERR_INVALID_ARGUMENT;
    }
    f.offs[0] = 0;
    for (int s = 0; s < f.n_s; ++s)
        f.offs[s + 1] = f.offs[s] + f.widths[s];
    f.out_f = f.offs[f.n_s];
    f.R = d->max_lora_rank;
    f.C = f.n_s * f.R;
    f.L = d->max_num_loras;
    f.elem = d->dtype == LORA_DTYPE_BF16 ? 2 : 4;
    *fs = f;
    return LORA_OK;
}

static ShrinkPlan plan_from_tiles(const FamilyShape& fs, int n_tiles, int64_t end)
{
    ShrinkPlan p;
    p.n_tiles = n_tiles;
    p.end = end;
    p.nz = (fs.C + kShrinkCols - 1) / kShrinkCols;
    p.cb = ((fs.C + p.nz - 1) / p.nz + 15) / 16 * 16;
    const int grains = (fs.in_f + kKGrain - 1) / kKGrain;
    const int blocks = std::max(1, n_tiles * p.nz);
    const int target = kShrinkTargetBlocks;
    int S = (target + blocks - 1) / blocks;
    S = std::min(std::max(S, 1), grains);
    p.kc = (grains + S - 1) / S * kKGrain;
    p.S = (fs.in_f + p.kc - 1) / p.kc;
    p.slab_bytes = (size_t)end * fs.C * sizeof(float);
    return p;
}

ShrinkPlan plan_shrink(const FamilyShape& fs, int64_t end, int groups)
{
    int n_tiles = end > 0 ? (int)((end + kTileM - 1) / kTileM) + groups : 0;
    return plan_from_tiles(fs, n_tiles, end);
}

size_t shrink_workspace(const ShrinkPlan& p) { return p.S > 1 ? (size_t)p.S * p.slab_bytes : 0; }

LongPlan plan_long(const FamilyShape& fs, int64_t tiles)
{
    LongPlan p;
    p.nz = (fs.C + kLongCols - 1) / kLongCols;
    p.cb = ((fs.C + p.nz - 1) / p.nz + 15) / 16 * 16;
    const int64_t units = (fs.in_f + kLongKUnit - 1) / kLongKUnit;
    int64_t S = kPlanCUs / std::max<int64_t>(1, tiles * p.nz);
    S = std::min(std::max<int64_t>(S, 1), units);
    p.kc = (int)((units + S - 1) / S) * kLongKUnit;
    p.S = (fs.in_f + p.kc - 1) / p.kc;
    return p;
}

size_t delta_workspace(const ShrinkPlan& p) { return (size_t)p.S * p.slab_bytes; }

size_t workspace_bound(const FamilyShape& fs, int64_t max_tokens)
{
    // A batch of `end` tokens has at least ceil(end / kTileM) + 1 tiles, and S
    // only grows as the tile count shrinks: bound S * end over tile counts k.
    // Once S reaches 1 the bound grows with end alone, so the scan stops there
    // and the largest batch closes it.
    size_t best = 0;
    const int64_t most = (max_tokens + kTileM - 1) / kTileM;
    for (int64_t k = 1; k <= most; ++k) {
        const int64_t e = std::min<int64_t>(k * kTileM, max_tokens);
        ShrinkPlan p = plan_from_tiles(fs, (int)std::min<int64_t>(k + 1, 1 << 30), e);
        best = std::max(best, delta_workspace(p));
        if (p.S == 1)
            break;
    }
    if (most > 0) {
        ShrinkPlan p = plan_from_tiles(fs, (int)std::min<int64_t>(most + 1, 1 << 30), max_tokens);
        best = std::max(best, delta_workspace(p));
    }
    // the long-segment kernel: a batch of `end` tokens has at least
    // ceil(end / kLongRows) tiles of kLongRows, and S only grows as the tile
    // count shrinks; every call keeps u (S slabs) in the workspace at most
    const size_t row = (size_t)fs.C * sizeof(float);
    const int64_t lmost = (max_tokens + kLongRows - 1) / kLongRows;
    for (int64_t k = 1; k <= lmost; ++k) {
        const int64_t e = std::min<int64_t>(k * kLongRows, max_tokens);
        const LongPlan p = plan_long(fs, k);
        best = std::max(best, (size_t)p.S * (size_t)e * row);
        if (p.S == 1)
            break;
    }
    best = std::max(best, (size_t)plan_long(fs, lmost).S * (size_t)max_tokens * row);
    return best;
}

int expand_tile(const FamilyShape& fs)
{
    int ft = kExpandCols;
    for (;;) {
        bool ok = true;
        for (int s = 0; s < fs.n_s; ++s)
            ok = ok && fs.widths[s] % ft == 0;
        if (ok || ft == 8)
            return ft;
        ft /= 2;
    }
}

// Round to nearest even bf16: add half an ulp (minus one when the kept part
// is even) and truncate; NaN keeps its sign and becomes quiet.
static inline uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace lora

using namespace lora;

extern "C" {

int32_t lora_abi_version(void) { return LORA_ABI_VERSION; }

const char* lora_status_string(lora_status_t s)
{
    switch (s) {
    case LORA_OK: return "LORA_OK";
    case LORA_ERR_INVALID_ARGUMENT: return "LORA_ERR_INVALID_ARGUMENT";
    case LORA_ERR_INVALID_ADAPTER: return "LORA_ERR_INVALID_ADAPTER";
    case LORA_ERR_SLOT_OUT_OF_RANGE: return "LORA_ERR_SLOT_OUT_OF_RANGE";
    case LORA_ERR_CAPACITY: return "LORA_ERR_CAPACITY";
    case LORA_ERR_DEVICE: return "LORA_ERR_DEVICE";
    case LORA_ERR_UNSPECIFIED: return "LORA_ERR_UNSPECIFIED";
    case LORA_ERR_NO_FREE_SLOT: return "LORA_ERR_NO_FREE_SLOT";
    case LORA_ERR_NOT_ACTIVE: return "LORA_ERR_NOT_ACTIVE";
    default: return "LORA_ERR_UNKNOWN";
    }
}

lora_status_t lora_family_shape(const lora_dims_t* dims, int32_t family, int32_t* in_features,
                                int32_t* n_slices, int32_t* slice_widths, int32_t* out_features)
{
    if (!in_features || !n_slices || !slice_widths || !out_features)
        return LORA_ERR_INVALID_ARGUMENT;
    FamilyShape fs;
    lora_status_t st = family_shape(dims, family, &fs);
    if (st != LORA_OK)
        return st;
    *in_features = fs.in_f;
    *n_slices = fs.n_s;
    for (int s = 0; s < 4; ++s)
        slice_widths[s] = s < fs.n_s ? fs.widths[s] : 0;
    *out_features = fs.out_f;
    return LORA_OK;
}

lora_status_t lora_pack_adapter(const lora_dims_t* dims, int32_t rank, float lora_alpha,
                                int32_t use_rslora, int32_t bias_none, uint32_t target_mask,
                                const float* A_q, const float* B_q, const float* A_k,
                                const float* B_k, const float* A_v, const float* B_v,
                                const float* A_o, const float* B_o, void* A_qkv_out,
                                void* B_qkv_out, void* A_o_out, void* B_o_out)
{
    lora_status_t st = check_dims(dims);
    if (st != LORA_OK)
        return st;
    if (!A_qkv_out || !B_qkv_out || !A_o_out || !B_o_out)
        return LORA_ERR_INVALID_ARGUMENT;
    // validation (bias, rank range, target whitelist)
    if (!bias_none || rank < 1 || rank > dims->max_lora_rank || (target_mask & ~0xFu))
        return LORA_ERR_INVALID_ADAPTER;
    if (!(lora_alpha == lora_alpha))
        return LORA_ERR_INVALID_ARGUMENT;
    const float* A_in[4] = {A_q, A_k, A_v, A_o};
    const float* B_in[4] = {B_q, B_k, B_v, B_o};
    for (int p = 0; p < 4; ++p)
        if (((target_mask >> p) & 1u) && (!A_in[p] || !B_in[p]))
            return LORA_ERR_INVALID_ARGUMENT;

    const int64_t R = dims->max_lora_rank, r = rank;
    const int64_t H = dims->hidden;
    const int64_t nq = (int64_t)dims->n_heads * dims->head_dim;
    const int64_t nkv = (int64_t)dims->n_kv_heads * dims->head_dim;
    const int64_t in_p[4] = {H, H, H, nq};
    const int64_t out_p[4] = {nq, nkv, nkv, H};
    // A rows and B rows of each projection inside its packed tensor
    const int64_t a_row0[4] = {0, R, 2 * R, 0};
    const int64_t b_row0[4] = {0, nq, nq + nkv, 0};
    void* A_dst[4] = {A_qkv_out, A_qkv_out, A_qkv_out, A_o_out};
    void* B_dst[4] = {B_qkv_out, B_qkv_out, B_qkv_out, B_o_out};

    const double scale = use_rslora ? (double)lora_alpha / sqrt((double)rank)
                                    : (double)lora_alpha / (double)rank;
    const float scale32 = (float)scale;
    const bool bf16 = dims->dtype == LORA_DTYPE_BF16;

    // A tensors are written in the tiled device layout (a_tiled_index); rows
    // of the last 16-row block past n_slices*R are zero
    if (bf16) {
        memset(A_qkv_out, 0, (size_t)a_tiled_elems(3 * R, H) * 2);
        memset(A_o_out, 0, (size_t)a_tiled_elems(R, nq) * 2);
    } else {
        memset(A_qkv_out, 0, (size_t)a_tiled_elems(3 * R, H) * 4);
        memset(A_o_out, 0, (size_t)a_tiled_elems(R, nq) * 4);
    }
    for (int p = 0; p < 4; ++p) {
        const bool on = (target_mask >> p) & 1u;
        // A block: rows [a_row0, a_row0 + R) of width in_p; rows >= rank are zero
        for (int64_t i = 0; i < R; ++i) {
            const int64_t row = a_row0[p] + i;
            for (int64_t k = 0; k < in_p[p]; ++k) {
                const float v = (on && i < r) ? A_in[p][i * in_p[p] + k] : 0.0f;
                const int64_t at = a_tiled_index(row, k, in_p[p]);
                if (bf16)
                    ((uint16_t*)A_dst[p])[at] = to_bf16(v);
                else
                    ((float*)A_dst[p])[at] = v;
            }
        }
        // B block: rows [b_row0, b_row0 + out_p) of width R; columns >= rank are zero
        for (int64_t o = 0; o < out_p[p]; ++o) {
            const int64_t row = b_row0[p] + o;
            for (int64_t j = 0; j < R; ++j) {
                float v = (on && j < r) ? B_in[p][o * r + j] * scale32 : 0.0f;
                if (bf16)
                    ((uint16_t*)B_dst[p])[row * R + j] = to_bf16(v);
                else
                    ((float*)B_dst[p])[row * R + j] = v;
            }
        }
    }
    return LORA_OK;
}

lora_status_t lora_pack_family(const lora_dims_t* dims, int32_t family, int32_t rank, float lora_alpha,
                               int32_t use_rslora, int32_t bias_none, uint32_t slice_mask,
                               const float* const* A_slices, const float* const* B_slices, void* A_out,
                               void* B_out)
{
    FamilyShape fs;
    lora_status_t st = family_shape(dims, family, &fs);
    if (st != LORA_OK)
        return st;
    if (!A_out || !B_out)
        return LORA_ERR_INVALID_ARGUMENT;
    if (!bias_none || rank < 1 || rank > dims->max_lora_rank || (slice_mask >> fs.n_s))
        return LORA_ERR_INVALID_ADAPTER;
    if (!(lora_alpha == lora_alpha))
        return LORA_ERR_INVALID_ARGUMENT;
    for (int s = 0; s < fs.n_s; ++s)
        if (((slice_mask >> s) & 1u) && (!A_slices || !B_slices || !A_slices[s] || !B_slices[s]))
            return LORA_ERR_INVALID_ARGUMENT;
    const int64_t R = fs.R, r = rank, K = fs.in_f;
    const double scale = use_rslora ? (double)lora_alpha / sqrt((double)rank) : (double)lora_alpha / (double)rank;
    const float scale32 = (float)scale;
    const bool bf16 = fs.elem == 2;
    memset(A_out, 0, (size_t)a_tiled_elems(fs.C, K) * fs.elem);
    for (int s = 0; s < fs.n_s; ++s) {
        const bool on = (slice_mask >> s) & 1u;
        // A rows [s R, s R + R) in the tiled layout; rows >= rank are zero
        for (int64_t i = 0; i < R; ++i)
            for (int64_t k = 0; k < K; ++k) {
                const float v = (on && i < r) ? A_slices[s][i * K + k] : 0.0f;
                const int64_t at = a_tiled_index(s * R + i, k, K);
                if (bf16)
                    ((uint16_t*)A_out)[at] = to_bf16(v);
                else
                    ((float*)A_out)[at] = v;
            }
        // B rows [offs[s], offs[s] + width) of width R; columns >= rank are zero
        for (int64_t o = 0; o < fs.widths[s]; ++o) {
            const int64_t row = fs.offs[s] + o;
            for (int64_t j = 0; j < R; ++j) {
                const float v = (on && j < r) ? B_slices[s][o * r + j] * scale32 : 0.0f;
                if (bf16)
                    ((uint16_t*)B_out)[row * R + j] = to_bf16(v);
                else
                    ((float*)B_out)[row * R + j] = v;
            }
        }
    }
    return LORA_OK;
}

lora_status_t lora_pack_bias(const lora_dims_t* dims, int32_t family, uint32_t slice_mask,
                             const float* const* bias_slices, void* bias_out)
{
    FamilyShape fs;
    lora_status_t st = family_shape(dims, family, &fs);
    if (st != LORA_OK)
        return st;
    if (!bias_out)
        return LORA_ERR_INVALID_ARGUMENT;
    if (slice_mask >> fs.n_s)
        return LORA_ERR_INVALID_ADAPTER;
    for (int s = 0; s < fs.n_s; ++s)
        if (((slice_mask >> s) & 1u) && (!bias_slices || !bias_slices[s]))
            return LORA_ERR_INVALID_ARGUMENT;
    for (int s = 0; s < fs.n_s; ++s) {
        const bool on = (slice_mask >> s) & 1u;
        for (int64_t o = 0; o < fs.widths[s]; ++o) {
            const float v = on ? bias_slices[s][o] : 0.0f;
            const int64_t at = fs.offs[s] + o;
            if (fs.elem == 2)
                ((uint16_t*)bias_out)[at] = to_bf16(v);
            else
                ((float*)bias_out)[at] = v;
        }
    }
    return LORA_OK;
}

lora_status_t lora_build_routing(int32_t num_requests, const int32_t* request_slot,
                                 const int64_t* row_offsets, int32_t max_num_loras,
                                 int32_t* perm, int64_t* sorted_row_offsets, int32_t* lora_ids,
                                 int32_t* grouped_offsets, int32_t* num_groups, int64_t* end)
{
    if (num_requests < 0 || max_num_loras < 1 || !row_offsets || !sorted_row_offsets ||
        !lora_ids || !grouped_offsets || !num_groups || !end)
        return LORA_ERR_INVALID_ARGUMENT;
    if (num_requests > 0 && (!request_slot || !perm))
        return LORA_ERR_INVALID_ARGUMENT;
    if (row_offsets[0] != 0)
        return LORA_ERR_INVALID_ARGUMENT;
    for (int32_t i = 0; i < num_requests; ++i) {
        if (row_offsets[i + 1] < row_offsets[i])
            return LORA_ERR_INVALID_ARGUMENT;
        if (request_slot[i] < -1 || request_slot[i] >= max_num_loras)
            return LORA_ERR_SLOT_OUT_OF_RANGE;
    }

    // adapter order by slot id; base (-1) after every adapter; stable
    std::vector<int32_t> order((size_t)num_requests);
    std::iota(order.begin(), order.end(), 0);
    auto key = [&](int32_t i) -> int64_t {
        return request_slot[i] < 0 ? (int64_t)max_num_loras : (int64_t)request_slot[i];
    };
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return key(a) < key(b); });

    // the routed token count must fit the int32 device offsets; checked before
    // any output is written
    int64_t lora_tokens = 0;
    for (int32_t i = 0; i < num_requests; ++i) {
        if (request_slot[order[i]] < 0)
            break;
        lora_tokens += row_offsets[order[i] + 1] - row_offsets[order[i]];
    }
    if (lora_tokens > 2147483647LL)
        return LORA_ERR_INVALID_ARGUMENT;
    int32_t G = 0;

    sorted_row_offsets[0] = 0;
    for (int32_t i = 0; i < num_requests; ++i) {
        const int32_t a = order[i];
        perm[i] = a;
        sorted_row_offsets[i + 1] = sorted_row_offsets[i] + (row_offsets[a + 1] - row_offsets[a]);
    }
    // consecutive same-slot requests form a group; stop at the first base request
    G = 0;
    grouped_offsets[0] = 0;
    for (int32_t i = 0; i < num_requests; ++i) {
        const int32_t s = request_slot[order[i]];
        if (s < 0)
            break;
        if (G == 0 || lora_ids[G - 1] != s) {
            lora_ids[G] = s;
            grouped_offsets[G] = (int32_t)sorted_row_offsets[i];
            ++G;
        }
        grouped_offsets[G] = (int32_t)sorted_row_offsets[i + 1];
    }
    *num_groups = G;
    *end = grouped_offsets[G];
    return LORA_OK;
}

// One request per token: a counting sort by slot (stable, base last) gives
// the same order, groups and end as lora_build_routing with unit requests,
// in O(num_tokens + max_num_loras).
lora_status_t lora_build_token_routing(int32_t num_tokens, const int32_t* token_slot, int32_t max_num_loras,
                                       int32_t* token_indices_sorted, int32_t* lora_ids,
                                       int32_t* grouped_offsets, int32_t* num_groups, int64_t* end)
{
    if (num_tokens < 0 || max_num_loras < 1 || !lora_ids || !grouped_offsets || !num_groups || !end)
        return LORA_ERR_INVALID_ARGUMENT;
    if (num_tokens > 0 && (!token_slot || !token_indices_sorted))
        return LORA_ERR_INVALID_ARGUMENT;
    const int32_t L = max_num_loras;
    std::vector<int32_t> count((size_t)L + 1, 0);  // bucket L: base tokens
    for (int32_t t = 0; t < num_tokens; ++t) {
        const int32_t s = token_slot[t];
        if (s < -1 || s >= L)
            return LORA_ERR_SLOT_OUT_OF_RANGE;
        ++count[s < 0 ? L : s];
    }
    std::vector<int32_t> next((size_t)L + 1);
    int32_t acc = 0, G = 0;
    grouped_offsets[0] = 0;
    for (int32_t s = 0; s <= L; ++s) {
        next[s] = acc;
        acc += count[s];
        if (s < L && count[s] > 0) {
            lora_ids[G] = s;
            grouped_offsets[G + 1] = acc;
            ++G;
        }
    }
    for (int32_t t = 0; t < num_tokens; ++t) {
        const int32_t s = token_slot[t];
        token_indices_sorted[next[s < 0 ? L : s]++] = t;
    }
    *num_groups = G;
    *end = (int64_t)num_tokens - count[L];
    return LORA_OK;
}

lora_status_t lora_sgmv_workspace_bytes(const lora_dims_t* dims, int32_t family,
                                        int64_t max_tokens, size_t* bytes)
{
    if (!bytes || max_tokens < 0 || max_tokens > 2147483647LL)
        return LORA_ERR_INVALID_ARGUMENT;
    FamilyShape fs;
    lora_status_t st = family_shape(dims, family, &fs);
    if (st != LORA_OK)
        return st;
    *bytes = workspace_bound(fs, max_tokens);
    return LORA_OK;
}

}  // extern "C"
