// Internal declarations shared by the host part (lora_host.cpp) and the
// device part (lora_sgmv.hip) of the library: argument checks, the projection
// family shapes and the launch plans (tile sizes, K split, workspace layout).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "lora_sgmv.h"

namespace lora {

// Token tile of every kernel: a tile never straddles two routing groups.
constexpr int kTileM = 64;
// Columns of the rank-space output one shrink workgroup produces.
constexpr int kShrinkCols = 64;
// Granularity of the shrink's K chunks (4 waves x 32-element MFMA steps).
constexpr int kKGrain = 128;
// Largest output-feature tile of one expand workgroup; the launch uses the
// largest power of two <= this that divides every slice width, so that a
// tile never straddles two slices.
constexpr int kExpandCols = 256;
// Workgroups a shrink launch aims for before it stops splitting K.
constexpr int kShrinkTargetBlocks = 512;
// Largest rank the kernels accept (bounds the expand's LDS u tile to 32 KB).
constexpr int kMaxRank = 128;
// Largest width (hidden, q, k/v) and largest row stride in bytes of x / y:
// they keep every per-tile buffer resource of the kernels below 2^31 bytes.
constexpr int kMaxWidth = 1 << 20;
constexpr int64_t kMaxRowBytes = 1 << 24;

struct FamilyShape {
    int in_f;        // contraction length of the shrink
    int n_s;         // output slices
    int widths[4];   // slice widths
    int offs[5];     // slice offsets, offs[n_s] = out_f
    int out_f;       // total output width
    int R;           // padded rank
    int C;           // n_s * R, width of u
    int L;           // slots
    int elem;        // bytes per element of x / y / stacks
};

// Device layout of an A stack slot (rows = the n_slices*R rank rows, K = the
// input width, a multiple of 8): the rows in blocks of 16; inside a block,
// 8-element pieces along K are stored piece-major, then row:
//   A[row][k] -> ((row / 16) * (K / 8) + k / 8) * 128 + (row % 16) * 8 + k % 8.
// One MFMA operand load (lane = 16 * k-group + row, 16 bytes each) of a
// 32-element K step is then one contiguous 1 KB run.
inline int64_t a_tiled_rows(int64_t rows) { return (rows + 15) / 16 * 16; }
inline int64_t a_tiled_elems(int64_t rows, int64_t K) { return a_tiled_rows(rows) * K; }
inline int64_t a_tiled_index(int64_t row, int64_t k, int64_t K)
{
    return ((row / 16) * (K / 8) + k / 8) * 128 + (row % 16) * 8 + k % 8;
}

lora_status_t check_dims(const lora_dims_t* d);
lora_status_t family_shape(const lora_dims_t* d, int32_t family, FamilyShape* fs);

// Split-K plan of the shrink.  With S > 1 the shrink writes S partial slabs
// [S][end][C] (fp32) that the expand (or a reduce kernel) sums in split order.
struct ShrinkPlan {
    int n_tiles;  // token-tile slots launched (upper bound on real tiles)
    int nz;       // column groups
    int cb;       // columns per group (multiple of 16, <= kShrinkCols)
    int S;        // K splits
    int kc;       // K chunk length (multiple of kKGrain)
    int64_t end;  // routed tokens
    size_t slab_bytes;  // end * C * 4
};

// Plan for a given number of routed tokens and groups.
ShrinkPlan plan_shrink(const FamilyShape& fs, int64_t end, int groups);

// Plan of the long-segment shrink (bf16): column groups of at most 64
// columns, and K split S ways in ranges of kc (a multiple of kLongKUnit)
// so that a batch of `tiles` 64-token tiles fills about kPlanCUs workgroups.
// (kPlanCUs is MI355X's compute-unit count, a constant so that the
// workspace bound does not depend on the device.)
constexpr int kLongRows = 64;
constexpr int kLongKUnit = 256;
constexpr int kLongCols = 64;
constexpr int kPlanCUs = 256;
struct LongPlan {
    int nz;  // column groups
    int cb;  // columns per group (multiple of 16, <= kLongCols)
    int S;   // K splits
    int kc;  // K range of one split
};
LongPlan plan_long(const FamilyShape& fs, int64_t tiles);
// Workspace of lora_sgmv_shrink (slabs only when S > 1).
size_t shrink_workspace(const ShrinkPlan& p);
// Workspace of lora_sgmv_delta (always the S slabs).
size_t delta_workspace(const ShrinkPlan& p);
// Workspace covering both calls for every batch with end <= max_tokens.
size_t workspace_bound(const FamilyShape& fs, int64_t max_tokens);
// Output-feature tile of the expand for this family.
int expand_tile(const FamilyShape& fs);

}  // namespace lora
