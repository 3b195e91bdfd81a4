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
// Output features one expand workgroup covers.
constexpr int kExpandCols = 256;
// Workgroups a shrink launch aims for before it stops splitting K.
constexpr int kShrinkTargetBlocks = 512;
// Largest rank the kernels accept.
constexpr int kMaxRank = 512;

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

lora_status_t check_dims(const lora_dims_t* d);
lora_status_t family_shape(const lora_dims_t* d, int32_t family, FamilyShape* fs);

struct ShrinkPlan {
    int n_tiles;           // token-tile slots launched (upper bound on real tiles)
    int nz;                // column groups
    int cb;                // columns per group (multiple of 16, <= kShrinkCols)
    int S;                 // K splits
    int kc;                // K chunk length (multiple of kKGrain)
    size_t counter_bytes;  // per-(tile, column group) arrival counters, 256-byte padded
    size_t partial_bytes;  // fp32 partial tiles [n_tiles][S][kTileM][C]
};

// Plan for a given number of routed tokens and groups.
ShrinkPlan plan_shrink(const FamilyShape& fs, int64_t end, int groups);
// Workspace bytes covering every plan with end <= max_tokens, groups <= L.
size_t shrink_workspace_bound(const FamilyShape& fs, int64_t max_tokens);

}  // namespace lora
