// Host-side check of the launch tables the library builds from the host copy
// of the routing, with no GPU call: the library source is compiled into this
// program and its table builders are called on synthetic routings.
//   - the split shrink's XCD placement table: every (tile, K split, column
//     group) of the plan appears exactly once, and nothing else;
//   - the one-kernel delta's feature-tile table (also with the uneven split
//     to one workgroup per compute unit) and the split-K expand half's: the
//     tiles of each slice are whole 32-feature pairs, no wider than the
//     launch allows, and cover the slice exactly once, in order.
// Prints one line per failed case and "bad N" at the end; exits nonzero if
// any case failed.
#include "lora_sgmv.hip"

#include <cstdio>
#include <random>
#include <set>
#include <vector>

using namespace lora;

namespace {

int g_tables = 0;  // tables actually built and checked

bool make_common(int hidden, int n_kv_heads, int inter, int R, int L, int family, const std::vector<int>& lens,
                 std::vector<int>& offs, std::vector<int>& ids, Common& c)
{
    lora_dims_t d{};
    d.hidden = hidden;
    d.head_dim = 128;
    d.n_heads = hidden / 128;
    d.n_kv_heads = n_kv_heads;
    d.max_lora_rank = R;
    d.max_num_loras = L;
    d.dtype = LORA_DTYPE_BF16;
    d.intermediate_size = inter;
    const int G = (int)lens.size();
    offs.assign(G + 1, 0);
    ids.resize(G);
    for (int g = 0; g < G; ++g) {
        offs[g + 1] = offs[g] + lens[g];
        ids[g] = g % L;
    }
    lora_routing_t rt{};
    rt.end = offs[G];
    rt.num_groups = G;
    rt.host_lora_ids = ids.data();
    rt.host_grouped_offsets = offs.data();
    return check_common(&d, family, LORA_PATH_AUTO, &rt, nullptr, &c) == LORA_OK;
}

// The shrink placement table against the plain enumeration of the plan.
int check_shrink(const Common& c, const char* what)
{
    const ShrinkPlan p = plan_shrink(c.fs, c.r.end, c.r.G);
    static ShrinkArgs a;
    a.xmap_on = 0;
    int64_t grid = (int64_t)p.n_tiles * p.S * p.nz;
    if (!shrink_xcd_map(c, p, a, grid))
        return 0;  // plain order: nothing to check
    ++g_tables;
    int bad = 0;
    std::multiset<uint32_t> seen;
    for (int64_t b = 0; b < grid; ++b)
        if (a.xmap[b] != kNoEntry)
            seen.insert(a.xmap[b]);
    if (grid > kShrinkMapMax || grid % kXcds != 0)
        ++bad;
    size_t want = 0;
    for (int t = 0; t < c.r.k_tile0[c.r.G]; ++t)
        for (int s = 0; s < p.S; ++s)
            for (int z = 0; z < p.nz; ++z, ++want)
                if (seen.count((uint32_t)t << 16 | (uint32_t)s << 8 | (uint32_t)z) != 1)
                    ++bad;
    if (seen.size() != want)
        ++bad;
    if (bad)
        printf("shrink table %s: %d wrong entries (grid %lld)\n", what, bad, (long long)grid);
    return bad;
}

// A feature-tile table against the family's slices: whole pairs of at most
// max_pairs, each slice covered once, in order.
int check_feature_tiles(const Common& c, const FusedArgs& a, int max_pairs, const char* what)
{
    int bad = 0;
    int next[4], cover[4] = {0, 0, 0, 0};
    for (int sl = 0; sl < c.fs.n_s; ++sl)
        next[sl] = c.fs.offs[sl];
    if (a.nf < 1 || a.nf > kFusedHostFt)
        ++bad;
    for (int i = 0; i < a.nf && i < kFusedHostFt; ++i) {
        const int sl = a.fts[i].x & 0xFF, pairs = a.fts[i].x >> 8, f = a.fts[i].y;
        if (sl >= c.fs.n_s || pairs < 1 || pairs > max_pairs || f != next[sl]) {
            ++bad;
            continue;
        }
        next[sl] += 32 * pairs;
        cover[sl] += 32 * pairs;
    }
    for (int sl = 0; sl < c.fs.n_s; ++sl)
        if (cover[sl] != c.fs.widths[sl])
            ++bad;
    if (bad)
        printf("feature tiles %s: %d problems (nf %d)\n", what, bad, a.nf);
    return bad;
}

int check_fused(const Common& c, int64_t rows, int F0, bool uneven, const char* what)
{
    static FusedArgs a;
    fused_common_args(c, a, nullptr, 0, nullptr, nullptr, nullptr, nullptr, 0);
    set_fused_feat(c, a, F0 ? F0 : fused_widest_feat(c));
    if (a.nf > kFusedHostFt)
        return 0;  // the callers launch without the table then
    const int max_pairs = a.F / 32;
    fused_feature_tiles(c, a, rows, true, uneven);
    ++g_tables;
    return check_feature_tiles(c, a, max_pairs, what);
}

}  // namespace

int main()
{
    int bad = 0;
    std::vector<int> offs, ids;
    Common c;
    // the mixed batch's groups (hidden 5120, 8 kv heads, rank 64, 32 slots)
    const std::vector<int> mixed = {216, 155, 112, 107, 105, 22, 13, 9, 6, 6, 5, 5, 5, 4, 3,
                                    3,   3,   3,   2,   2,   2,  2,  1, 1, 1, 1, 1, 1, 1, 1};
    for (int fam : {LORA_FAMILY_QKV, LORA_FAMILY_O}) {
        if (!make_common(5120, 8, 0, 64, 32, fam, mixed, offs, ids, c)) {
            printf("mixed routing rejected\n");
            ++bad;
            continue;
        }
        bad += check_shrink(c, "mixed");
    }
    // random routings: group lengths from one token to a few 64-token tiles
    std::mt19937 rng(12345);
    for (int it = 0; it < 300; ++it) {
        const int G = 1 + (int)(rng() % 40);
        std::vector<int> lens(G);
        for (int g = 0; g < G; ++g)
            lens[g] = (rng() % 4 == 0) ? (int)(rng() % 300) : (int)(rng() % 20);
        const int R = 16 << (rng() % 3);
        const int fam = (rng() & 1) ? LORA_FAMILY_QKV : LORA_FAMILY_O;
        if (!make_common(4096, 8, 0, R, 64, fam, lens, offs, ids, c)) {
            printf("random routing %d rejected\n", it);
            ++bad;
            continue;
        }
        bad += check_shrink(c, "random");
    }
    // feature tiles: decode attention (2 tiles per XCD), MLP expand half
    // (gate_up at 2048 features, down at 512), random shapes and heights
    const std::vector<int> one = {16};
    if (make_common(4096, 8, 0, 16, 8, LORA_FAMILY_QKV, one, offs, ids, c))
        bad += check_fused(c, 2, 0, true, "decode qkv");
    if (make_common(4096, 8, 0, 16, 8, LORA_FAMILY_O, one, offs, ids, c))
        bad += check_fused(c, 2, 0, true, "decode o");
    if (make_common(4096, 8, 14336, 16, 8, LORA_FAMILY_GATE_UP, one, offs, ids, c))
        bad += check_fused(c, 2, 2048, true, "gate_up expand half");
    if (make_common(4096, 8, 14336, 16, 8, LORA_FAMILY_DOWN, one, offs, ids, c))
        bad += check_fused(c, 2, 512, true, "down expand half");
    for (int it = 0; it < 500; ++it) {
        const int hidden = 128 * (1 + (int)(rng() % 64));
        int kv = 1 + (int)(rng() % 8);
        if (128 * kv > hidden)
            kv = hidden / 128;
        const int fam = (rng() & 1) ? LORA_FAMILY_QKV : LORA_FAMILY_O;
        if (!make_common(hidden, kv, 0, 16 << (rng() % 2), 8, fam, one, offs, ids, c)) {
            printf("random shape %d rejected\n", it);
            ++bad;
            continue;
        }
        bad += check_fused(c, 1 + (int)(rng() % 8), 0, (rng() & 1) != 0, "random");
    }
    // most cases must have built a table (else the check is empty)
    if (g_tables < 500) {
        printf("only %d tables built\n", g_tables);
        ++bad;
    }
    printf("tables %d bad %d\n", g_tables, bad);
    return bad != 0;
}
