// gfx950 (MI355X, CDNA4) kernels of the segment-routed multi-adapter LoRA
// delta and the device entry points of the C ABI.
//
//   shrink:  u[t, c]       = sum_k A[slot(t), c, k] * x[t, k]          (fp32 acc)
//   expand:  y[t, off_s+o] = y[t, off_s+o] + sum_j B[slot(t), off_s+o, j] * u[t, s R + j]
//
// The routing triple (lora_ids, grouped_offsets, end) comes from the
// LoRAManagerV3 API page (get_lora_graph_inputs: consecutive same-adapter
// requests grouped, truncated at the first base group, `end` = routed tokens
// read by the boundary-aware expand).  The shrink/expand split is the one of
// the vLLM page (§6, lora_shrink A·x and lora_expand B·(A·x)); the fused q/k/v
// layout (A stacked along the rank dim, B along the output dim) is the one of
// the MAX page (加载时的处理管线, QKV 融合).
//
// Work decomposition.  Every group g (one adapter slot, a contiguous run of
// sorted tokens) is cut into token tiles of kTileM tokens that never straddle
// two groups; a 1-D grid enumerates (token tile x K split x column group) for
// the shrink and (token tile x feature tile) for the expand.  Each workgroup
// finds its group with one wave-wide scan over grouped_offsets, so the host
// needs only `end` and the group count.
//
// Paths.  A tile with few tokens (decode-shaped) is a batch of GEMVs: the
// shrink streams A rows with 16-lane groups along K and finishes with
// wavefront reductions; the expand keeps B rows in registers and streams
// y.  Longer bf16 tiles are real dense contractions and use
// v_mfma_f32_16x16x32_bf16.  Both read x, A, B and y with 16-byte vector loads.
//
// Split K.  Decode batches have few tokens per group, so the shrink splits K
// over S workgroups to occupy the chip.  Each split writes its own fp32 slab
// of u; the consumer (the expand of lora_sgmv_delta, or reduce_slabs after
// lora_sgmv_shrink) adds the slabs in split order.  Kernel boundaries are the
// only synchronisation: no atomics, no device-scope fences, deterministic
// results.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <type_traits>
#include <atomic>
#include <mutex>
#include <string.h>

#include "lora_internal.h"

// Scratch of lora_sgmv_delta_noalloc: the partial sums that lora_sgmv_delta
// keeps in the caller's workspace, in a device array of fixed size instead
// (each device holds its own copy while the library is loaded).  In host
// code `scratch` names a host-side stand-in, not a device address: the
// array's address on a device comes from hipGetSymbolAddress with that
// device current, once per device, and only that address reaches kernels.
static constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

#ifndef LORA_SHRINK_KC
#define LORA_SHRINK_KC 128
#endif

namespace lora {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;  // consecutive workgroups go to consecutive XCDs
// K elements one MFMA-shrink workgroup stages per pass (row runs of 2 KC bytes)
constexpr int kShrinkKC = LORA_SHRINK_KC;
// Host placement table of the 256-thread shrink (host routing only): one
// entry per workgroup (shrink_xcd_map).
constexpr int kShrinkMapMax = 640;
constexpr uint32_t kNoEntry = 0xFFFFFFFFu;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint32_t h16) { return __uint_as_float(h16 << 16); }

// fp32 -> bf16 round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t f2bf_pair(float lo, float hi)
{
    f32x2_t v = {lo, hi};
    bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Buffer-resource access (raw buffer loads/stores with a byte offset).  An
// offset at or past the resource size reads as zero and drops stores, which
// masks rows and K positions without branches; every resource covers less
// than 2^31 bytes (the entry points check this for the per-token layout,
// where one resource spans all of x or y) and every masked offset is kOOB
// plus a small constant.
constexpr uint32_t kOOB = 0x80000000u;

// Cache policy bits of an access (kKeep: default; kStream: non-temporal).
// The long-group kernels touch x (and the one-kernel delta y) once, and
// access them non-temporally: kept out of the caches they no longer push
// out the lines the next call would otherwise have to write back first
// (prefill step, 4 layers: 0.653 -> 0.611 ms).  So does the rank-16 MFMA
// expand with y (prefill split API step 0.646 -> 0.606 ms) and the expand
// half of the split-K delta for short groups (MLP decode step 0.835 ->
// 0.791 ms).  The same policy measured slower on the decode kernel's x and
// on the rank-32/64 expand's y (32-layer stack +5 %), which keep kKeep.
enum CachePolicy { kKeep = 0, kStream = 2 };

template <int POL = kKeep>
struct BufT {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ BufT(const void* base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000))
    {
    }
    // the same buffer with another cache policy
    template <int P2>
    __device__ __forceinline__ explicit BufT(const BufT<P2>& o) : r(o.r)
    {
    }
    __device__ __forceinline__ uint4 ld16(uint32_t off) const
    {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POL));
    }
    __device__ __forceinline__ uint2 ld8(uint32_t off) const
    {
        return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, POL));
    }
    __device__ __forceinline__ void st8(uint32_t off, uint2 v) const
    {
        typedef unsigned int u32x2 __attribute__((__vector_size__(8)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, POL);
    }
    __device__ __forceinline__ void st16(uint32_t off, uint4 v) const
    {
        typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, POL);
    }
};
typedef BufT<kKeep> Buf;
typedef BufT<kStream> StreamBuf;

// 8 consecutive elements of T as fp32
template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
    typedef uint4 Raw;
    template <class B>
    static __device__ __forceinline__ Raw load_raw(const B& b, uint32_t off) { return b.ld16(off); }
    template <class B>
    static __device__ __forceinline__ void store_buf(const B& b, uint32_t off, const float* f)
    {
        uint4 v;
        v.x = f2bf_pair(f[0], f[1]);
        v.y = f2bf_pair(f[2], f[3]);
        v.z = f2bf_pair(f[4], f[5]);
        v.w = f2bf_pair(f[6], f[7]);
        b.st16(off, v);
    }
    static __device__ __forceinline__ Raw load_raw(const uint16_t* p) { return ld16(p); }
    static __device__ __forceinline__ void store_raw(uint16_t* p, const Raw& v) { st16(p, v); }
    static __device__ __forceinline__ void unpack(const Raw& v, float* f)
    {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf2f(w[i] & 0xFFFFu);
            f[2 * i + 1] = bf2f(w[i] >> 16);
        }
    }
    static __device__ __forceinline__ void load(const uint16_t* p, float* f)
    {
        uint4 v = ld16(p);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf2f(w[i] & 0xFFFFu);
            f[2 * i + 1] = bf2f(w[i] >> 16);
        }
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float* f)
    {
        uint4 v;
        v.x = f2bf_pair(f[0], f[1]);
        v.y = f2bf_pair(f[2], f[3]);
        v.z = f2bf_pair(f[4], f[5]);
        v.w = f2bf_pair(f[6], f[7]);
        st16(p, v);
    }
};
template <> struct Vec8<float> {
    struct Raw {
        uint4 a, b;
    };
    template <class B>
    static __device__ __forceinline__ Raw load_raw(const B& b, uint32_t off)
    {
        return Raw{b.ld16(off), b.ld16(off + 16)};
    }
    template <class B>
    static __device__ __forceinline__ void store_buf(const B& b, uint32_t off, const float* f)
    {
        b.st16(off, make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                               __float_as_uint(f[3])));
        b.st16(off + 16, make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                                    __float_as_uint(f[7])));
    }
    static __device__ __forceinline__ Raw load_raw(const float* p) { return Raw{ld16(p), ld16(p + 4)}; }
    static __device__ __forceinline__ void store_raw(float* p, const Raw& v)
    {
        st16(p, v.a);
        st16(p + 4, v.b);
    }
    static __device__ __forceinline__ void unpack(const Raw& v, float* f)
    {
        f[0] = __uint_as_float(v.a.x); f[1] = __uint_as_float(v.a.y);
        f[2] = __uint_as_float(v.a.z); f[3] = __uint_as_float(v.a.w);
        f[4] = __uint_as_float(v.b.x); f[5] = __uint_as_float(v.b.y);
        f[6] = __uint_as_float(v.b.z); f[7] = __uint_as_float(v.b.w);
    }
    static __device__ __forceinline__ void load(const float* p, float* f)
    {
        uint4 a = ld16(p), b = ld16(p + 4);
        f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y);
        f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
        f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y);
        f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
    }
    static __device__ __forceinline__ void store(float* p, const float* f)
    {
        st16(p, make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                           __float_as_uint(f[3])));
        st16(p + 4, make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                               __float_as_uint(f[7])));
    }
};

__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(v, d, 64);
        if (lane >= d)
            v += o;
    }
    return v;
}

struct TileInfo {
    int g;     // group
    int slot;  // adapter slot of the group
    int t0;    // first token (sorted order)
    int n;     // tokens in the tile, 1..kTileM
    int glen;  // tokens in the whole group (decides the kernel path)
};

// Rows of one token tile in x or y.  Sorted layout (GATHER false): the
// tile's tokens are rows t0 .. t0 + n - 1 and the tile's buffer resource
// spans just those rows, so a row past the tile lies outside it.  Per-token
// routing ([vLLM] §6 LoRAMapping, token_indices_sorted_by_lora_ids): sorted
// position t0 + r is row idx[t0 + r] of the caller's buffer of nrows rows;
// the resource spans the whole buffer, and a row past the tile, or an index
// outside [0, nrows), maps to row nrows, which lies outside it.
template <bool GATHER>
struct RowMap {
    const int* idx;
    int t0, n;
    uint32_t nrows;
    __device__ __forceinline__ uint32_t operator()(int r) const
    {
        // a negative r (possible on a padding tile, n = 0) is past the tile too
        if constexpr (GATHER)
            return (uint32_t)r < (uint32_t)n ? min((uint32_t)idx[t0 + r], nrows) : nrows;
        else
            return (uint32_t)r;
    }
    template <typename T>
    __device__ __forceinline__ Buf buf(const T* base, int64_t ld) const
    {
        if constexpr (GATHER)
            return Buf(base, (uint32_t)((int64_t)nrows * ld * (int64_t)sizeof(T)));
        else
            return Buf(base + (size_t)t0 * ld, (uint32_t)((int64_t)n * ld * (int64_t)sizeof(T)));
    }
};

// Routing as the kernels see it: the device arrays, or (kr != 0) a copy of
// them carried in the kernel arguments.
struct RouteArgs {
    const int* ids;
    const int* offs;
    int G, end, L;
    int kr;
    const int* rows;  // per-token routing: sorted position -> row of x and y (null: rows in sorted order)
    uint32_t nrows;   // rows of x and y under per-token routing
    int k_offs[LORA_MAX_HOST_GROUPS + 1];
    int k_ids[LORA_MAX_HOST_GROUPS];
    // host copy: first kTileM-token tile of each group (k_tile0[G] = tiles)
    int k_tile0[LORA_MAX_HOST_GROUPS + 1];
};

// Locate token tile `tile`: groups are cut into tiles of at most TM tokens
// in group order (BAL: a group of n tokens becomes ceil(n / TM) tiles of
// near-equal size; otherwise TM-token tiles and a shorter last one).  Every
// lane takes one group, a wave-wide inclusive scan of the per-group tile
// counts gives each group's first tile and a ballot finds the group holding
// `tile`.  Offsets are clamped into [0, end] and made non-decreasing per
// group, so malformed routing cannot move accesses outside rows [0, end).
// Returns false past the last tile or for a bad slot id.
template <int TM, bool BAL>
__device__ bool locate_tile(const RouteArgs& r, int tile, TileInfo& ti)
{
    const int lane = threadIdx.x & 63;
    if constexpr (TM == kTileM && !BAL) {
        if (r.kr) {
            // host copy: the groups' first tiles are in the arguments (at most
            // 64 groups, one per lane), so one load and a ballot find the
            // group; the host has checked the offsets (monotone, [0, end])
            // lane g loads group g's entries, all in one round; the group's
            // values are then read from its lane, with no second round
            const bool in = lane < r.G;
            const int first_l = in ? r.k_tile0[lane] : 0;
            const int last_l = in ? r.k_tile0[lane + 1] : 0;
            const int gs_l = in ? r.k_offs[lane] : 0;
            const int ge_l = in ? r.k_offs[lane + 1] : 0;
            const int id_l = in ? r.k_ids[lane] : -1;
            const unsigned long long hit = __ballot(in && tile < last_l);
            if (!hit)
                return false;
            const int g = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
            const int gs = __builtin_amdgcn_readlane(gs_l, g), ge = __builtin_amdgcn_readlane(ge_l, g);
            const int t0 = gs + (tile - __builtin_amdgcn_readlane(first_l, g)) * TM;
            ti.g = g;
            ti.t0 = t0;
            ti.n = min(t0 + TM, ge) - t0;
            ti.glen = ge - gs;
            ti.slot = __builtin_amdgcn_readlane(id_l, g);
            return ti.slot >= 0 && ti.slot < r.L;
        }
    }
    int base = 0;
    for (int c0 = 0; c0 < r.G; c0 += 64) {
        const int i = c0 + lane;
        int s = 0, e = 0;
        if (i < r.G) {
            const int o0 = r.kr ? r.k_offs[i] : r.offs[i];
            const int o1 = r.kr ? r.k_offs[i + 1] : r.offs[i + 1];
            s = min(max(o0, 0), r.end);
            e = min(max(o1, s), r.end);
        }
        const int nt = (e - s + TM - 1) / TM;
        const int incl = wave_incl_scan(nt);
        const unsigned long long hit = __ballot(i < r.G && base + incl > tile);
        if (hit) {
            const int src = __ffsll((long long)hit) - 1;
            const int gs = __shfl(s, src, 64), ge = __shfl(e, src, 64);
            const int gnt = __shfl(nt, src, 64);
            const int first = base + __shfl(incl, src, 64) - gnt;
            const int j = tile - first, len = ge - gs;
            int t0, t1;
            if (BAL) {
                t0 = gs + (int)(((int64_t)len * j) / gnt);
                t1 = gs + (int)(((int64_t)len * (j + 1)) / gnt);
            } else {
                t0 = gs + j * TM;
                t1 = min(t0 + TM, ge);
            }
            // wave-uniform values: keep them in scalar registers
            ti.g = __builtin_amdgcn_readfirstlane(c0 + src);
            ti.t0 = __builtin_amdgcn_readfirstlane(t0);
            ti.n = __builtin_amdgcn_readfirstlane(t1 - t0);
            ti.glen = __builtin_amdgcn_readfirstlane(len);
            ti.slot = __builtin_amdgcn_readfirstlane(r.kr ? r.k_ids[ti.g] : r.ids[ti.g]);
            return ti.slot >= 0 && ti.slot < r.L;
        }
        base += __shfl(incl, 63, 64);
    }
    return false;
}

// ---------------------------------------------------------------------------
// shrink

struct ShrinkArgs {
    const void* x;
    int64_t ldx;
    const void* A;  // [L][a_slot] in the tiled A layout (a_tiled_index)
    int64_t a_slot;  // elements per slot: C rounded up to 16, times in_f
    float* out;     // slab s at out + s * slab, each [end][C]; S == 1: u itself
    int64_t slab;
    int in_f, C;
    int S, kc, nz, cb;
    int valu_max;  // tiles with at most this many tokens take the VALU path
    RouteArgs r;
    // host placement (xmap_on): workgroup b takes xmap[b] = tile << 16 |
    // split << 8 | column group, or nothing (kNoEntry)
    int xmap_on;
    uint32_t xmap[kShrinkMapMax];
};
static_assert(sizeof(ShrinkArgs) <= 4096, "kernel argument segment");

// VALU path (decode-shaped tiles, and every fp32 tile).  The columns
// [c0, c1) are nbk <= 4 blocks of 16 A rows; the four waves take one block
// each (nbk >= 3) or split the K range 4 / nbk ways per block.  Lane
// (g = lane / 16, r = lane % 16) owns column 16 b + r and the K pieces
// (8 elements) g, g + 4, g + 8, ... of its wave's range, so the four 16-lane
// groups read four consecutive pieces of the tiled A: one contiguous run per
// load.  The range goes in chunks of kValuChunk pieces: each lane first
// issues the loads of its A pieces of the chunk, then the workgroup stages
// the chunk's x pieces of eight tokens in LDS with coalesced loads, and the
// lanes read x from there (the 16 lanes of a group read the same piece).
// Two xor steps over lane bits 4 and 5 add the four K groups; the K-split
// waves are added in wave order through LDS (res: [4][kTileM][16 nbk]).
// Rows past the tile read as zero.
constexpr int kValuChunk = 32;            // pieces per chunk
constexpr int kValuPer = kValuChunk / 4;  // pieces per lane and chunk

template <typename T, bool GATHER>
__device__ void shrink_valu(const ShrinkArgs& a, const TileInfo& ti, int k0, int k1, int c0,
                            int c1, float* dst, int64_t dst_ld, float* res, T* xs)
{
    constexpr int E = sizeof(T);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, r = lane & 15;
    const int cw = c1 - c0, nbk = (cw + 15) >> 4;
    const int kparts = 4 / nbk;
    const int b = w % nbk, kp = w / nbk;
    const int ldr = 16 * nbk;
    const bool active = kp < kparts;  // with three blocks the fourth wave idles
    // pieces of the workgroup's K range; wave kp takes the chunks' slices
    // [kp * per, (kp + 1) * per) of every chunk
    const int pw0 = k0 >> 3, pw1 = (k1 + 7) >> 3;
    const int per = kValuChunk / kparts;  // pieces of a chunk per wave
    const RowMap<GATHER> xm{a.r.rows, ti.t0, ti.n, a.r.nrows};
    const T* Ab = reinterpret_cast<const T*>(a.A) + (size_t)ti.slot * a.a_slot +
                  (size_t)((c0 >> 4) + b) * 16 * a.in_f;
    const Buf xb = xm.buf(reinterpret_cast<const T*>(a.x), a.ldx);
    const Buf ab(Ab, (uint32_t)(16 * a.in_f * E));
    constexpr int XJ = 8 * kValuChunk / kThreads;
    for (int tb = 0; tb < ti.n; tb += 8) {
        // the rows of this lane's x pieces, the same for every chunk
        uint32_t xrow[XJ];
#pragma unroll
        for (int j = 0; j < XJ; ++j)
            xrow[j] = xm(tb + (tid + kThreads * j) / kValuChunk);
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] = 0.f;
        for (int cb = pw0; cb < pw1; cb += kValuChunk) {
            // A pieces of this lane: cb + kp * per + g + 4 j, j < per / 4
            typename Vec8<T>::Raw aq[kValuPer];
#pragma unroll
            for (int j = 0; j < kValuPer; ++j) {
                const int pl = kp * per + g + 4 * j, p = cb + pl;
                aq[j] = Vec8<T>::load_raw(
                    ab, (active && 4 * j < per && p < pw1) ? (uint32_t)((p * 16 + r) * 8) * E : kOOB);
            }
            // x pieces of eight tokens: xs[token][piece] (rows past the tile are zero)
            typename Vec8<T>::Raw xr[XJ];
#pragma unroll
            for (int j = 0; j < XJ; ++j) {
                const int e = tid + kThreads * j, i = e / kValuChunk, pc = e - i * kValuChunk;
                xr[j] = Vec8<T>::load_raw(
                    xb, cb + pc < pw1 ? (uint32_t)(xrow[j] * a.ldx + 8 * (cb + pc)) * E : kOOB);
            }
            __syncthreads();  // the previous chunk's readers are done with xs
#pragma unroll
            for (int j = 0; j < 8 * kValuChunk / kThreads; ++j) {
                const int e = tid + kThreads * j;
                Vec8<T>::store_raw(xs + 8 * e, xr[j]);
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kValuPer; ++j) {
                const int pl = kp * per + g + 4 * j;
                if (active && 4 * j < per && cb + pl < pw1) {
                    float av[8];
                    Vec8<T>::unpack(aq[j], av);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        float xv[8];
                        Vec8<T>::unpack(Vec8<T>::load_raw(xs + 8 * (i * kValuChunk + pl)), xv);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[i] = fmaf(av[e], xv[e], acc[i]);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v = acc[i];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[i] = v;
        }
        if (active && g == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (tb + i < ti.n)
                    res[(kp * kTileM + tb + i) * ldr + 16 * b + r] = acc[i];
        }
    }
    __syncthreads();
    for (int e = tid; e < ti.n * cw; e += kThreads) {
        const int t = e / cw, c = e - t * cw;
        float v = res[t * ldr + c];
        for (int k = 1; k < kparts; ++k)
            v += res[(k * kTileM + t) * ldr + c];
        dst[(size_t)t * dst_ld + c] = v;
    }
}

// LDS footprint (bf16 elements) of the MFMA shrink: x chunk [kTileM][KC + 8]
// and A chunk [NB * 16][KC + 8]; the 8-element pad per row shifts
// consecutive rows by 4 banks, so the 16-row fragment reads do not conflict.
template <int NB, int KC>
struct ShrinkLds {
    static constexpr int kLd = KC + 8;
    static constexpr int kX = kTileM * kLd;
    static constexpr int kElems = kX + NB * 16 * kLd;
};

// MFMA path (bf16).  The workgroup walks its K chunk in pieces of KC
// elements.  All 256 threads load a piece of the x tile [64 x KC] and of the
// A tile [NB*16 x KC] as coalesced 16-byte runs (whole rows of KC elements),
// stage them in LDS, and while the MFMAs consume one piece from LDS the
// loads of the next piece are in flight.  Wave w owns the 16-token block w;
// each 32-element step is one v_mfma_f32_16x16x32_bf16 per 16-column block,
// x rows as the M operand and A rows as the N operand.  The wave writes its
// 16 x cw block of the result directly.
template <int NB, int KC, bool GATHER>
__device__ void shrink_mfma(const ShrinkArgs& a, const TileInfo& ti, int k0, int k1, int c0,
                            int c1, float* dst, int64_t dst_ld, uint16_t* lds)
{
    typedef ShrinkLds<NB, KC> Lay;
    constexpr int PIECES = KC / 8;  // 16-byte pieces per row
    constexpr int XR = kTileM * PIECES / kThreads;
    constexpr int APieces = NB * 16 * PIECES;
    constexpr int AR = (APieces + kThreads - 1) / kThreads;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, q = lane >> 4;
    uint16_t* lx = lds;
    uint16_t* la = lds + Lay::kX;
    const RowMap<GATHER> xm{a.r.rows, ti.t0, ti.n, a.r.nrows};
    // the group's A blocks in the tiled layout; blocks past the group read as zero
    const uint16_t* Ab =
        reinterpret_cast<const uint16_t*>(a.A) + (size_t)ti.slot * a.a_slot + (size_t)(c0 >> 4) * 16 * a.in_f;
    const Buf xb = xm.buf(reinterpret_cast<const uint16_t*>(a.x), a.ldx);  // rows past the tile read as zero
    const Buf ab(Ab, (uint32_t)(((c1 - c0 + 15) >> 4) * 16 * a.in_f * 2));
    const int nchunks = (k1 - k0 + KC - 1) / KC;

    uint4 xs[XR], as[AR];
    // the rows of this thread's x pieces, the same for every chunk
    uint32_t xrow[XR];
#pragma unroll
    for (int i = 0; i < XR; ++i)
        xrow[i] = xm((tid + kThreads * i) / PIECES);
    auto gload = [&](int ch) {
        const int kb = k0 + ch * KC;
#pragma unroll
        for (int i = 0; i < XR; ++i) {
            const int p = tid + kThreads * i, k = kb + 8 * (p % PIECES);
            xs[i] = xb.ld16(k < k1 ? (uint32_t)(xrow[i] * a.ldx + k) * 2 : kOOB);
        }
        // A piece p: row p % 16 of block p / (16 PIECES), K piece (p / 16) % PIECES;
        // 16 consecutive threads read one contiguous 256-byte piece group
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            const int p = tid + kThreads * i, rr = p & 15, pc = (p >> 4) % PIECES, nb = p / (16 * PIECES);
            const int k = kb + 8 * pc;
            as[i] = ab.ld16((p < APieces && k < k1)
                                ? (uint32_t)(((nb * (a.in_f >> 3) + (k >> 3)) * 16 + rr) * 8) * 2
                                : kOOB);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < XR; ++i) {
            const int p = tid + kThreads * i;
            *reinterpret_cast<uint4*>(lx + (p / PIECES) * Lay::kLd + 8 * (p % PIECES)) = xs[i];
        }
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            const int p = tid + kThreads * i, rr = p & 15, pc = (p >> 4) % PIECES, nb = p / (16 * PIECES);
            if (p < APieces)
                *reinterpret_cast<uint4*>(la + (nb * 16 + rr) * Lay::kLd + 8 * pc) = as[i];
        }
    };

    f32x4_t acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const bool active = 16 * w < ti.n;

    gload(0);
    lstore();
    __syncthreads();
    for (int ch = 0; ch < nchunks; ++ch) {
        if (ch + 1 < nchunks)
            gload(ch + 1);
        if (active) {
#pragma unroll
            for (int st = 0; st < KC / 32; ++st) {
                const int kk = 32 * st + 8 * q;
                const bf16x8_t xv =
                    __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(lx + (16 * w + l16) * Lay::kLd + kk));
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const bf16x8_t av = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const uint4*>(la + (nb * 16 + l16) * Lay::kLd + kk));
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, av, acc[nb], 0, 0, 0);
                }
            }
        }
        __syncthreads();
        if (ch + 1 < nchunks) {
            lstore();
            __syncthreads();
        }
    }
    if (!active)
        return;
    // D[i][j]: lane holds column j = lane%16 and rows 4*(lane/16) + r
    const int cw = c1 - c0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int c = nb * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * w + 4 * q + r;
            if (t < ti.n && c < cw)
                dst[(size_t)t * dst_ld + c] = acc[nb][r];
        }
    }
}

// Kernel variants: kMixed picks the path per tile (VALU for groups of at most
// valu_max tokens, MFMA otherwise); kMfmaOnly / kValuOnly compile one path
// only, which keeps the register budget of that path alone.
enum { kMixed = 0, kMfmaOnly = 1, kValuOnly = 2 };

// One workgroup per (token tile, K split, column group).  With one split the
// result is u itself; with S splits each workgroup writes its split's slab
// and the sum over splits is taken later, in split order, by the expand or
// by reduce_slabs — there is no cross-workgroup synchronisation.
template <typename T, int NB, int MODE, bool GATHER>
__global__ __launch_bounds__(kThreads) void shrink_kernel(ShrinkArgs a)
{
    constexpr int KC = kShrinkKC;
    constexpr bool kHasValu = MODE != kValuOnly ? MODE == kMixed : true;
    constexpr bool kHasMfma = MODE != kValuOnly;
    constexpr int kValuRes = 4 * kTileM * 16 * 4;  // shrink_valu's res
    constexpr int kValuLds = kValuRes + 8 * kValuChunk * 8 * (int)sizeof(T);  // + its x chunk
    constexpr int kLdsBytes = (kHasMfma ? ShrinkLds<NB, KC>::kElems * 2 : 0) > (kHasValu ? kValuLds : 0)
                                  ? (kHasMfma ? ShrinkLds<NB, KC>::kElems * 2 : 0)
                                  : (kHasValu ? kValuLds : 0);
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes > 0 ? kLdsBytes : 16];
    // the arguments the data addresses need, in scalar registers before the
    // tile lookup, so that they load in the same round as its own arguments
    asm volatile("" ::"s"(a.x), "s"(a.ldx), "s"(a.A), "s"(a.a_slot), "s"(a.out), "s"(a.slab), "s"(a.in_f), "s"(a.C),
                 "s"(a.S), "s"(a.kc), "s"(a.nz), "s"(a.cb), "s"(a.valu_max), "s"(a.r.G), "s"(a.r.end), "s"(a.r.L),
                 "s"(a.r.kr));

    int z, s, tile;
    if (a.xmap_on) {
        const uint32_t e = a.xmap[blockIdx.x];
        if (e == kNoEntry)
            return;
        tile = (int)(e >> 16);
        s = (int)((e >> 8) & 0xFFu);
        z = (int)(e & 0xFFu);
    } else {
        const int lin = blockIdx.x;
        z = lin % a.nz;
        s = (lin / a.nz) % a.S;
        tile = lin / (a.nz * a.S);
    }
    TileInfo ti;
    if (!locate_tile<kTileM, false>(a.r, tile, ti))
        return;
    const int k0 = s * a.kc, k1 = min(k0 + a.kc, a.in_f);
    const int c0 = z * a.cb, c1 = min(c0 + a.cb, a.C);
    float* dst = a.out + (size_t)s * a.slab + (size_t)ti.t0 * a.C + c0;

    if constexpr (MODE == kMfmaOnly) {
        shrink_mfma<NB, KC, GATHER>(a, ti, k0, k1, c0, c1, dst, a.C, reinterpret_cast<uint16_t*>(smem));
        return;
    }
    if constexpr (MODE == kMixed) {
        if (ti.glen > a.valu_max) {
            shrink_mfma<NB, KC, GATHER>(a, ti, k0, k1, c0, c1, dst, a.C, reinterpret_cast<uint16_t*>(smem));
            return;
        }
    }
    if constexpr (kHasValu)
        shrink_valu<T, GATHER>(a, ti, k0, k1, c0, c1, dst, a.C, reinterpret_cast<float*>(smem),
                       reinterpret_cast<T*>(smem + kValuRes));
}

// u = sum of the S slabs, in split order; 4 floats per thread.
__global__ __launch_bounds__(kThreads) void reduce_slabs(const float* P, int64_t slab4, int S,
                                                         float* u, int64_t n4)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n4)
        return;
    const float4* p = reinterpret_cast<const float4*>(P) + i;
    float4 acc = p[0];
    for (int s = 1; s < S; ++s) {
        const float4 v = p[(int64_t)s * slab4];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    reinterpret_cast<float4*>(u)[i] = acc;
}

// ---------------------------------------------------------------------------
// long-segment shrink (bf16, MFMA)
//
// One 512-thread workgroup owns a piece of at most 64 consecutive tokens of
// one group, one group of at most 16 NB columns of u, and one K range
// [kb, ke) (all of K unless the launch splits K).  Its 8 waves split the K
// range; wave w streams the piece's 64 rows of x over its K share in chunks
// of 64 K values, D chunks ahead of the matrix instructions, with no barrier
// in the loop.  A chunk is eight loads of whole 128-byte lines (8 rows x 128
// B each; the matrix layout would split every line over two loads, which
// streams about 20 % slower on this part) into registers, written into the
// wave's own 8 KB LDS region with the 16-byte pieces rotated by row (so that
// the line writes and the fragment reads spread over the banks), from which
// the wave reads the M operands of its four 16-row blocks.  The A fragments
// (16 columns x 32 K values each, one contiguous 1 KB run of the tiled
// layout: the N operands) come straight into registers.  Per 32-element step
// the wave runs 4 NB v_mfma_f32_16x16x32_bf16.  K positions past the range
// and rows past the piece read zero through the buffer bounds.  The 8
// partial tiles are then
// added in LDS in a fixed tree order ((w0 + w4) + (w2 + w6)) + ((w1 + w5) +
// (w3 + w7)), so the result is deterministic, and written to u, or to slab s
// of the workspace when K is split.
//
// Pieces: each group is cut into n_g near-equal pieces of at most 64 tokens;
// n_g is raised above ceil(len / 64) while that still leaves one workgroup
// per compute unit, so a batch of a few long groups spreads over the whole
// chip.  Workgroup b runs on XCD b % 8 and the pieces are dealt to the XCDs
// in contiguous runs, so a group's A rows are fetched into few L2s.
constexpr int kLsWaves = 8;
constexpr int kLsThreads = 64 * kLsWaves;
constexpr int kLdWaveBytes = 64 * 128;  // a wave's LDS region: 64 rows x 128 B

// byte offset in a wave's region of 16-byte piece p (0..7) of row r
__device__ __forceinline__ int ld_slot(int r, int p) { return r * 128 + ((p ^ (r & 7)) << 4); }
constexpr int kLsRows = 64;               // tokens of a piece: four 16-row MFMA blocks
constexpr int kLsKUnit = 32 * kLsWaves;   // K split granularity: one step of every wave

struct LongShrinkArgs {
    const uint16_t* x;
    int64_t ldx;
    const uint16_t* A;  // [L][a_slot] in the tiled A layout
    int64_t a_slot;
    float* out;         // u (S == 1) or slab s at out + s * slab, each [end][C]
    int64_t slab;
    int in_f, C;
    int kc;       // K range of one split (a multiple of kLsKUnit)
    int zs;       // column groups x K splits
    int S;        // K splits
    int cb;       // columns per column group (a multiple of 16)
    int per_xcd;  // pieces dealt to each XCD
    int pieces;   // pieces in total
    RouteArgs r;
    int k_piece0[LORA_MAX_HOST_GROUPS + 1];  // host routing: first piece of each group
};

// The piece: with the host copy of the routing, group g holds pieces
// [k_piece0[g], k_piece0[g + 1]) of near-equal length; without it, 64-token
// tiles found by a scan over the device arrays.
__device__ __forceinline__ bool locate_piece(const LongShrinkArgs& a, int piece, TileInfo& ti)
{
    if (!a.r.kr)
        return locate_tile<kLsRows, false>(a.r, piece, ti);
    const int lane = threadIdx.x & 63;
    const bool in = lane < a.r.G;
    const int p0_l = in ? a.k_piece0[lane] : 0;
    const int p1_l = in ? a.k_piece0[lane + 1] : 0;
    const int gs_l = in ? a.r.k_offs[lane] : 0;
    const int ge_l = in ? a.r.k_offs[lane + 1] : 0;
    const int id_l = in ? a.r.k_ids[lane] : -1;
    const unsigned long long hit = __ballot(in && piece < p1_l);
    if (!hit)
        return false;
    const int g = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
    const int p0 = __builtin_amdgcn_readlane(p0_l, g), np = __builtin_amdgcn_readlane(p1_l, g) - p0;
    const int gs = __builtin_amdgcn_readlane(gs_l, g), len = __builtin_amdgcn_readlane(ge_l, g) - gs;
    const int j = piece - p0;
    const int t0 = gs + (int)(((int64_t)len * j) / np);
    const int t1 = gs + (int)(((int64_t)len * (j + 1)) / np);
    ti.g = g;
    ti.t0 = t0;
    ti.n = t1 - t0;
    ti.glen = len;
    ti.slot = __builtin_amdgcn_readlane(id_l, g);
    return ti.slot >= 0 && ti.slot < a.r.L;
}

template <int NB>
struct LongShrinkLds {
    static constexpr int kLd = 16 * NB + 4;          // padded row of a partial tile (floats)
    static constexpr int kTile = kLsRows * kLd;      // one wave's partial tile
    static constexpr int kFloats = 4 * kTile;        // four tiles in flight in the tree
    // the waves' regions during the K loop, the tree after it
    static constexpr int kBytes = kLsWaves * kLdWaveBytes > kFloats * 4 ? kLsWaves * kLdWaveBytes : kFloats * 4;
};

template <int NB, int D, bool NTX, bool GATHER>
__global__ __launch_bounds__(kLsThreads) void shrink_long_kernel(LongShrinkArgs a)
{
    typedef LongShrinkLds<NB> Lay;
    __shared__ __attribute__((aligned(16))) char smem[Lay::kBytes];
    float* red = reinterpret_cast<float*>(smem);
    asm volatile("" ::"s"(a.x), "s"(a.ldx), "s"(a.A), "s"(a.a_slot), "s"(a.out), "s"(a.slab), "s"(a.in_f),
                 "s"(a.C), "s"(a.kc), "s"(a.zs), "s"(a.S), "s"(a.cb), "s"(a.per_xcd), "s"(a.pieces), "s"(a.r.G),
                 "s"(a.r.kr));
    const int b = blockIdx.x;
    const int i = b / kXcds;
    const int zsi = i % a.zs;
    const int piece = (b % kXcds) * a.per_xcd + i / a.zs;
    if (piece >= a.pieces)
        return;
    TileInfo ti;
    if (!locate_piece(a, piece, ti))
        return;
    const int z = zsi / a.S, s = zsi - z * a.S;
    const int c0 = z * a.cb, cw = min(a.cb, a.C - c0);
    const int kb = s * a.kc, ke = min(kb + a.kc, a.in_f);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int lr = lane >> 3, lp = lane & 7;  // whole-line layout: row lr + 8 i, 16-byte piece lp
    char* region = smem + w * kLdWaveBytes;
    const int kw = a.kc / kLsWaves;
    const int k0 = kb + w * kw, k1 = min(k0 + kw, ke);
    const int nch = k1 > k0 ? (k1 - k0 + 63) >> 6 : 0;

    const RowMap<GATHER> xm{a.r.rows, ti.t0, ti.n, a.r.nrows};
    // with one column group x is read once: non-temporal (NTX)
    typedef typename std::conditional<NTX, StreamBuf, Buf>::type XBuf;
    const XBuf xb(xm.buf(a.x, a.ldx));
    uint32_t xro[8];
#pragma unroll
    for (int i8 = 0; i8 < 8; ++i8)
        xro[i8] = (uint32_t)(xm(lr + 8 * i8) * a.ldx) * 2;
    const Buf ab(a.A + (size_t)ti.slot * a.a_slot + (size_t)(c0 >> 4) * 16 * a.in_f,
                 (uint32_t)(((cw + 15) >> 4) * 16 * a.in_f * 2));
    const uint32_t ablk = (uint32_t)(16 * a.in_f) * 2;

    f32x4_t acc[4][NB];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 xs[D][8], as[D][2][NB];
    auto load = [&](int ch, uint4(&xv)[8], uint4(&av)[2][NB]) {
        const int kx = k0 + 64 * ch + 8 * lp;
        const bool okx = kx < k1;
#pragma unroll
        for (int i8 = 0; i8 < 8; ++i8)
            xv[i8] = xb.ld16(okx ? xro[i8] + (uint32_t)kx * 2 : kOOB);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kk = k0 + 64 * ch + 32 * h + 8 * q;
            const uint32_t ao = (uint32_t)(((kk >> 3) * 16 + l16) * 16);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                av[h][nb] = ab.ld16(kk < k1 ? nb * ablk + ao : kOOB);
        }
    };
    // the prologue issues the chunks in slot order too, so that at the loop
    // head slot j's loads are as old along both incoming edges
#pragma unroll
    for (int j = 0; j < D; ++j) {
        load(j, xs[j], as[j]);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int base = 0; base < nch; base += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            // whole lines into the wave's region, then the M operands out of it
#pragma unroll
            for (int i8 = 0; i8 < 8; ++i8)
                *reinterpret_cast<uint4*>(region + ld_slot(lr + 8 * i8, lp)) = xs[j][i8];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint4 xf = *reinterpret_cast<const uint4*>(region + ld_slot(16 * m + l16, 4 * h + q));
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, xf), __builtin_bit_cast(bf16x8_t, as[j][h][nb]), acc[m][nb],
                            0, 0, 0);
                }
            load(base + D + j, xs[j], as[j]);
            // keep each chunk's reload right after its matrix instructions:
            // left alone, the scheduler sinks every reload to the end of the
            // body and the loop head then waits for all of them
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();  // every wave is done with its region before the tree reuses it

    // D of block (m, nb): lane holds column 16 nb + l16 of rows 16 m + 4 q + r
    auto put = [&](int t) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    red[t * Lay::kTile + (16 * m + 4 * q + r) * Lay::kLd + 16 * nb + l16] = acc[m][nb][r];
    };
    auto add = [&](int t) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[m][nb][r] += red[t * Lay::kTile + (16 * m + 4 * q + r) * Lay::kLd + 16 * nb + l16];
    };
    if (w >= 4)
        put(w - 4);
    __syncthreads();
    if (w < 4)
        add(w);
    __syncthreads();
    if (w == 2 || w == 3)
        put(w - 2);
    __syncthreads();
    if (w < 2)
        add(w);
    __syncthreads();
    if (w == 1)
        put(0);
    __syncthreads();
    if (w == 0) {
        add(0);
        put(0);
    }
    __syncthreads();
    // rows [0, n) x columns [0, cw) of the sum, four floats per thread
    float* dst = a.out + (size_t)s * a.slab + (size_t)ti.t0 * a.C + c0;
    const int c4 = cw >> 2;
    for (int e = tid; e < ti.n * c4; e += kLsThreads) {
        const int row = e / c4, c = e - row * c4;
        *reinterpret_cast<float4*>(dst + (size_t)row * a.C + 4 * c) =
            *reinterpret_cast<const float4*>(red + row * Lay::kLd + 4 * c);
    }
}

// Zero n 16-byte words (slot reset; a kernel rather than a memset so that
// it can be recorded in a HIP graph).
__global__ __launch_bounds__(kThreads) void zero_words(uint4* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        p[i] = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// expand

struct ExpandArgs {
    const void* bias;  // [L][out_f] per-adapter bias added in the epilogue, or null
    const float* u;  // slab s at u + s * slab, each [end][C]
    int64_t slab;
    int S;
    const void* B;  // [L][out_f][R]
    void* y;
    int64_t ldy;
    int C, R, n_s, out_f;
    int soff[5];  // slice offsets, soff[n_s] = out_f
    int ft;       // feature tile (divides every slice width)
    int n_ftiles;
    int valu_max;  // tiles with at most this many tokens take the VALU path
    RouteArgs r;
};

__device__ __forceinline__ int slice_of(const ExpandArgs& a, int f)
{
    int s = 0;
#pragma unroll
    for (int i = 1; i < 4; ++i)
        if (i < a.n_s && f >= a.soff[i])
            s = i;
    return s;
}

// Sum the S slabs of u for the tile's tokens and one slice's R columns into
// LDS us[n][R] (fp32).  With many items per workgroup each thread adds all S
// slabs of its items; with few items (decode tiles) P groups of threads add
// interleaved subsets of the slabs and the P partial sums are then added in
// group order.  The order depends only on (n, R, S): results are
// deterministic.
__device__ __forceinline__ void stage_u(const ExpandArgs& a, const TileInfo& ti, int ucol0,
                                        float* us, float4* part)
{
    const int r4 = a.R >> 2;
    const int NI = ti.n * r4;
    const float* base = a.u + (size_t)ti.t0 * a.C + ucol0;
    const int tid = threadIdx.x;
    const int P = (a.S > 1 && 2 * NI <= kThreads) ? min(kThreads / NI, a.S) : 1;
    if (P == 1) {
        for (int e = tid; e < NI; e += kThreads) {
            const int i = e / r4, j = (e - i * r4) * 4;
            const float* p = base + (size_t)i * a.C + j;
            float4 acc = *reinterpret_cast<const float4*>(p);
#pragma unroll 4
            for (int sl = 1; sl < a.S; ++sl) {
                const float4 v = *reinterpret_cast<const float4*>(p + (size_t)sl * a.slab);
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
            }
            *reinterpret_cast<float4*>(us + i * a.R + j) = acc;
        }
        return;
    }
    if (tid < P * NI) {
        const int e = tid % NI, g = tid / NI;
        const int i = e / r4, j = (e - i * r4) * 4;
        const float* p = base + (size_t)i * a.C + j;
        float4 acc = *reinterpret_cast<const float4*>(p + (size_t)g * a.slab);
#pragma unroll 8
        for (int sl = g + P; sl < a.S; sl += P) {
            const float4 v = *reinterpret_cast<const float4*>(p + (size_t)sl * a.slab);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        part[g * NI + e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < NI; e += kThreads) {
        float4 acc = part[e];
        for (int g = 1; g < P; ++g) {
            const float4 v = part[g * NI + e];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        const int i = e / r4, j = (e - i * r4) * 4;
        *reinterpret_cast<float4*>(us + i * a.R + j) = acc;
    }
}

// stage_u for a rank R known at compile time (the MFMA expands), with the
// same summation order.  The loads are batched so that a thread waits once
// per slab, not once per slab and item: with one group (long tiles) the
// slab loop is outside and each pass loads the thread's items of one slab
// together (R / 16 of them for a full tile); with P groups each thread
// loads up to four of its slabs at a time.  The generic version's loop
// waited on every load before issuing the next, a chain of items x slabs
// round trips for a full tile.
template <int R>
__device__ __forceinline__ void stage_u_r(const ExpandArgs& a, const TileInfo& ti, int ucol0, float* us,
                                          float4* part)
{
    constexpr int r4 = R / 4;
    constexpr int kItems = (kTileM * r4 + kThreads - 1) / kThreads;  // items of a thread in a full tile
    const int NI = ti.n * r4;
    const float* base = a.u + (size_t)ti.t0 * a.C + ucol0;
    const int tid = threadIdx.x;
    const int P = (a.S > 1 && 2 * NI <= kThreads) ? min(kThreads / NI, a.S) : 1;
    if (P == 1) {
        const float* src[kItems];
        bool ok[kItems];
        float4 acc[kItems];
        // an item past the tile reads the tile's first row (the workgroup
        // has at least one token) and is not stored: no branch between loads
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int e = tid + kThreads * k, i = e / r4, j = (e - i * r4) * 4;
            ok[k] = e < NI;
            src[k] = ok[k] ? base + (size_t)i * a.C + j : base;
            acc[k] = *reinterpret_cast<const float4*>(src[k]);
        }
        for (int sl = 1; sl < a.S; ++sl) {
            float4 v[kItems];
#pragma unroll
            for (int k = 0; k < kItems; ++k)
                v[k] = *reinterpret_cast<const float4*>(src[k] + (size_t)sl * a.slab);
#pragma unroll
            for (int k = 0; k < kItems; ++k) {
                acc[k].x += v[k].x;
                acc[k].y += v[k].y;
                acc[k].z += v[k].z;
                acc[k].w += v[k].w;
            }
        }
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const int e = tid + kThreads * k, i = e / r4, j = (e - i * r4) * 4;
            if (ok[k])
                *reinterpret_cast<float4*>(us + i * R + j) = acc[k];
        }
        return;
    }
    if (tid < P * NI) {
        const int e = tid % NI, g = tid / NI;
        const int i = e / r4, j = (e - i * r4) * 4;
        const float* p = base + (size_t)i * a.C + j;
        float4 acc = *reinterpret_cast<const float4*>(p + (size_t)g * a.slab);
        for (int sl = g + P; sl < a.S; sl += 4 * P) {
            float4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)  // past the last slab: the last one again, not added
                v[k] = *reinterpret_cast<const float4*>(p + (size_t)min(sl + k * P, a.S - 1) * a.slab);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (sl + k * P < a.S) {
                    acc.x += v[k].x;
                    acc.y += v[k].y;
                    acc.z += v[k].z;
                    acc.w += v[k].w;
                }
            }
        }
        part[g * NI + e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < NI; e += kThreads) {
        float4 acc = part[e];
        for (int g = 1; g < P; ++g) {
            const float4 v = part[g * NI + e];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        const int i = e / r4, j = (e - i * r4) * 4;
        *reinterpret_cast<float4*>(us + i * R + j) = acc;
    }
}

// MFMA path (bf16).  Wave w owns tokens 16w .. 16w+15 of the tile and walks
// the feature tile in pairs of 16-feature MFMA blocks.  For each 16 ranks one
// v_mfma_f32_16x16x32_bf16 per block computes B·u with K = 32 = 16 ranks of
// the high bf16 half of u followed by the same 16 ranks of its low half
// (u = hi + lo to ~2^-17 relative), so u keeps fp32 precision while the
// products run on the bf16 matrix cores.  B rows are the M operand
// (features) and u the N operand (tokens).  The M rows of block h of pair p
// are permuted to features 32p + 8(i/4) + 4h + i%4, so that lane (token j,
// group q) holds features 32p + 8q .. 32p + 8q + 7 across the two
// accumulators, and y is the C operand.
//
// y and B move through LDS: the workgroup loads its [64 x ft] tile of y and
// its [ft x R] tile of B with coalesced 16-byte runs (whole 128-byte lines),
// the waves read their MFMA operands from LDS and write the results back
// into the y tile in place, and the tile is stored with the same coalesced
// runs.  Reading y in the MFMA layout directly would split every line over
// two instructions (16 rows x 64 bytes each), and every wave would fetch all
// of B.  The 16-byte chunks of each B row are XOR-swizzled by bits of the
// row (b_swizzle) so that a fragment read, 16 rows of one chunk column,
// touches each LDS bank slot at most twice.  y, B and u loads all go out
// before the first wait.
constexpr int kYLd = kExpandCols + 8;  // padded LDS row of the y tile (bf16 elements)

template <int NH>
__device__ __forceinline__ int b_swizzle(int f)
{
    if constexpr (NH == 1)
        return (f >> 3) & 1;
    else if constexpr (NH == 2)
        return ((f >> 1) & 1) | (((f >> 3) & 1) << 1);
    else
        return (f & 1) | (((f >> 1) & 1) << 1) | (((f >> 3) & 1) << 2);
}

// The adapter's bias for the 8 features a lane holds in the MFMA layout
// (acc0: f .. f+3, acc1: f+4 .. f+7), added to the accumulators ([MAX-lora]
// LoRAType BIAS: a bias attached to B).  b holds the 8 bf16 values.
__device__ __forceinline__ void add_bias8(uint4 b, f32x4_t& acc0, f32x4_t& acc1)
{
    acc0[0] += bf2f(b.x & 0xFFFFu);
    acc0[1] += bf2f(b.x >> 16);
    acc0[2] += bf2f(b.y & 0xFFFFu);
    acc0[3] += bf2f(b.y >> 16);
    acc1[0] += bf2f(b.z & 0xFFFFu);
    acc1[1] += bf2f(b.z >> 16);
    acc1[2] += bf2f(b.w & 0xFFFFu);
    acc1[3] += bf2f(b.w >> 16);
}

// The MFMA expands stage the tile's bias row (ft bf16 values) in LDS: the
// first ft / 8 threads load one 16-byte piece each together with the y and B
// loads (without a bias the size is zero and the load reads zero), store it
// with the other LDS tiles, and the epilogue reads a lane's 8 values there.
__device__ __forceinline__ uint4 load_bias_piece(const ExpandArgs& a, const TileInfo& ti, int f0)
{
    const Buf bb(reinterpret_cast<const uint16_t*>(a.bias) + (size_t)ti.slot * a.out_f + f0,
                 a.bias ? (uint32_t)(a.ft * 2) : 0u);
    return bb.ld16((int)threadIdx.x < (a.ft >> 3) ? (uint32_t)threadIdx.x * 16 : kOOB);
}

__device__ __forceinline__ void store_bias_piece(const ExpandArgs& a, uint16_t* bls, uint4 v)
{
    if (a.bias && (int)threadIdx.x < (a.ft >> 3))
        *reinterpret_cast<uint4*>(bls + 8 * threadIdx.x) = v;
}

__device__ __forceinline__ void add_bias8_lds(const ExpandArgs& a, const uint16_t* bls, int f, f32x4_t& acc0,
                                              f32x4_t& acc1)
{
    if (a.bias)
        add_bias8(*reinterpret_cast<const uint4*>(bls + f), acc0, acc1);
}

template <int NH, bool GATHER>
__device__ __forceinline__ void expand_mfma(const ExpandArgs& a, const TileInfo& ti, int f0,
                                            const Buf& yb, const RowMap<GATHER>& ym, int ucol0, float* us,
                                            float4* part, uint16_t* ylds, uint16_t* blds, uint16_t* bls)
{
    const StreamBuf ybn(yb);  // y is read and written once: non-temporal
    static_assert(NH == 1 || NH == 2 || NH == 4, "B chunk swizzle needs a power-of-two chunk count");
    constexpr int R = 16 * NH;
    constexpr int NCH = R / 8;                      // 16-byte chunks per B row
    constexpr int kMaxPairs = kExpandCols / 32;
    constexpr int BR = kExpandCols * NCH / kThreads;  // B chunks per thread for the largest tile
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, q = lane >> 4;
    const int np = a.ft >> 5;
    const int pieces = a.ft >> 3;  // 16-byte pieces per row of the y tile
    const int mrow = 8 * (l16 >> 2) + (l16 & 3);  // permuted M row of block 0
    const Buf bb(reinterpret_cast<const uint16_t*>(a.B) + ((size_t)ti.slot * a.out_f + f0) * R,
                 (uint32_t)(a.ft * R * 2));

    // coalesced y tile: 64 rows x `pieces` pieces, kMaxPairs rounds of 256 pieces
    // (per-token routing keeps each piece's buffer row for the store)
    uint32_t yrow[GATHER ? kMaxPairs : 1];
    if constexpr (GATHER) {
#pragma unroll
        for (int i = 0; i < kMaxPairs; ++i)
            yrow[i] = ym((tid + kThreads * i) / pieces);
    }
    auto yrow_of = [&](int i, int row) -> uint32_t {
        if constexpr (GATHER)
            return yrow[i];
        else
            return (uint32_t)row;
    };
    uint4 yraw[kMaxPairs];
#pragma unroll
    for (int i = 0; i < kMaxPairs; ++i) {
        const int p = tid + kThreads * i, row = p / pieces, pc = p - row * pieces;
        yraw[i] = ybn.ld16(i < np ? (uint32_t)(yrow_of(i, row) * a.ldy + f0 + 8 * pc) * 2 : kOOB);
    }
    // coalesced B tile: ft rows x NCH chunks (past the tile: kOOB)
    uint4 braw[BR];
#pragma unroll
    for (int i = 0; i < BR; ++i) {
        const int p = tid + kThreads * i;
        braw[i] = bb.ld16(p < a.ft * NCH ? (uint32_t)p * 16 : kOOB);
    }
    const uint4 bpiece = load_bias_piece(a, ti, f0);
    // u next: its loads go out before the wait on y and B
    stage_u_r<R>(a, ti, ucol0, us, part);
#pragma unroll
    for (int i = 0; i < kMaxPairs; ++i) {
        if (i < np) {
            const int p = tid + kThreads * i, row = p / pieces, pc = p - row * pieces;
            *reinterpret_cast<uint4*>(ylds + row * kYLd + 8 * pc) = yraw[i];
        }
    }
    store_bias_piece(a, bls, bpiece);
#pragma unroll
    for (int i = 0; i < BR; ++i) {
        const int p = tid + kThreads * i, f = p / NCH, c = p % NCH;
        if (p < a.ft * NCH)
            *reinterpret_cast<uint4*>(blds + f * R + 8 * (c ^ b_swizzle<NH>(f))) = braw[i];
    }
    __syncthreads();

    if (16 * w < ti.n) {
        // u fragments: lanes q<2 carry hi(u[t][16kh+8q..]), lanes q>=2 lo(u[t][16kh+8(q-2)..])
        const int t = 16 * w + l16;
        bf16x8_t uf[NH];
#pragma unroll
        for (int kh = 0; kh < NH; ++kh) {
            const float* up = us + min(t, ti.n - 1) * R + 16 * kh + 8 * (q & 1);
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v0 = up[2 * e], v1 = up[2 * e + 1];
                uint32_t hi = f2bf_pair(v0, v1);
                if (q >= 2)
                    hi = f2bf_pair(v0 - bf2f(hi & 0xFFFFu), v1 - bf2f(hi >> 16));
                pk[e] = hi;
            }
            uf[kh] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
        }

#pragma unroll
        for (int p = 0; p < kMaxPairs; ++p) {
            if (p < np) {
                uint4* cell = reinterpret_cast<uint4*>(ylds + t * kYLd + 32 * p + 8 * q);
                const uint4 yv = *cell;
                f32x4_t acc0 = {bf2f(yv.x & 0xFFFFu), bf2f(yv.x >> 16), bf2f(yv.y & 0xFFFFu), bf2f(yv.y >> 16)};
                f32x4_t acc1 = {bf2f(yv.z & 0xFFFFu), bf2f(yv.z >> 16), bf2f(yv.w & 0xFFFFu), bf2f(yv.w >> 16)};
                add_bias8_lds(a, bls, 32 * p + 8 * q, acc0, acc1);
#pragma unroll
                for (int kh = 0; kh < NH; ++kh) {
                    const int c = 2 * kh + (q & 1);
                    const int f0r = 32 * p + mrow, f1r = f0r + 4;
                    const uint4 b0 =
                        *reinterpret_cast<const uint4*>(blds + f0r * R + 8 * (c ^ b_swizzle<NH>(f0r)));
                    const uint4 b1 =
                        *reinterpret_cast<const uint4*>(blds + f1r * R + 8 * (c ^ b_swizzle<NH>(f1r)));
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b0), uf[kh], acc0,
                                                                  0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b1), uf[kh], acc1,
                                                                  0, 0, 0);
                }
                uint4 o;
                o.x = f2bf_pair(acc0[0], acc0[1]);
                o.y = f2bf_pair(acc0[2], acc0[3]);
                o.z = f2bf_pair(acc1[0], acc1[1]);
                o.w = f2bf_pair(acc1[2], acc1[3]);
                *cell = o;
            }
        }
    }
    __syncthreads();
    // rows past the tile's tokens drop their stores (offset past the resource)
#pragma unroll
    for (int i = 0; i < kMaxPairs; ++i) {
        if (i < np) {
            const int p = tid + kThreads * i, row = p / pieces, pc = p - row * pieces;
            ybn.st16((uint32_t)(yrow_of(i, row) * a.ldy + f0 + 8 * pc) * 2,
                    *reinterpret_cast<const uint4*>(ylds + row * kYLd + 8 * pc));
        }
    }
}

// MFMA path for ranks 32 and 64: B through LDS, y in registers.  The
// workgroup loads its [ft x R] tile of B with coalesced 16-byte runs into
// LDS (chunks XOR-swizzled per row, as in expand_mfma) and the waves read
// their M-operand fragments from there; y stays in registers in the MFMA
// layout as in expand_mfma_reg.  Reading B fragments straight from memory
// touches 16 rows per instruction and leans on L1 reuse across the rank
// steps and the four waves, which breaks down once several workgroups share
// a CU; an LDS tile of y as well would cut the workgroups per CU to one or
// two.  Waves with no token in the tile help with the B tile only.
template <int NH, bool GATHER>
__device__ __forceinline__ void expand_mfma_lb(const ExpandArgs& a, const TileInfo& ti, int f0,
                                               const Buf& yb, const RowMap<GATHER>& ym, int ucol0, float* us,
                                               float4* part, uint16_t* blds, uint16_t* bls)
{
    static_assert(NH == 2 || NH == 4, "B chunk swizzle needs a power-of-two chunk count");
    constexpr int R = 16 * NH;
    constexpr int NCH = R / 8;                        // 16-byte chunks per B row
    constexpr int kMaxPairs = kExpandCols / 32;
    constexpr int BR = kExpandCols * NCH / kThreads;  // B chunks per thread for the largest tile
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, q = lane >> 4;
    const int np = a.ft >> 5;
    const int t = 16 * w + l16;
    const bool tok = t < ti.n;
    const int mrow = 8 * (l16 >> 2) + (l16 & 3);  // permuted M row of block 0
    const Buf bb(reinterpret_cast<const uint16_t*>(a.B) + ((size_t)ti.slot * a.out_f + f0) * R,
                 (uint32_t)(a.ft * R * 2));

    const uint32_t yt = ym(t);  // the buffer row of this lane's token
    uint4 yraw[kMaxPairs];
#pragma unroll
    for (int p = 0; p < kMaxPairs; ++p)
        yraw[p] = yb.ld16((p < np && tok) ? (uint32_t)(yt * a.ldy + f0 + 32 * p + 8 * q) * 2 : kOOB);
    uint4 braw[BR];
#pragma unroll
    for (int i = 0; i < BR; ++i) {
        const int p = tid + kThreads * i;
        braw[i] = bb.ld16(p < a.ft * NCH ? (uint32_t)p * 16 : kOOB);
    }
    const uint4 bpiece = load_bias_piece(a, ti, f0);
    stage_u_r<R>(a, ti, ucol0, us, part);
    store_bias_piece(a, bls, bpiece);
#pragma unroll
    for (int i = 0; i < BR; ++i) {
        const int p = tid + kThreads * i, f = p / NCH, c = p % NCH;
        if (p < a.ft * NCH)
            *reinterpret_cast<uint4*>(blds + f * R + 8 * (c ^ b_swizzle<NH>(f))) = braw[i];
    }
    __syncthreads();
    if (16 * w >= ti.n)
        return;

    // u fragments: lanes q<2 carry hi(u[t][16kh+8q..]), lanes q>=2 lo(u[t][16kh+8(q-2)..])
    bf16x8_t uf[NH];
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) {
        const float* up = us + min(t, ti.n - 1) * R + 16 * kh + 8 * (q & 1);
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v0 = up[2 * e], v1 = up[2 * e + 1];
            uint32_t hi = f2bf_pair(v0, v1);
            if (q >= 2)
                hi = f2bf_pair(v0 - bf2f(hi & 0xFFFFu), v1 - bf2f(hi >> 16));
            pk[e] = hi;
        }
        uf[kh] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }

#pragma unroll
    for (int p = 0; p < kMaxPairs; ++p) {
        if (p < np) {
            const uint4 yv = yraw[p];
            f32x4_t acc0 = {bf2f(yv.x & 0xFFFFu), bf2f(yv.x >> 16), bf2f(yv.y & 0xFFFFu), bf2f(yv.y >> 16)};
            f32x4_t acc1 = {bf2f(yv.z & 0xFFFFu), bf2f(yv.z >> 16), bf2f(yv.w & 0xFFFFu), bf2f(yv.w >> 16)};
            add_bias8_lds(a, bls, 32 * p + 8 * q, acc0, acc1);
#pragma unroll
            for (int kh = 0; kh < NH; ++kh) {
                const int c = 2 * kh + (q & 1);
                const int f0r = 32 * p + mrow, f1r = f0r + 4;
                const uint4 b0 = *reinterpret_cast<const uint4*>(blds + f0r * R + 8 * (c ^ b_swizzle<NH>(f0r)));
                const uint4 b1 = *reinterpret_cast<const uint4*>(blds + f1r * R + 8 * (c ^ b_swizzle<NH>(f1r)));
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b0), uf[kh], acc0,
                                                              0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b1), uf[kh], acc1,
                                                              0, 0, 0);
            }
            uint4 o;
            o.x = f2bf_pair(acc0[0], acc0[1]);
            o.y = f2bf_pair(acc0[2], acc0[3]);
            o.z = f2bf_pair(acc1[0], acc1[1]);
            o.w = f2bf_pair(acc1[2], acc1[3]);
            yb.st16(tok ? (uint32_t)(yt * a.ldy + f0 + 32 * p + 8 * q) * 2 : kOOB, o);
        }
    }
}

// MFMA path with y in registers (ranks 32 to 64, for which LDS tiles of y
// and B would leave one or two workgroups per CU).  Wave w owns tokens
// 16w .. 16w+15 of the tile and walks
// the feature tile in pairs of 16-feature MFMA blocks.  For each 16 ranks one
// v_mfma_f32_16x16x32_bf16 per block computes B·u with K = 32 = 16 ranks of
// the high bf16 half of u followed by the same 16 ranks of its low half
// (u = hi + lo to ~2^-17 relative), so u keeps fp32 precision while the
// products run on the bf16 matrix cores.  B rows are the M operand
// (features) and u the N operand (tokens).  The M rows of block h of pair p
// are permuted to features 32p + 8(i/4) + 4h + i%4, so that lane (token j,
// group q) holds features 32p + 8q .. 32p + 8q + 7 across the two
// accumulators: y is the C operand, read and written as 16-byte runs in the
// MFMA layout itself, and a wave covers 16 rows x 512 contiguous bytes.
// y and (for NH <= 2) B fragments are loaded before u is staged.
template <int NH, bool GATHER>
__device__ __forceinline__ void expand_mfma_reg(const ExpandArgs& a, const TileInfo& ti, int f0,
                                            const Buf& yb, const RowMap<GATHER>& ym, int ucol0, float* us,
                                            float4* part, uint16_t* bls)
{
    constexpr int kMaxPairs = kExpandCols / 32;
    constexpr bool kPrefetchB = NH == 1;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, q = lane >> 4;
    const int np = a.ft >> 5;
    const int t = 16 * w + l16;
    const bool tok = t < ti.n;
    const int mrow = 8 * (l16 >> 2) + (l16 & 3);  // permuted M row of block 0
    const uint16_t* Bb = reinterpret_cast<const uint16_t*>(a.B) + ((size_t)ti.slot * a.out_f + f0) * a.R;

    const uint32_t yt = ym(t);  // the buffer row of this lane's token
    uint4 yraw[kMaxPairs];
#pragma unroll
    for (int p = 0; p < kMaxPairs; ++p)
        yraw[p] = yb.ld16((p < np && tok) ? (uint32_t)(yt * a.ldy + f0 + 32 * p + 8 * q) * 2 : kOOB);
    uint4 bfr[kPrefetchB ? kMaxPairs : 1][2][NH];
    if constexpr (kPrefetchB) {
#pragma unroll
        for (int p = 0; p < kMaxPairs; ++p)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int kh = 0; kh < NH; ++kh)
                    bfr[p][h][kh] = ld16(Bb + (size_t)(min(p, np - 1) * 32 + mrow + 4 * h) * a.R + 16 * kh +
                                         8 * (q & 1));
    }
    const uint4 bpiece = load_bias_piece(a, ti, f0);

    stage_u_r<16 * NH>(a, ti, ucol0, us, part);
    store_bias_piece(a, bls, bpiece);
    __syncthreads();
    if (16 * w >= ti.n)
        return;

    // u fragments: lanes q<2 carry hi(u[t][16kh+8q..]), lanes q>=2 lo(u[t][16kh+8(q-2)..])
    bf16x8_t uf[NH];
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) {
        const float* up = us + min(t, ti.n - 1) * a.R + 16 * kh + 8 * (q & 1);
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v0 = up[2 * e], v1 = up[2 * e + 1];
            uint32_t hi = f2bf_pair(v0, v1);
            if (q >= 2)
                hi = f2bf_pair(v0 - bf2f(hi & 0xFFFFu), v1 - bf2f(hi >> 16));
            pk[e] = hi;
        }
        uf[kh] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }

#pragma unroll
    for (int p = 0; p < kMaxPairs; ++p) {
        if (p < np) {
            const uint4 yv = yraw[p];
            f32x4_t acc0 = {bf2f(yv.x & 0xFFFFu), bf2f(yv.x >> 16), bf2f(yv.y & 0xFFFFu), bf2f(yv.y >> 16)};
            f32x4_t acc1 = {bf2f(yv.z & 0xFFFFu), bf2f(yv.z >> 16), bf2f(yv.w & 0xFFFFu), bf2f(yv.w >> 16)};
            add_bias8_lds(a, bls, 32 * p + 8 * q, acc0, acc1);
#pragma unroll
            for (int kh = 0; kh < NH; ++kh) {
                uint4 b0, b1;
                if constexpr (kPrefetchB) {
                    b0 = bfr[p][0][kh];
                    b1 = bfr[p][1][kh];
                } else {
                    const uint16_t* bp = Bb + (size_t)(p * 32 + mrow) * a.R + 16 * kh + 8 * (q & 1);
                    b0 = ld16(bp);
                    b1 = ld16(bp + 4 * a.R);
                }
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b0), uf[kh], acc0,
                                                              0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b1), uf[kh], acc1,
                                                              0, 0, 0);
            }
            uint4 o;
            o.x = f2bf_pair(acc0[0], acc0[1]);
            o.y = f2bf_pair(acc0[2], acc0[3]);
            o.z = f2bf_pair(acc1[0], acc1[1]);
            o.w = f2bf_pair(acc1[2], acc1[3]);
            yb.st16(tok ? (uint32_t)(yt * a.ldy + f0 + 32 * p + 8 * q) * 2 : kOOB, o);
        }
    }
}

// VALU path (decode-shaped tiles, and every fp32 tile).  Thread (rr, fl) owns
// features f0 + 8 fl .. +8 of rows rr, rr + RP, ... (RP = rows per pass), so
// every y access is a 16-byte run and a wave covers whole row segments.  Row
// passes go two at a time; the first two are loaded before u is staged.  B is
// read 8 ranks at a time and reused for both rows.
template <typename T, bool GATHER>
__device__ __forceinline__ void expand_valu(const ExpandArgs& a, const TileInfo& ti, int f0,
                                            const Buf& yb, const RowMap<GATHER>& ym, int ucol0, float* us,
                                            float4* part)
{
    constexpr int E = sizeof(T);
    const int fgroups = a.ft >> 3;
    const int rp = kThreads / fgroups;
    const int fl = threadIdx.x % fgroups, rr = threadIdx.x / fgroups;
    const int f = f0 + 8 * fl;
    const int npass = (ti.n + rp - 1) / rp;

    typename Vec8<T>::Raw yraw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = rr + i * rp;
        yraw[i] = Vec8<T>::load_raw(yb, row < ti.n ? (uint32_t)(ym(row) * a.ldy + f) * E : kOOB);
    }
    stage_u(a, ti, ucol0, us, part);
    __syncthreads();

    const T* Bb = reinterpret_cast<const T*>(a.B) + ((size_t)ti.slot * a.out_f + f) * a.R;
    for (int p0 = 0; p0 < npass; p0 += 2) {
        if (p0 > 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = rr + (p0 + i) * rp;
                yraw[i] = Vec8<T>::load_raw(yb, row < ti.n ? (uint32_t)(ym(row) * a.ldy + f) * E : kOOB);
            }
        }
        float delta[2][8];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                delta[i][e] = 0.f;
        for (int j0 = 0; j0 < a.R; j0 += 8) {
            float bv[8][8];  // [feature][rank]
#pragma unroll
            for (int ff = 0; ff < 8; ++ff)
                Vec8<T>::load(Bb + (size_t)ff * a.R + j0, bv[ff]);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = rr + (p0 + i) * rp;
                if (row < ti.n) {
                    const float* up = us + row * a.R + j0;
                    float uv[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
                        uv[jj] = up[jj];
#pragma unroll
                    for (int ff = 0; ff < 8; ++ff)
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj)
                            delta[i][ff] = fmaf(bv[ff][jj], uv[jj], delta[i][ff]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = rr + (p0 + i) * rp;
            if (row < ti.n) {
                float out[8], bias[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                Vec8<T>::unpack(yraw[i], out);
                if (a.bias)
                    Vec8<T>::load(reinterpret_cast<const T*>(a.bias) + (size_t)ti.slot * a.out_f + f, bias);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    out[e] += bias[e] + delta[i][e];
                Vec8<T>::store_buf(yb, (uint32_t)(ym(row) * a.ldy + f) * E, out);
            }
        }
    }
}

// One workgroup per (token tile, feature tile); the feature tile lies in one
// slice.  NH = R / 16 when the MFMA path may run (bf16, R <= 64, slice widths
// multiple of 32); NH = 0 builds the VALU path alone.  MODE as for the shrink.
template <typename T, int NH, int MODE, bool GATHER>
__global__ __launch_bounds__(kThreads) void expand_kernel(ExpandArgs a)
{
    extern __shared__ float smem[];
    float* us = smem;                                             // [kTileM][R]
    float4* part = reinterpret_cast<float4*>(us + kTileM * a.R);  // [kThreads]
    // MFMA path, rank 16: y tile [kTileM][kYLd], then B tile [kExpandCols][R];
    // ranks 32 and 64: B tile alone, at ylds
    uint16_t* ylds = reinterpret_cast<uint16_t*>(part + kThreads);
    uint16_t* blds = ylds + kTileM * kYLd;
    // the bias row of the tile, after the y and B tiles (only with a bias)
    uint16_t* bls = ylds + (NH == 1 ? kTileM * kYLd + kExpandCols * 16 : NH == 2 || NH == 4 ? kExpandCols * 16 * NH : 0);
    // the arguments the data addresses need, in scalar registers before the
    // tile lookup, so that they load in the same round as its own arguments
    asm volatile("" ::"s"(a.u), "s"(a.slab), "s"(a.S), "s"(a.B), "s"(a.y), "s"(a.ldy), "s"(a.C), "s"(a.R),
                 "s"(a.out_f), "s"(a.ft), "s"(a.n_ftiles), "s"(a.valu_max), "s"(a.bias), "s"(a.r.G), "s"(a.r.end),
                 "s"(a.r.L), "s"(a.r.kr));

    const int lin = blockIdx.x;
    const int ftile = lin % a.n_ftiles;
    const int tile = lin / a.n_ftiles;
    TileInfo ti;
    if (!locate_tile<kTileM, false>(a.r, tile, ti))
        return;
    const int f0 = ftile * a.ft;
    const int ucol0 = slice_of(a, f0) * a.R;
    const RowMap<GATHER> ym{a.r.rows, ti.t0, ti.n, a.r.nrows};
    const Buf yb = ym.buf(reinterpret_cast<const T*>(a.y), a.ldy);
    // rank 16 stages y and B in LDS; ranks 32 and 64 stage B alone and keep y
    // in registers (an LDS tile of y as well would cut the workgroups per CU
    // to two or one); rank 48 reads both from memory
    if constexpr (NH > 0 && MODE == kMfmaOnly) {
        if constexpr (NH == 1)
            expand_mfma<NH, GATHER>(a, ti, f0, yb, ym, ucol0, us, part, ylds, blds, bls);
        else if constexpr (NH == 2 || NH == 4)
            expand_mfma_lb<NH, GATHER>(a, ti, f0, yb, ym, ucol0, us, part, ylds, bls);
        else
            expand_mfma_reg<NH, GATHER>(a, ti, f0, yb, ym, ucol0, us, part, bls);
    } else if constexpr (NH > 0 && MODE == kMixed) {
        if (ti.glen > a.valu_max) {
            if constexpr (NH == 1)
                expand_mfma<NH, GATHER>(a, ti, f0, yb, ym, ucol0, us, part, ylds, blds, bls);
            else if constexpr (NH == 2 || NH == 4)
                expand_mfma_lb<NH, GATHER>(a, ti, f0, yb, ym, ucol0, us, part, ylds, bls);
            else
                expand_mfma_reg<NH, GATHER>(a, ti, f0, yb, ym, ucol0, us, part, bls);
        } else
            expand_valu<T, GATHER>(a, ti, f0, yb, ym, ucol0, us, part);
    } else {
        expand_valu<T, GATHER>(a, ti, f0, yb, ym, ucol0, us, part);
    }
}

// ---------------------------------------------------------------------------
// one-kernel delta for long groups (prefill-sized batches; bf16, C <= 64)
//
// One 512-thread workgroup owns a piece of at most 64 consecutive tokens of
// one group (the long shrink's pieces: about one workgroup per compute unit)
// and computes its whole delta, so u never leaves the chip and the family
// takes one launch.
//
// Phase 1 (shrink): the 8 waves split K.  A wave moves x in chunks of 64 K
// values: eight loads of whole 128-byte lines (8 rows x 128 B each; the
// matrix layout would split every line over two loads, which measured about
// 20 % slower on this part) into registers, then into its own 8 KB LDS
// region (16-byte pieces rotated by row, so that both the line writes and
// the fragment reads spread over the banks), from which it reads the
// v_mfma_f32_16x16x32_bf16 M operands of its 64 rows.  A fragments come
// straight from the tiled layout (one contiguous 1 KB run each).  Loads run
// D chunks ahead.  The 8 partial tiles are added in LDS in the long shrink's
// fixed tree order; u [64][C] (fp32) stays in LDS.
//
// Phase 2 (expand): the waves split the output features in runs of 64.  For
// each run a wave loads the piece's 64 rows x 128 B of y as whole lines,
// rotates them through its LDS region into the MFMA C layout (lane = token,
// 8 consecutive features), adds B.u (B rows as the M operand, u = hi + lo
// bf16 halves as the N operand, as in the other expand kernels) and the
// bias, writes the rounded result back in place, and stores it as whole
// lines.  All accesses of x and y go through buffer bounds: rows past the
// piece read zero and drop their stores.
struct LongDeltaArgs {
    const uint16_t* x;
    int64_t ldx;
    const uint16_t* A;  // [L][a_slot] in the tiled A layout
    int64_t a_slot;
    const uint16_t* B;     // [L][out_f][R]
    const uint16_t* bias;  // [L][out_f] or null
    uint16_t* y;
    int64_t ldy;
    int in_f, C, out_f, n_s;
    int soff[5];
    int kw;  // K range of one wave (a multiple of 32)
    int fw;  // output features of one wave (a multiple of 64)
    int per_xcd, pieces;
    RouteArgs r;
    int k_piece0[LORA_MAX_HOST_GROUPS + 1];
};

template <int NB, int NH>
struct LongDeltaLds {
    static constexpr int kRegions = kLsWaves * kLdWaveBytes;
    static constexpr int kRed = LongShrinkLds<NB>::kFloats * 4;
    static constexpr int kU = (kRegions > kRed ? kRegions : kRed);  // offset of u [64][16 NB] fp32
    static constexpr int kBytes = kU + kLsRows * 16 * NB * 4;
};

// g holds one 16-byte fragment in lanes 0..31 and another in lanes 32..63;
// lo gets the first in every lane, hi the second (v_permlane32_swap).
__device__ __forceinline__ void permlane32_split(uint4 g, uint4& lo, uint4& hi)
{
    const auto sx = __builtin_amdgcn_permlane32_swap(g.x, g.x, false, false);
    const auto sy = __builtin_amdgcn_permlane32_swap(g.y, g.y, false, false);
    const auto sz = __builtin_amdgcn_permlane32_swap(g.z, g.z, false, false);
    const auto sw = __builtin_amdgcn_permlane32_swap(g.w, g.w, false, false);
    lo = make_uint4(sx[0], sy[0], sz[0], sw[0]);
    hi = make_uint4(sx[1], sy[1], sz[1], sw[1]);
}

template <int NB, int NH, int D, int D2, bool HB, bool GATHER>
__global__ __launch_bounds__(kLsThreads) void delta_long_kernel(LongDeltaArgs a)
{
    typedef LongDeltaLds<NB, NH> Lay;
    constexpr int R = 16 * NH;
    __shared__ __attribute__((aligned(16))) char smem[Lay::kBytes];
    asm volatile("" ::"s"(a.x), "s"(a.ldx), "s"(a.A), "s"(a.a_slot), "s"(a.B), "s"(a.bias), "s"(a.y), "s"(a.ldy),
                 "s"(a.in_f), "s"(a.C), "s"(a.out_f), "s"(a.kw), "s"(a.fw), "s"(a.per_xcd), "s"(a.pieces),
                 "s"(a.r.G), "s"(a.r.kr));
    const int b = blockIdx.x;
    const int piece = (b % kXcds) * a.per_xcd + b / kXcds;
    if (piece >= a.pieces)
        return;
    TileInfo ti;
    {
        // the long shrink's pieces (locate_piece)
        if (!a.r.kr) {
            if (!locate_tile<kLsRows, false>(a.r, piece, ti))
                return;
        } else {
            const int lane = threadIdx.x & 63;
            const bool in = lane < a.r.G;
            const int p0_l = in ? a.k_piece0[lane] : 0;
            const int p1_l = in ? a.k_piece0[lane + 1] : 0;
            const int gs_l = in ? a.r.k_offs[lane] : 0;
            const int ge_l = in ? a.r.k_offs[lane + 1] : 0;
            const int id_l = in ? a.r.k_ids[lane] : -1;
            const unsigned long long hit = __ballot(in && piece < p1_l);
            if (!hit)
                return;
            const int g = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
            const int p0 = __builtin_amdgcn_readlane(p0_l, g), np = __builtin_amdgcn_readlane(p1_l, g) - p0;
            const int gs = __builtin_amdgcn_readlane(gs_l, g), len = __builtin_amdgcn_readlane(ge_l, g) - gs;
            const int j = piece - p0;
            ti.t0 = gs + (int)(((int64_t)len * j) / np);
            ti.n = gs + (int)(((int64_t)len * (j + 1)) / np) - ti.t0;
            ti.slot = __builtin_amdgcn_readlane(id_l, g);
            if (ti.slot < 0 || ti.slot >= a.r.L)
                return;
        }
    }
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int lr = lane >> 3, lp = lane & 7;  // whole-line layout: row lr + 8 i, 16-byte piece lp
    char* region = smem + w * kLdWaveBytes;
    const RowMap<GATHER> rm{a.r.rows, ti.t0, ti.n, a.r.nrows};

    // ---------------- phase 1: u = A . x over the wave's K range
    const StreamBuf xb(rm.buf(a.x, a.ldx));  // x is read once: non-temporal
    uint32_t xro[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        xro[i] = (uint32_t)(rm(lr + 8 * i) * a.ldx) * 2;
    const Buf ab(a.A + (size_t)ti.slot * a.a_slot, (uint32_t)(NB * 16 * a.in_f * 2));
    const uint32_t ablk = (uint32_t)(16 * a.in_f) * 2;
    const int k0 = w * a.kw, k1 = min(k0 + a.kw, a.in_f);
    const int nch = k1 > k0 ? (k1 - k0 + 63) >> 6 : 0;
    f32x4_t acc[4][NB];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 xs[D][8], as[D][2][NB];
    auto load_x = [&](int ch, uint4(&xv)[8], uint4(&av)[2][NB]) {
        const int kx = k0 + 64 * ch + 8 * lp;
        const bool okx = kx < k1;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            xv[i] = xb.ld16(okx ? xro[i] + (uint32_t)kx * 2 : kOOB);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int kk = k0 + 64 * ch + 32 * s + 8 * q;
            const uint32_t ao = (uint32_t)(((kk >> 3) * 16 + l16) * 16);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                av[s][nb] = ab.ld16(kk < k1 ? nb * ablk + ao : kOOB);
        }
    };
#pragma unroll
    for (int j = 0; j < D; ++j) {
        load_x(j, xs[j], as[j]);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int base = 0; base < nch; base += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            // whole lines into the wave's region, then the M operands out of it
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<uint4*>(region + ld_slot(lr + 8 * i, lp)) = xs[j][i];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint4 xf = *reinterpret_cast<const uint4*>(region + ld_slot(16 * m + l16, 4 * s + q));
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, xf), __builtin_bit_cast(bf16x8_t, as[j][s][nb]), acc[m][nb],
                            0, 0, 0);
                }
            load_x(base + D + j, xs[j], as[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // partial tiles -> LDS tree (fixed order) -> u [64][16 NB] in LDS
    float* red = reinterpret_cast<float*>(smem);
    float* us = reinterpret_cast<float*>(smem + Lay::kU);
    constexpr int kLd = LongShrinkLds<NB>::kLd, kTile = LongShrinkLds<NB>::kTile;
    auto put = [&](int t) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    red[t * kTile + (16 * m + 4 * q + r) * kLd + 16 * nb + l16] = acc[m][nb][r];
    };
    auto add = [&](int t) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[m][nb][r] += red[t * kTile + (16 * m + 4 * q + r) * kLd + 16 * nb + l16];
    };
    __syncthreads();  // every wave is done with its region before the tree reuses it
    if (w >= 4)
        put(w - 4);
    __syncthreads();
    if (w < 4)
        add(w);
    __syncthreads();
    if (w == 2 || w == 3)
        put(w - 2);
    __syncthreads();
    if (w < 2)
        add(w);
    __syncthreads();
    if (w == 1)
        put(0);
    __syncthreads();
    if (w == 0) {
        add(0);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    us[(16 * m + 4 * q + r) * (16 * NB) + 16 * nb + l16] = acc[m][nb][r];
    }
    __syncthreads();

    // ---------------- phase 2: y += B . u (+ bias) over the wave's features
    const StreamBuf yb(rm.buf(a.y, a.ldy));  // y is read and written once: non-temporal
    uint32_t yro[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        yro[i] = (uint32_t)(rm(lr + 8 * i) * a.ldy) * 2;
    const Buf bb(a.B + (size_t)ti.slot * a.out_f * R, (uint32_t)(a.out_f * R * 2));
    const Buf biasb(a.bias + (size_t)ti.slot * a.out_f, a.bias ? (uint32_t)(a.out_f * 2) : 0u);
    const int mrow = 8 * (l16 >> 2) + (l16 & 3);  // permuted M row of block 0 (see expand_mfma)
    const int fb = w * a.fw, fe = min(fb + a.fw, a.out_f);
    const int ntl = fe > fb ? (fe - fb) >> 6 : 0;
    // B fragments: lanes q < 2 fetch the rows of the first 4-row half (hh =
    // 0), lanes q >= 2 those of the second; a permlane32 swap then gives
    // every lane both (the two halves of a wave need the same fragments),
    // which halves the B loads
    uint4 ys[D2][8], bs[D2][2][NH], bis[D2][2];
    auto load_y = [&](int t, uint4(&yv)[8], uint4(&bv)[2][NH], uint4(&biv)[2]) {
        const int f = fb + 64 * t;
        const bool ok = t < ntl;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            yv[i] = yb.ld16(ok ? yro[i] + (uint32_t)(f + 8 * lp) * 2 : kOOB);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int kh = 0; kh < NH; ++kh)
                bv[h][kh] = bb.ld16(
                    ok ? (uint32_t)((f + 32 * h + mrow + 4 * (q >> 1)) * R + 16 * kh + 8 * (q & 1)) * 2 : kOOB);
            if constexpr (HB)
                biv[h] = biasb.ld16(ok ? (uint32_t)(f + 32 * h + 8 * q) * 2 : kOOB);
        }
    };
#pragma unroll
    for (int j = 0; j < D2; ++j) {
        load_y(j, ys[j], bs[j], bis[j]);
        __builtin_amdgcn_sched_barrier(0);
    }
    int cur_sl = -1;
    bf16x8_t uf[4][NH];
    for (int base = 0; base < ntl; base += D2) {
#pragma unroll
        for (int j = 0; j < D2; ++j) {
            const int t = base + j;
            if (t < ntl) {
                const int f = fb + 64 * t;
                int sl = 0;
#pragma unroll
                for (int i = 1; i < 4; ++i)
                    if (i < a.n_s && f >= a.soff[i])
                        sl = i;
                if (sl != cur_sl) {
                    // u fragments of the slice: lanes q < 2 carry hi(u), q >= 2 lo(u)
                    cur_sl = sl;
#pragma unroll
                    for (int m = 0; m < 4; ++m)
#pragma unroll
                        for (int kh = 0; kh < NH; ++kh) {
                            const float* up = us + (16 * m + l16) * (16 * NB) + sl * R + 16 * kh + 8 * (q & 1);
                            uint32_t pk[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float v0 = up[2 * e], v1 = up[2 * e + 1];
                                uint32_t hi = f2bf_pair(v0, v1);
                                if (q >= 2)
                                    hi = f2bf_pair(v0 - bf2f(hi & 0xFFFFu), v1 - bf2f(hi >> 16));
                                pk[e] = hi;
                            }
                            uf[m][kh] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
                        }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<uint4*>(region + ld_slot(lr + 8 * i, lp)) = ys[j][i];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        uint4* cell = reinterpret_cast<uint4*>(region + ld_slot(16 * m + l16, 4 * h + q));
                        const uint4 yv = *cell;
                        f32x4_t acc0 = {bf2f(yv.x & 0xFFFFu), bf2f(yv.x >> 16), bf2f(yv.y & 0xFFFFu), bf2f(yv.y >> 16)};
                        f32x4_t acc1 = {bf2f(yv.z & 0xFFFFu), bf2f(yv.z >> 16), bf2f(yv.w & 0xFFFFu), bf2f(yv.w >> 16)};
                        if constexpr (HB)
                            add_bias8(bis[j][h], acc0, acc1);
#pragma unroll
                        for (int kh = 0; kh < NH; ++kh) {
                            uint4 b0, b1;
                            permlane32_split(bs[j][h][kh], b0, b1);
                            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b0), uf[m][kh],
                                                                          acc0, 0, 0, 0);
                            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b1), uf[m][kh],
                                                                          acc1, 0, 0, 0);
                        }
                        uint4 o;
                        o.x = f2bf_pair(acc0[0], acc0[1]);
                        o.y = f2bf_pair(acc0[2], acc0[3]);
                        o.z = f2bf_pair(acc1[0], acc1[1]);
                        o.w = f2bf_pair(acc1[2], acc1[3]);
                        *cell = o;
                    }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    yb.st16(yro[i] + (uint32_t)(f + 8 * lp) * 2,
                            *reinterpret_cast<const uint4*>(region + ld_slot(lr + 8 * i, lp)));
            }
            load_y(base + D2 + j, ys[j], bs[j], bis[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// ---------------------------------------------------------------------------
// one-kernel delta for short groups (decode batches)
//
// A decode batch moves a few MB per family, so a launch and a round trip to
// memory cost more than the transfer itself; the split-K shrink followed by
// the expand pays two of each and moves the split partial sums through
// memory.  Here one workgroup owns a tile of at most 16 tokens of one group,
// one slice (R columns of u) and one feature tile of that slice.  Its 16
// waves split K; every wave issues all its loads (x rows, A rows, its y run
// and B rows) at once, computes its K share of u with MFMA, and the 16
// partial u tiles are summed in LDS in wave order.  The waves then expand u
// into their 32-feature pair of y.  Each workgroup recomputes u for its
// slice: A and x are re-read from L2 once per feature tile, traded for the
// second launch and round trip.  Workgroups of one token tile are placed on
// one XCD (consecutive workgroups go to consecutive XCDs), so the tile's x
// rows and the group's A rows are fetched into that XCD's L2 once.

constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kFusedTileM = 16;
constexpr int kFusedMaxFeat = 32 * kFusedWaves;  // one 32-feature pair per wave

// A token tile as the host lays it out from its copy of the routing (the
// same tiles locate_tile<kFusedTileM, true> finds).
struct TileEntry {
    int t0, n, slot, glen;
};
constexpr int kFusedHostTiles = 128;
constexpr int kFusedHostFt = 64;

// The fields every workgroup needs before its first data load come first,
// so that they are one contiguous run of the argument segment.
struct FusedArgs {
    const uint16_t* bias;  // [L][out_f] per-adapter bias added in the epilogue, or null
    const uint16_t* x;
    int64_t ldx;
    const uint16_t* A;  // [L][a_slot] in the tiled A layout (a_tiled_index)
    int64_t a_slot;     // elements per slot
    const uint16_t* B;  // [L][out_f][R]
    uint16_t* y;
    int64_t ldy;
    int in_f, out_f;
    int F;           // feature tile width (multiple of 32, at most kFusedMaxFeat; up to four
                     // times that in the expand-only launch)
    int wave_steps;  // 32-element K steps per wave
    int C, n_s;
    int soff[5];
    int nft[4];      // feature tiles per slice
    int nf;          // feature tiles per token tile
    int krot;        // nonzero: wave w takes K range (w + feature tile) mod waves
    int kc;          // kPartShrink: K range of one split (a multiple of 32)
    float* slabs;    // split launches: fp32 slab s at slabs + s * slab, each [end][C]
    int64_t slab;
    int nsplit;      // kPartExpand: slabs to add (at most kFusedWaves)
    RouteArgs r;
    TileEntry tt[kFusedHostTiles];  // tiles built on the host (HOSTT launches)
    int2 fts[kFusedHostFt];         // (slice | 32-feature pairs << 8, first feature) of each
                                    // feature tile (HOSTT); SHRINK: (slice, K split)
};

// STEPS = K steps a wave keeps in flight per batch (register budget).
// XLDS: x goes through LDS (the wave's whole K range in one batch of 8
// steps, i.e. wave_steps <= 8).  Each wave moves its 16 rows x 512 bytes of
// x with eight LDS-DMA loads of whole 128-byte lines (2 rows per load); in
// each line the 16-byte pieces are rotated by (row mod 8), so that the MFMA
// operand reads (16 rows of one piece column) fall on distinct LDS banks.
// Lanes whose piece lies past the tile's rows or the wave's K range load a
// valid in-range piece instead: its row's results are never stored, and past
// the K range A reads as zero.
constexpr int kXLdsSteps = 8;
constexpr int kXLdsWaveBytes = 16 * 32 * kXLdsSteps * 2;  // 16 rows x 8 steps x 32 bf16

// HOSTT: the tile comes from the host-built table tt (entries with n = 0
// pad the grid), else from locate_tile over the routing.
// PART kPartShrink: the shrink half alone, with K split over workgroups.
// Workgroup (tile, slice, split s) sums x . A over K range [s kc, (s + 1) kc)
// of its slice and writes the tile's rows of slab s.  Nothing of y or B is
// read.
// PART kPartExpand: the expand half alone, from those slabs
// (fused_expand_from_slabs).
enum { kPartAll = 0, kPartShrink = 1, kPartExpand = 2, kPartExpand4 = 3 };

// The expand half of the split-K delta, from the shrink half's slabs: one
// workgroup per (16-token tile, feature tile of up to 512 NPAIR features),
// both from the host tables.  Wave w expands the 32-feature pairs 32 w + 512 p
// of the tile, p < NPAIR.  Its y runs, B rows and bias, and the tile's rows
// of its slice's columns of every slab, are loaded in one round; the slabs
// are added in LDS in split order (at most kFusedWaves of them) and the
// result is expanded as in the one-kernel delta.  part: kFusedWaves * 16 * R
// floats of LDS; us: 16 * R floats.
template <int NH, bool GATHER, int NPAIR>
__device__ __forceinline__ void fused_expand_from_slabs(const FusedArgs& a, float* part, float* us)
{
    constexpr int R = 16 * NH;
    const int tile = blockIdx.y * kXcds + blockIdx.x % kXcds;
    const int ftile = blockIdx.x / kXcds;
    const TileEntry te = a.tt[min(tile, kFusedHostTiles - 1)];
    const int2 fe = a.fts[min(ftile, kFusedHostFt - 1)];
    const int sl = fe.x & 0xFF, f0 = fe.y, fw = 32 * (fe.x >> 8);
    const uint32_t live = te.n > 0 ? 1u : 0u;  // 0 for a padding tile
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, q = lane >> 4;
    const int np = fw >> 5;
    const bool tok = l16 < te.n;
    const RowMap<GATHER> rm{a.r.rows, te.t0, te.n, a.r.nrows};
    const uint32_t trow = rm(l16);
    const StreamBuf yb(rm.buf(a.y, a.ldy));  // y is read and written once: non-temporal
    const Buf biasb(a.bias + (size_t)te.slot * a.out_f + f0, a.bias ? live * (uint32_t)(fw * 2) : 0u);
    const Buf bb(a.B + ((size_t)te.slot * a.out_f + f0) * R, live * (uint32_t)(fw * R * 2));
    const int mrow = 8 * (l16 >> 2) + (l16 & 3);
    uint32_t yoff[NPAIR];
    // B fragments: lanes q < 2 fetch the rows of a pair's block 0 (the
    // first MFMA), lanes q >= 2 those of block 1; a permlane32 swap at use
    // gives every lane its row of each block, so every fragment is fetched
    // once per wave.
    uint4 yraw[NPAIR], braw_bias[NPAIR], bfr[NPAIR][NH];
#pragma unroll
    for (int p = 0; p < NPAIR; ++p) {
        const int fp = 32 * (w + kFusedWaves * p);  // first feature of pair p in the tile
        const bool pv = w + kFusedWaves * p < np;
        yoff[p] = (pv && tok) ? (uint32_t)(trow * a.ldy + f0 + fp + 8 * q) * 2 : kOOB;
        yraw[p] = yb.ld16(yoff[p]);
        braw_bias[p] = biasb.ld16(pv ? (uint32_t)(fp + 8 * q) * 2 : kOOB);
        // B rows as the M operand, permuted: row i of block h is feature
        // fp + 8 (i / 4) + 4 h + i % 4 (see expand_mfma)
#pragma unroll
        for (int kh = 0; kh < NH; ++kh)
            bfr[p][kh] = bb.ld16(pv ? (uint32_t)((fp + mrow + 4 * (q >> 1)) * R + 16 * kh + 8 * (q & 1)) * 2 : kOOB);
    }
    // u of the tile from the slabs: entry e is 4 floats of slab e / Q, token
    // row (e % Q) / (R / 4), columns 4 ((e % Q) % (R / 4)) .. + 3 of the
    // slice; slabs past nsplit and rows past the tile read zero
    constexpr int Q = kFusedTileM * R / 4;
    const Buf sb(a.slabs, (uint32_t)((size_t)a.nsplit * a.slab * 4));
    for (int e = threadIdx.x; e < kFusedWaves * Q; e += kFusedThreads) {
        const int sp = e / Q, rem = e % Q, t = rem / (R / 4), j4 = rem % (R / 4);
        const bool ok = live && sp < a.nsplit && t < te.n;
        const uint4 v = sb.ld16(ok ? (uint32_t)(((size_t)sp * a.slab + (size_t)(te.t0 + t) * a.C + sl * R + 4 * j4) * 4)
                                   : kOOB);
        *reinterpret_cast<uint4*>(part + (sp * kFusedTileM + t) * R + 4 * j4) = v;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kFusedTileM * R; e += kFusedThreads) {
        float v = part[e];
#pragma unroll
        for (int sp = 1; sp < kFusedWaves; ++sp)
            v += part[sp * kFusedTileM * R + e];
        us[e] = v;
    }
    __syncthreads();
    if (w >= np)
        return;
    // u = hi + lo in bf16 as the N operand (tokens), y as C
    bf16x8_t uf[NH];
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) {
        const float* up = us + l16 * R + 16 * kh + 8 * (q & 1);
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v0 = up[2 * e], v1 = up[2 * e + 1];
            uint32_t hi = f2bf_pair(v0, v1);
            if (q >= 2)
                hi = f2bf_pair(v0 - bf2f(hi & 0xFFFFu), v1 - bf2f(hi >> 16));
            pk[e] = hi;
        }
        uf[kh] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
#pragma unroll
    for (int p = 0; p < NPAIR; ++p) {
        if (w + kFusedWaves * p >= np)
            break;
        f32x4_t acc0 = {bf2f(yraw[p].x & 0xFFFFu), bf2f(yraw[p].x >> 16), bf2f(yraw[p].y & 0xFFFFu),
                        bf2f(yraw[p].y >> 16)};
        f32x4_t acc1 = {bf2f(yraw[p].z & 0xFFFFu), bf2f(yraw[p].z >> 16), bf2f(yraw[p].w & 0xFFFFu),
                        bf2f(yraw[p].w >> 16)};
        if (a.bias)
            add_bias8(braw_bias[p], acc0, acc1);
#pragma unroll
        for (int kh = 0; kh < NH; ++kh) {
            uint4 b0, b1;
            permlane32_split(bfr[p][kh], b0, b1);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b0), uf[kh], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b1), uf[kh], acc1, 0, 0, 0);
        }
        uint4 o;
        o.x = f2bf_pair(acc0[0], acc0[1]);
        o.y = f2bf_pair(acc0[2], acc0[3]);
        o.z = f2bf_pair(acc1[0], acc1[1]);
        o.w = f2bf_pair(acc1[2], acc1[3]);
        yb.st16(yoff[p], o);
    }
}
template <int NH, int STEPS, bool XLDS, bool HOSTT, bool GATHER, int PART = kPartAll>
__global__ __launch_bounds__(kFusedThreads) void fused_delta_kernel(FusedArgs a)
{
    constexpr bool SHRINK = PART == kPartShrink;
    static_assert(PART == kPartAll || HOSTT, "the split launches use the host tile table");
    constexpr int R = 16 * NH;
    constexpr int kPartBytes = kFusedWaves * kFusedTileM * R * 4;
    constexpr int kXBytes = XLDS ? kFusedWaves * kXLdsWaveBytes : 0;
    static_assert(!XLDS || STEPS == kXLdsSteps, "x staging covers one batch of 8 steps");
    // x staging (XLDS) and, after the K loop, the per-wave partial u share
    // the first region
    __shared__ __attribute__((aligned(16))) char smem[(kXBytes > kPartBytes ? kXBytes : kPartBytes)];
    __shared__ float us[kFusedTileM * R];  // u of the tile
    float* part = reinterpret_cast<float*>(smem);
    if constexpr (PART == kPartExpand || PART == kPartExpand4) {
        fused_expand_from_slabs<NH, GATHER, PART == kPartExpand4 ? 4 : 2>(a, part, us);
        return;
    }

    // grid (kXcds * nf, tiles / kXcds): the linear block id b = x + y * gridDim.x
    // runs over XCDs as b % kXcds, so the nf workgroups of tile y * kXcds +
    // x % kXcds share one XCD; tile and feature tile need no kernel argument
    const int tile = blockIdx.y * kXcds + blockIdx.x % kXcds;
    const int ftile = blockIdx.x / kXcds;
    TileInfo ti;
    int sl = 0, f0, fw = a.F;  // slice, first feature and width of the feature tile
    if constexpr (HOSTT) {
        // the entries' addresses depend on blockIdx only, and nothing branches
        // before the data loads: the argument loads take one round trip.  A
        // padding entry has n = 0, which masks every access of the workgroup.
        const TileEntry te = a.tt[min(tile, kFusedHostTiles - 1)];
        const int2 fe = a.fts[min(ftile, kFusedHostFt - 1)];
        ti.g = 0;
        ti.t0 = te.t0;
        ti.n = te.n;
        ti.slot = te.slot;
        ti.glen = te.glen;
        sl = fe.x & 0xFF;
        fw = 32 * (fe.x >> 8);
        f0 = fe.y;
        // every argument the data addresses need, in scalar registers before
        // anything else: the compiler would otherwise split the argument
        // loads into two dependent rounds
        asm volatile("" ::"s"(a.x), "s"(a.A), "s"(a.B), "s"(a.y), "s"(a.ldx), "s"(a.ldy), "s"(a.a_slot),
                     "s"(a.in_f), "s"(a.out_f), "s"(a.F), "s"(a.wave_steps), "s"(te.t0), "s"(te.n), "s"(te.slot),
                     "s"(te.glen), "s"(fe.x), "s"(fe.y), "s"(a.bias), "s"(a.krot));
    } else {
        if (!locate_tile<kFusedTileM, true>(a.r, tile, ti))
            return;
        int rem = ftile;
        while (sl < a.n_s - 1 && rem >= a.nft[sl]) {
            rem -= a.nft[sl];
            ++sl;
        }
        f0 = a.soff[sl] + rem * a.F;
    }
    const uint32_t live = ti.n > 0 ? 1u : 0u;  // 0 for a padding tile
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, q = lane >> 4;

    // --- issue the loads: the wave's y run and B rows, then x / A batches
    const int np = fw >> 5;
    const bool pair = w < np;
    const bool tok = l16 < ti.n;
    const RowMap<GATHER> rm{a.r.rows, ti.t0, ti.n, a.r.nrows};
    const uint32_t trow = rm(l16);  // the buffer row of this lane's token
    const Buf yb = rm.buf(a.y, a.ldy);
    const uint32_t yoff = (pair && tok) ? (uint32_t)(trow * a.ldy + f0 + 32 * w + 8 * q) * 2 : kOOB;
    const uint4 yraw = SHRINK ? make_uint4(0u, 0u, 0u, 0u) : yb.ld16(yoff);
    // the wave's 8 bias values, read with y (zero without a bias)
    const Buf biasb(a.bias + (size_t)ti.slot * a.out_f + f0, a.bias ? live * (uint32_t)(fw * 2) : 0u);
    const uint4 braw_bias = SHRINK ? make_uint4(0u, 0u, 0u, 0u) : biasb.ld16(pair ? (uint32_t)(32 * w + 8 * q) * 2 : kOOB);
    // B rows as the M operand, permuted: row i of block h is feature
    // 32 w + 8 (i / 4) + 4 h + i % 4 (see expand_mfma)
    const Buf bb(a.B + ((size_t)ti.slot * a.out_f + f0) * R, live * (uint32_t)(fw * R * 2));
    const int mrow = 8 * (l16 >> 2) + (l16 & 3);
    uint4 bfr[2][NH];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kh = 0; kh < NH; ++kh)
            bfr[h][kh] = SHRINK ? make_uint4(0u, 0u, 0u, 0u)
                                : bb.ld16(pair ? (uint32_t)((32 * w + mrow + 4 * h) * R + 16 * kh + 8 * (q & 1)) * 2 : kOOB);

    // --- u partial over the wave's K range: x rows as M, A rows as N.  K
    // positions past the wave's range read as zero (offset kOOB).
    const Buf xb = rm.buf(a.x, a.ldx);  // rows >= n read zero
    // the slice's NH blocks of the tiled A: one step of one block is a 1 KB run
    const Buf ab(a.A + (size_t)ti.slot * a.a_slot + (size_t)sl * R * a.in_f, live * (uint32_t)(R * a.in_f * 2));
    // K range of this wave.  With krot the feature tiles of one token tile
    // start on different K ranges, so the workgroups that read the same x
    // and A lines do not ask for them in the same order; the partial sums are
    // still added in K-range order, so the result does not depend on it.
    const int kr = a.krot ? (w + ftile) & (kFusedWaves - 1) : w;
    // SHRINK: this workgroup's split of K (f0 holds the split index)
    const int kbase = SHRINK ? f0 * a.kc : 0;
    const int kend = SHRINK ? min(kbase + a.kc, a.in_f) : a.in_f;
    const int kw0 = kbase + kr * a.wave_steps * 32;
    const int kw1 = min(kw0 + a.wave_steps * 32, kend);
    const uint32_t xrow = (uint32_t)(trow * a.ldx) * 2, ablk = (uint32_t)(16 * a.in_f) * 2;
    f32x4_t acc[NH];
#pragma unroll
    for (int nb = 0; nb < NH; ++nb)
        acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (XLDS) {
        // x: eight LDS-DMA loads of 2 rows x 512 bytes into the wave's region
        char* xw = smem + w * kXLdsWaveBytes;
        {
            const int h = lane >> 5, u = (lane >> 3) & 3, j = lane & 7;
            const Buf xv = rm.buf(a.x, a.ldx);
#pragma unroll
            for (int i = 0; i < kXLdsSteps; ++i) {
                const int row = 2 * i + h;
                const int c = 8 * u + ((j - row) & 7);  // piece of the row this lane carries
                const int kk = kw0 + 8 * c;
                const int rr = max(min(row, ti.n - 1), 0);
                const int kc = kk < kw1 ? kk : min(kw0, a.in_f - 8);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xv.r, (__attribute__((address_space(3))) void*)(xw + 1024 * i), 16,
                    (int)((rm(rr) * a.ldx + kc) * 2), 0, 0, 0);
            }
        }
        uint4 ar[kXLdsSteps][NH];
#pragma unroll
        for (int i = 0; i < kXLdsSteps; ++i) {
            const int kk = kw0 + 32 * i + 8 * q;
            const uint32_t ao = (uint32_t)(((kk >> 3) * 16 + l16) * 8) * 2;
#pragma unroll
            for (int nb = 0; nb < NH; ++nb)
                ar[i][nb] = ab.ld16(kk < kw1 ? nb * ablk + ao : kOOB);
        }
        // every load (y, B, x, A) is out before the first wait: one round trip
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kXLdsSteps; ++i) {
            // piece 4 i + q of row l16: load l16 / 2, half l16 % 2, rotated slot
            const int c = 4 * i + q;
            const int slot = 32 * (l16 & 1) + 8 * (c >> 3) + ((c + l16) & 7);
            const uint4 xr = *reinterpret_cast<const uint4*>(xw + 1024 * (l16 >> 1) + 16 * slot);
#pragma unroll
            for (int nb = 0; nb < NH; ++nb)
                acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xr),
                                                                  __builtin_bit_cast(bf16x8_t, ar[i][nb]),
                                                                  acc[nb], 0, 0, 0);
        }
        __syncthreads();  // every wave is done with its x region before part overwrites it
    } else {
        const int nbatch = (a.wave_steps + STEPS - 1) / STEPS;
        for (int bt = 0; bt < nbatch; ++bt) {
            uint4 xr[STEPS], ar[STEPS][NH];
#pragma unroll
            for (int i = 0; i < STEPS; ++i) {
                const int kk = kw0 + 32 * (bt * STEPS + i) + 8 * q;
                const bool ok = kk < kw1;
                xr[i] = xb.ld16(ok ? xrow + (uint32_t)kk * 2 : kOOB);
                // piece kk / 8, row l16 of block nb: lane-contiguous 16-byte pieces
                const uint32_t ao = (uint32_t)(((kk >> 3) * 16 + l16) * 8) * 2;
#pragma unroll
                for (int nb = 0; nb < NH; ++nb)
                    ar[i][nb] = ab.ld16(ok ? nb * ablk + ao : kOOB);
            }
            // keep every load of the batch ahead of the first MFMA: one round trip
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < STEPS; ++i)
#pragma unroll
                for (int nb = 0; nb < NH; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xr[i]),
                                                                      __builtin_bit_cast(bf16x8_t, ar[i][nb]),
                                                                      acc[nb], 0, 0, 0);
        }
    }
    // D: lane holds rank column 16 nb + lane % 16 of token rows 4 (lane / 16) + r
#pragma unroll
    for (int nb = 0; nb < NH; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            part[(kr * kFusedTileM + 4 * q + r) * R + 16 * nb + l16] = acc[nb][r];
    __syncthreads();
    for (int e = threadIdx.x; e < kFusedTileM * R; e += kFusedThreads) {
        float v = part[e];
#pragma unroll
        for (int ww = 1; ww < kFusedWaves; ++ww)
            v += part[ww * kFusedTileM * R + e];
        us[e] = v;
    }
    __syncthreads();
    if constexpr (SHRINK) {
        // the tile's rows of slab f0, columns of slice sl
        float* dst = a.slabs + (size_t)f0 * a.slab + (size_t)ti.t0 * a.C + sl * R;
        for (int e = threadIdx.x; e < ti.n * R; e += kFusedThreads)
            dst[(size_t)(e / R) * a.C + e % R] = us[e];
        return;
    }
    if (!pair)
        return;

    // --- expand: u = hi + lo in bf16 as the N operand (tokens), y as C
    bf16x8_t uf[NH];
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) {
        const float* up = us + l16 * R + 16 * kh + 8 * (q & 1);
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v0 = up[2 * e], v1 = up[2 * e + 1];
            uint32_t hi = f2bf_pair(v0, v1);
            if (q >= 2)
                hi = f2bf_pair(v0 - bf2f(hi & 0xFFFFu), v1 - bf2f(hi >> 16));
            pk[e] = hi;
        }
        uf[kh] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
    f32x4_t acc0 = {bf2f(yraw.x & 0xFFFFu), bf2f(yraw.x >> 16), bf2f(yraw.y & 0xFFFFu), bf2f(yraw.y >> 16)};
    f32x4_t acc1 = {bf2f(yraw.z & 0xFFFFu), bf2f(yraw.z >> 16), bf2f(yraw.w & 0xFFFFu), bf2f(yraw.w >> 16)};
    if (a.bias)
        add_bias8(braw_bias, acc0, acc1);
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bfr[0][kh]), uf[kh], acc0, 0,
                                                      0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bfr[1][kh]), uf[kh], acc1, 0,
                                                      0, 0);
    }
    uint4 o;
    o.x = f2bf_pair(acc0[0], acc0[1]);
    o.y = f2bf_pair(acc0[2], acc0[3]);
    o.z = f2bf_pair(acc1[0], acc1[1]);
    o.w = f2bf_pair(acc1[2], acc1[3]);
    yb.st16(yoff, o);
}

// ---------------------------------------------------------------------------
// launch helpers

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device, queried once per device.
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Groups of at most this many tokens take the VALU path on AUTO (rank 16;
// ranks 32 and up take the MFMA path for every tile).
constexpr int kValuMaxTokens = 8;

int valu_max_for(int path, bool mfma_ok, int dflt_auto)
{
    if (!mfma_ok || path == LORA_PATH_VALU)
        return kTileM;  // every tile on the VALU path
    if (path == LORA_PATH_MFMA)
        return 0;
    return dflt_auto;
}

template <typename T, int MODE, bool G>
hipError_t launch_shrink_mode(const ShrinkArgs& a, int nb, int grid, hipStream_t st)
{
    switch (nb) {
    case 1: hipLaunchKernelGGL((shrink_kernel<T, 1, MODE, G>), dim3(grid), dim3(kThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((shrink_kernel<T, 2, MODE, G>), dim3(grid), dim3(kThreads), 0, st, a); break;
    case 3: hipLaunchKernelGGL((shrink_kernel<T, 3, MODE, G>), dim3(grid), dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((shrink_kernel<T, 4, MODE, G>), dim3(grid), dim3(kThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

template <bool G>
hipError_t launch_shrink_g(bool bf16, int mode, const ShrinkArgs& a, int nb, int grid, hipStream_t st)
{
    if (!bf16)
        return launch_shrink_mode<float, kValuOnly, G>(a, nb, grid, st);
    if (mode == kMfmaOnly)
        return launch_shrink_mode<uint16_t, kMfmaOnly, G>(a, nb, grid, st);
    if (mode == kValuOnly)
        return launch_shrink_mode<uint16_t, kValuOnly, G>(a, nb, grid, st);
    return launch_shrink_mode<uint16_t, kMixed, G>(a, nb, grid, st);
}

hipError_t launch_shrink(bool bf16, int mode, const ShrinkArgs& a, int nb, int grid, hipStream_t st)
{
    return a.r.rows ? launch_shrink_g<true>(bf16, mode, a, nb, grid, st)
                    : launch_shrink_g<false>(bf16, mode, a, nb, grid, st);
}

// Path mode of a launch: forced paths map to one variant; AUTO with a host
// copy of the routing looks at the group lengths (VALU for groups of at most
// valu_max tokens) and picks a single-path variant when all groups agree.
int pick_mode(int path, bool mfma_ok, int valu_max, const RouteArgs& r)
{
    if (!mfma_ok || path == LORA_PATH_VALU)
        return kValuOnly;
    if (path == LORA_PATH_MFMA)
        return kMfmaOnly;
    if (!r.kr)
        return kMixed;
    bool any_short = false, any_long = false;
    for (int g = 0; g < r.G; ++g) {
        const int len = r.k_offs[g + 1] - r.k_offs[g];
        if (len == 0)
            continue;
        if (len > valu_max)
            any_long = true;
        else
            any_short = true;
    }
    if (!any_short)
        return kMfmaOnly;
    if (!any_long)
        return kValuOnly;
    return kMixed;
}

// The caller's tuning choices (lora_options_t), resolved to values.
struct Tuning {
    int long_delta;    // -1 auto, 0 never, 1 whenever it applies
    int fused_max;     // longest group for which AUTO takes the one-kernel delta
    int splitk_short;  // -1 auto, 0 never, 1 whenever it applies
    int feat;          // one-kernel feature tile cap (0: automatic)
    int krot;          // staggered wave K ranges in the one-kernel delta
    int fold;          // -1 auto, 0 never, 1 always
};

// Longest group for which AUTO takes the one-kernel delta.
constexpr int kFusedMaxTokens = 32;

lora_status_t resolve_options(const lora_options_t* o, Tuning* t)
{
    t->long_delta = -1;
    t->fused_max = kFusedMaxTokens;
    t->splitk_short = -1;
    t->feat = 0;
    t->krot = 1;
    t->fold = -1;
    if (!o)
        return LORA_OK;
    if (o->fused_max_tokens >= 0)
        t->fused_max = o->fused_max_tokens;
    t->splitk_short = o->splitk_short < 0 ? -1 : o->splitk_short > 0;
    if (o->fused_feature_tile != 0) {
        const int f = o->fused_feature_tile;
        if (f < 32 || f > 512 || (f & (f - 1)) != 0)
            return LORA_ERR_INVALID_ARGUMENT;
        t->feat = f;
    }
    if (o->fused_k_rotation >= 0)
        t->krot = o->fused_k_rotation > 0;
    t->fold = o->fold_slabs < 0 ? -1 : o->fold_slabs > 0;
    t->long_delta = o->long_delta < 0 ? -1 : o->long_delta > 0;
    return LORA_OK;
}

struct Common {
    FamilyShape fs;
    bool bf16;
    RouteArgs r;
    Tuning t;
};

// Checks dims, family, path and the routing; fills the kernels' routing
// arguments (with the host copy of the routing when one is given).
lora_status_t check_common(const lora_dims_t* dims, int32_t family, int32_t path,
                           const lora_routing_t* rt, const lora_options_t* opts, Common* c)
{
    lora_status_t st = family_shape(dims, family, &c->fs);
    if (st != LORA_OK)
        return st;
    st = resolve_options(opts, &c->t);
    if (st != LORA_OK)
        return st;
    if (path < LORA_PATH_AUTO || path > LORA_PATH_FUSED || !rt)
        return LORA_ERR_INVALID_ARGUMENT;
    c->bf16 = dims->dtype == LORA_DTYPE_BF16;
    const int64_t end = rt->end;
    const int G = rt->num_groups;
    if (end < 0 || end > 2147483647LL || G < 0 || G > c->fs.L)
        return LORA_ERR_INVALID_ARGUMENT;
    RouteArgs& r = c->r;
    memset(&r, 0, sizeof(r));
    r.ids = rt->lora_ids;
    r.offs = rt->grouped_offsets;
    r.G = G;
    r.end = (int)end;
    r.L = c->fs.L;
    const bool host = rt->host_lora_ids && rt->host_grouped_offsets && G <= LORA_MAX_HOST_GROUPS;
    if (end > 0 && G > 0 && !host && (!rt->lora_ids || !rt->grouped_offsets))
        return LORA_ERR_INVALID_ARGUMENT;
    if (rt->token_rows) {
        // per-token routing: x and y hold num_rows rows in the caller's order
        if (rt->num_rows < end || rt->num_rows > 2147483647LL)
            return LORA_ERR_INVALID_ARGUMENT;
        r.rows = rt->token_rows;
        r.nrows = (uint32_t)rt->num_rows;
    }
    if (host) {
        const int32_t* o = rt->host_grouped_offsets;
        if (o[0] != 0 || o[G] != end)
            return LORA_ERR_INVALID_ARGUMENT;
        for (int g = 0; g < G; ++g) {
            if (o[g + 1] < o[g])
                return LORA_ERR_INVALID_ARGUMENT;
            if (rt->host_lora_ids[g] < 0 || rt->host_lora_ids[g] >= c->fs.L)
                return LORA_ERR_SLOT_OUT_OF_RANGE;
            r.k_ids[g] = rt->host_lora_ids[g];
        }
        for (int g = 0; g <= G; ++g)
            r.k_offs[g] = o[g];
        r.k_tile0[0] = 0;
        for (int g = 0; g < G; ++g)
            r.k_tile0[g + 1] = r.k_tile0[g] + (o[g + 1] - o[g] + kTileM - 1) / kTileM;
        r.kr = 1;
    }
    return LORA_OK;
}

bool shrink_mfma_ok(const Common& c) { return c.bf16; }

bool expand_mfma_ok(const Common& c)
{
    bool widths32 = true;
    for (int s = 0; s < c.fs.n_s; ++s)
        widths32 = widths32 && c.fs.widths[s] % 32 == 0;
    return c.bf16 && c.fs.R % 16 == 0 && c.fs.R <= 64 && widths32;
}

// Longest-processing-time placement of n items with costs cost[] on the
// XCDs: items in decreasing cost (ties in index order), each to the XCD with
// the least cost so far.  xcd_of gets each item's XCD; order the items in
// placement order (within an XCD the items run in that order).
void place_on_xcds(int n, const double* cost, int* order, int* xcd_of)
{
    for (int i = 0; i < n; ++i)
        order[i] = i;
    std::stable_sort(order, order + n, [&](int p, int q) { return cost[p] > cost[q]; });
    double load[kXcds] = {};
    for (int i = 0; i < n; ++i) {
        int best = 0;
        for (int x = 1; x < kXcds; ++x)
            if (load[x] < load[best])
                best = x;
        xcd_of[order[i]] = best;
        load[best] += cost[order[i]];
    }
}

// Shrink placement from the host routing.  The workgroups of one (group,
// K split) item, i.e. all the group's 64-token tiles and column groups for
// that K range, run on one XCD next to one another, so that a tile's x range
// is fetched into one L2 for all its column groups and the group's A range
// for all its tiles; the items are placed by their bytes (A range, x rows
// and a fixed cost per workgroup).  With the plain order the column groups
// of a tile fall on different XCDs and the tiles of a group on two (mixed
// batch, hidden 5120, rank 64: shrink traffic 96 -> 70 MB per QKV call,
// step 0.558 -> 0.545 ms; 32-layer stack 2.585 -> 2.572 ms).  Placing the
// expand's workgroups the same way (all feature tiles of a tile on one XCD)
// cut its traffic as well but ran slower (mixed 0.579 ms, stack 2.722 ms).
// False (plain order) when the table cannot hold the grid.
bool shrink_xcd_map(const Common& c, const ShrinkPlan& p, ShrinkArgs& a, int64_t& grid)
{
    if (!c.r.kr || p.S > 255 || p.nz > 255 || p.n_tiles > 65535)
        return false;
    int item_g[kShrinkMapMax], item_s[kShrinkMapMax], order[kShrinkMapMax], xcd_of[kShrinkMapMax];
    double cost[kShrinkMapMax];
    int n = 0, wgs = 0;
    const double rows16 = (double)a_tiled_rows(c.fs.C);
    for (int g = 0; g < c.r.G; ++g) {
        const int nt = c.r.k_tile0[g + 1] - c.r.k_tile0[g];
        const int len = c.r.k_offs[g + 1] - c.r.k_offs[g];
        if (nt <= 0)
            continue;
        for (int sp = 0; sp < p.S; ++sp) {
            wgs += nt * p.nz;
            if (n == kShrinkMapMax || wgs > kShrinkMapMax)
                return false;
            const double kcs = std::min(p.kc, c.fs.in_f - sp * p.kc);
            item_g[n] = g;
            item_s[n] = sp;
            cost[n] = 2.0 * kcs * (rows16 + len) + 16384.0 * nt * p.nz;
            ++n;
        }
    }
    place_on_xcds(n, cost, order, xcd_of);
    int cnt[kXcds] = {};
    for (int i = 0; i < n; ++i)
        cnt[xcd_of[i]] += (c.r.k_tile0[item_g[i] + 1] - c.r.k_tile0[item_g[i]]) * p.nz;
    const int rows = *std::max_element(cnt, cnt + kXcds);
    if (rows * kXcds > kShrinkMapMax)
        return false;
    for (int i = 0; i < kShrinkMapMax; ++i)
        a.xmap[i] = kNoEntry;
    int fill[kXcds] = {};
    for (int k = 0; k < n; ++k) {
        const int i = order[k], x = xcd_of[i], g = item_g[i];
        for (int t = c.r.k_tile0[g]; t < c.r.k_tile0[g + 1]; ++t)
            for (int z = 0; z < p.nz; ++z)
                a.xmap[fill[x]++ * kXcds + x] = (uint32_t)t << 16 | (uint32_t)item_s[i] << 8 | (uint32_t)z;
    }
    a.xmap_on = 1;
    grid = (int64_t)rows * kXcds;
    return true;
}

// shrink launch; `out` receives u (S == 1) or the S slabs
lora_status_t run_shrink(const Common& c, const ShrinkPlan& plan, const void* x, int64_t ldx,
                         const void* A_stack, float* out, int32_t path, hipStream_t s)
{
    ShrinkArgs a;
    a.x = x;
    a.ldx = ldx;
    a.A = A_stack;
    a.a_slot = a_tiled_elems(c.fs.C, c.fs.in_f);
    a.out = out;
    a.slab = (int64_t)c.r.end * c.fs.C;
    a.in_f = c.fs.in_f;
    a.C = c.fs.C;
    a.S = plan.S;
    a.kc = plan.kc;
    a.nz = plan.nz;
    a.cb = plan.cb;
    // ranks 32 and up take the MFMA path for every tile: the VALU path keeps
    // one chunk in flight and runs eight token rows per chunk whatever the
    // tile's length, which loses to the MFMA tile even for one-token groups
    a.valu_max = valu_max_for(path, shrink_mfma_ok(c), c.fs.R >= 32 ? 0 : kValuMaxTokens);
    a.r = c.r;
    a.xmap_on = 0;
    int64_t grid = (int64_t)plan.n_tiles * plan.S * plan.nz;
    if (grid > 2147483647LL)
        return LORA_ERR_INVALID_ARGUMENT;
    shrink_xcd_map(c, plan, a, grid);
    const int mode = pick_mode(path, shrink_mfma_ok(c), a.valu_max, c.r);
    const hipError_t e = launch_shrink(c.bf16, mode, a, plan.cb / 16, (int)grid, s);
    return e == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

// Which shrink kernel a call runs, with its launch plan.  The long-segment
// kernel takes every bf16 call that does not force the VALU path.
struct ShrinkChoice {
    bool lng;
    ShrinkPlan old;  // the 256-thread kernel's plan (lng false)
    LongPlan lp;     // the long-segment kernel's plan (lng true)
    int pieces, per_xcd;
    int k_piece0[LORA_MAX_HOST_GROUPS + 1];
    int S() const { return lng ? lp.S : old.S; }
    size_t slab_bytes(const Common& c) const { return (size_t)c.r.end * c.fs.C * sizeof(float); }
};

// 64-token tiles of the batch: exact with the host copy of the routing,
// else a bound.
int64_t long_tiles(const Common& c)
{
    if (!c.r.kr)
        return ((int64_t)c.r.end + kLongRows - 1) / kLongRows + c.r.G;
    int64_t t = 0;
    for (int g = 0; g < c.r.G; ++g)
        t += (c.r.k_offs[g + 1] - c.r.k_offs[g] + kLongRows - 1) / kLongRows;
    return t;
}

ShrinkChoice choose_shrink(const Common& c, int32_t path)
{
    ShrinkChoice ch;
    const int64_t tiles = long_tiles(c);
    ch.lp = plan_long(c.fs, tiles);
    // the long-segment kernel only where its plan splits no K (batches that
    // fill the chip with 64-token pieces): with a K split, the 256-thread
    // kernel measured faster (mixed batch 24.2 against 30.0 us).  The 32-layer
    // stack's rank-32 QKV (two column groups, pieces of ~28 tokens) takes it:
    // delta_qkv 47.4 against 49.1 us with the 256-thread kernel
    ch.lng = shrink_mfma_ok(c) && path != LORA_PATH_VALU && ch.lp.S == 1;
    if (!ch.lng)
        ch.old = plan_shrink(c.fs, c.r.end, c.r.G);
    // the pieces of the long-segment kernels (the long delta may be forced
    // where the long shrink is not taken)
    if (!c.r.kr) {
        ch.pieces = (int)tiles;
    } else {
        // more, shorter pieces while that still leaves about one workgroup
        // per compute unit (only when K is not split)
        const int64_t end = std::max<int64_t>(c.r.end, 1);
        ch.k_piece0[0] = 0;
        for (int g = 0; g < c.r.G; ++g) {
            const int64_t len = c.r.k_offs[g + 1] - c.r.k_offs[g];
            int64_t n = (len + kLongRows - 1) / kLongRows;
            if (ch.lp.S == 1)
                n = std::max<int64_t>(n, len * kPlanCUs / (end * ch.lp.nz));
            ch.k_piece0[g + 1] = ch.k_piece0[g] + (int)n;
        }
        ch.pieces = ch.k_piece0[c.r.G];
    }
    ch.per_xcd = (ch.pieces + kXcds - 1) / kXcds;
    return ch;
}

// Workspace a shrink choice needs: the S > 1 slabs (lora_sgmv_shrink), or
// u itself as well (lora_sgmv_delta keeps u in the workspace).
size_t shrink_need(const Common& c, const ShrinkChoice& ch, bool delta)
{
    const int S = ch.S();
    return (delta || S > 1) ? (size_t)S * ch.slab_bytes(c) : 0;
}

template <bool NTX, bool G>
hipError_t launch_shrink_long(const LongShrinkArgs& a, int nb, dim3 grid, hipStream_t st)
{
    switch (nb) {
    case 1: hipLaunchKernelGGL((shrink_long_kernel<1, 3, NTX, G>), grid, dim3(kLsThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((shrink_long_kernel<2, 3, NTX, G>), grid, dim3(kLsThreads), 0, st, a); break;
    case 3: hipLaunchKernelGGL((shrink_long_kernel<3, 2, NTX, G>), grid, dim3(kLsThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((shrink_long_kernel<4, 2, NTX, G>), grid, dim3(kLsThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

lora_status_t run_shrink_long(const Common& c, const ShrinkChoice& ch, const void* x, int64_t ldx,
                              const void* A_stack, float* out, hipStream_t s)
{
    LongShrinkArgs a;
    a.x = reinterpret_cast<const uint16_t*>(x);
    a.ldx = ldx;
    a.A = reinterpret_cast<const uint16_t*>(A_stack);
    a.a_slot = a_tiled_elems(c.fs.C, c.fs.in_f);
    a.out = out;
    a.slab = (int64_t)c.r.end * c.fs.C;
    a.in_f = c.fs.in_f;
    a.C = c.fs.C;
    a.kc = ch.lp.kc;
    a.S = ch.lp.S;
    a.zs = ch.lp.nz * ch.lp.S;
    a.cb = ch.lp.cb;
    a.per_xcd = ch.per_xcd;
    a.pieces = ch.pieces;
    a.r = c.r;
    for (int g = 0; g <= LORA_MAX_HOST_GROUPS; ++g)
        a.k_piece0[g] = c.r.kr && g <= c.r.G ? ch.k_piece0[g] : 0;
    const int64_t grid = (int64_t)kXcds * ch.per_xcd * a.zs;
    if (grid > 2147483647LL)
        return LORA_ERR_INVALID_ARGUMENT;
    if (grid == 0)
        return LORA_OK;
    const int nb = ch.lp.cb / 16;
    // one column group reads x once: non-temporal x loads (prefill, 4
    // layers: shrink_qkv 28.6 -> 25.3 us, shrink_o 26.6 -> 21.7 us); with
    // two, the second group's reads hit the caches the first one filled
    const dim3 g((unsigned)grid);
    const bool ntx = ch.lp.nz == 1;
    const hipError_t e = c.r.rows ? (ntx ? launch_shrink_long<true, true>(a, nb, g, s)
                                         : launch_shrink_long<false, true>(a, nb, g, s))
                                  : (ntx ? launch_shrink_long<true, false>(a, nb, g, s)
                                         : launch_shrink_long<false, false>(a, nb, g, s));
    return e == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

// The chosen shrink kernel; `out` receives u (S == 1) or the S slabs.
lora_status_t run_shrink_any(const Common& c, const ShrinkChoice& ch, const void* x, int64_t ldx,
                             const void* A_stack, float* out, int32_t path, hipStream_t s)
{
    if (ch.lng)
        return run_shrink_long(c, ch, x, ldx, A_stack, out, s);
    return run_shrink(c, ch.old, x, ldx, A_stack, out, path, s);
}

bool nh_possible(const Common& c, const ExpandArgs& a) { return expand_mfma_ok(c) && a.valu_max < kTileM; }

template <bool G>
void launch_expand(bool bf16, int nh, int mode, dim3 g, dim3 b, size_t lds, hipStream_t s, const ExpandArgs& a)
{
#define LORA_EXPAND_NH(NHV)                                                                       \
    if (mode == kMfmaOnly)                                                                        \
        hipLaunchKernelGGL((expand_kernel<uint16_t, NHV, kMfmaOnly, G>), g, b, lds, s, a);        \
    else if (mode == kValuOnly)                                                                   \
        hipLaunchKernelGGL((expand_kernel<uint16_t, 0, kValuOnly, G>), g, b, lds, s, a);          \
    else                                                                                          \
        hipLaunchKernelGGL((expand_kernel<uint16_t, NHV, kMixed, G>), g, b, lds, s, a);
    if (!bf16) {
        hipLaunchKernelGGL((expand_kernel<float, 0, kValuOnly, G>), g, b, lds, s, a);
    } else if (nh == 1) {
        LORA_EXPAND_NH(1)
    } else if (nh == 2) {
        LORA_EXPAND_NH(2)
    } else if (nh == 3) {
        LORA_EXPAND_NH(3)
    } else if (nh == 4) {
        LORA_EXPAND_NH(4)
    } else {
        hipLaunchKernelGGL((expand_kernel<uint16_t, 0, kValuOnly, G>), g, b, lds, s, a);
    }
#undef LORA_EXPAND_NH
}

lora_status_t run_expand(const Common& c, const float* u, int64_t slab, int S, const void* B_stack,
                         const void* bias, void* y, int64_t ldy, int32_t path, hipStream_t s)
{
    ExpandArgs a;
    a.bias = bias;
    a.u = u;
    a.slab = slab;
    a.S = S;
    a.B = B_stack;
    a.y = y;
    a.ldy = ldy;
    a.C = c.fs.C;
    a.R = c.fs.R;
    a.n_s = c.fs.n_s;
    a.out_f = c.fs.out_f;
    for (int i = 0; i < 5; ++i)
        a.soff[i] = i <= c.fs.n_s ? c.fs.offs[i] : c.fs.out_f;
    a.ft = expand_tile(c.fs);
    a.n_ftiles = c.fs.out_f / a.ft;
    // ranks 32 and 64 take the MFMA path (B through LDS) for every tile: the
    // VALU path reads B rows strided and is L1-bound there
    const bool lds_b = c.fs.R == 32 || c.fs.R == 64;
    a.valu_max = valu_max_for(path, expand_mfma_ok(c), lds_b ? 0 : kValuMaxTokens);
    a.r = c.r;
    const int64_t tiles = ((int64_t)c.r.end + kTileM - 1) / kTileM + c.r.G;
    const int64_t grid = tiles * a.n_ftiles;
    if (grid > 2147483647LL)
        return LORA_ERR_INVALID_ARGUMENT;
    const int nh = nh_possible(c, a) ? c.fs.R / 16 : 0;
    // u tile, slab partial sums, then the LDS tiles of the MFMA path: y and B
    // (rank 16) or B alone (ranks 32 and 64)
    const size_t lds = (size_t)kTileM * c.fs.R * sizeof(float) + kThreads * sizeof(float4) +
                       (nh == 1   ? ((size_t)kTileM * kYLd + (size_t)kExpandCols * c.fs.R) * sizeof(uint16_t)
                        : nh == 2 || nh == 4 ? (size_t)kExpandCols * c.fs.R * sizeof(uint16_t)
                                             : 0) +
                       (nh && bias ? (size_t)kExpandCols * sizeof(uint16_t) : 0);
    const dim3 g((unsigned)grid), b(kThreads);
    const int mode = nh ? pick_mode(path, true, a.valu_max, c.r) : kValuOnly;
    if (c.r.rows)
        launch_expand<true>(c.bf16, nh, mode, g, b, lds, s, a);
    else
        launch_expand<false>(c.bf16, nh, mode, g, b, lds, s, a);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

// One-kernel delta: bf16, R = 16 or 32, slice widths multiples of 32.
bool fused_ok(const Common& c)
{
    bool widths32 = true;
    for (int s = 0; s < c.fs.n_s; ++s)
        widths32 = widths32 && c.fs.widths[s] % 32 == 0;
    return c.bf16 && (c.fs.R == 16 || c.fs.R == 32) && widths32;
}

// AUTO takes the one-kernel delta when the host copy of the routing shows
// that no group is longer than the fused_max_tokens option (default 32).
bool fused_auto(const Common& c)
{
    if (!fused_ok(c) || !c.r.kr)
        return false;
    for (int g = 0; g < c.r.G; ++g)
        if (c.r.k_offs[g + 1] - c.r.k_offs[g] > c.t.fused_max)
            return false;
    return true;
}

// Feature tiles of width f: F, nft and nf of the launch arguments.
void set_fused_feat(const Common& c, FusedArgs& a, int f)
{
    a.F = f;
    a.nf = 0;
    for (int sl = 0; sl < 4; ++sl) {
        a.nft[sl] = sl < c.fs.n_s ? c.fs.widths[sl] / f : 0;
        a.nf += a.nft[sl];
    }
}

// The widest feature tile: the largest power of two <= kFusedMaxFeat
// dividing every slice width (the fused_feature_tile option, a power of two
// in [32, 512], caps it).  Slice widths are multiples of 32 here, so the
// result is a power of two of at least 32.
int fused_widest_feat(const Common& c)
{
    int F = c.t.feat > 0 ? c.t.feat : kFusedMaxFeat;
    for (int sl = 0; sl < c.fs.n_s; ++sl)
        while (F > 32 && c.fs.widths[sl] % F)
            F >>= 1;
    return F;
}

// Final feature tiles once the grid height (rows, tiles per XCD) is known,
// and the feature-tile table of a host-table launch.
// Every workgroup of the one-kernel delta reads its token tile's x rows and
// its slice's A rows whatever its feature tile, and that read is most of its
// time; halving the feature tile doubles the workgroups without changing that
// read.  So the tile is halved (down to 128 features) only while each XCD
// still runs at most one workgroup per compute unit: then the extra
// workgroups land on idle units and each one's y and B share shrinks.
// uneven (the one-kernel launch with the host table): where that still
// leaves compute units idle, the slices are cut into more, near-equal tiles
// of whole 32-feature pairs, one more tile at a time for the slice whose
// widest tile is widest, until each XCD runs one workgroup per compute unit
// (decode QKV: Q in 10 tiles of 12-13 pairs and K, V in 3 of 10-11, i.e. 256
// workgroups instead of 192 of 16 pairs).
void fused_feature_tiles(const Common& c, FusedArgs& a, int64_t rows, bool hostt, bool uneven = false)
{
    int F = a.F;
    const int per_xcd = device_cus() / kXcds;
    if (c.t.feat <= 0) {
        while (F > 128) {
            int nf2 = 0;
            for (int sl = 0; sl < c.fs.n_s; ++sl)
                nf2 += c.fs.widths[sl] / (F / 2);
            if (rows * nf2 > per_xcd || (hostt && nf2 > kFusedHostFt))
                break;
            F /= 2;
        }
        set_fused_feat(c, a, F);
    }
    if (hostt) {
        int n[4] = {0, 0, 0, 0}, tot = 0;
        for (int sl = 0; sl < c.fs.n_s; ++sl)
            tot += n[sl] = a.nft[sl];
        if (uneven && c.t.feat <= 0) {
            const int64_t target = std::min<int64_t>(per_xcd / std::max<int64_t>(rows, 1), kFusedHostFt);
            while (tot < target) {
                int best = -1, widest = 1;
                for (int sl = 0; sl < c.fs.n_s; ++sl) {
                    const int p = c.fs.widths[sl] / 32, wmax = (p + n[sl] - 1) / n[sl];
                    if (wmax > widest) {
                        widest = wmax;
                        best = sl;
                    }
                }
                if (best < 0)
                    break;  // every tile is one pair
                ++n[best];
                ++tot;
            }
        }
        int ft = 0, most = 0;
        for (int sl = 0; sl < c.fs.n_s; ++sl) {
            const int p = c.fs.widths[sl] / 32;
            int f = a.soff[sl];
            for (int i = 0; i < n[sl]; ++i) {
                const int pi = p / n[sl] + (i < p % n[sl] ? 1 : 0);
                a.fts[ft++] = make_int2(sl | pi << 8, f);
                f += 32 * pi;
                most = std::max(most, pi);
            }
            a.nft[sl] = n[sl];
        }
        a.nf = ft;
        a.F = 32 * most;
        for (; ft < kFusedHostFt; ++ft)
            a.fts[ft] = make_int2(0, 0);
    }
}

// The launch arguments every one-kernel launch shares.
void fused_common_args(const Common& c, FusedArgs& a, const void* x, int64_t ldx, const void* A_stack,
                       const void* B_stack, const void* bias, void* y, int64_t ldy)
{
    a.bias = reinterpret_cast<const uint16_t*>(bias);
    a.x = reinterpret_cast<const uint16_t*>(x);
    a.ldx = ldx;
    a.A = reinterpret_cast<const uint16_t*>(A_stack);
    a.a_slot = a_tiled_elems(c.fs.C, c.fs.in_f);
    a.B = reinterpret_cast<const uint16_t*>(B_stack);
    a.y = reinterpret_cast<uint16_t*>(y);
    a.ldy = ldy;
    a.in_f = c.fs.in_f;
    a.C = c.fs.C;
    a.out_f = c.fs.out_f;
    a.n_s = c.fs.n_s;
    for (int i = 0; i < 5; ++i)
        a.soff[i] = i <= c.fs.n_s ? c.fs.offs[i] : c.fs.out_f;
    a.krot = c.t.krot;
    a.kc = 0;
    a.slabs = nullptr;
    a.slab = 0;
    a.nsplit = 0;
    a.r = c.r;
}

// Token tiles of the one-kernel launches from the host routing: each group
// cut into ceil(len / 16) near-equal tiles (the tiles locate_tile<kFusedTileM,
// true> finds).
int64_t fused_host_tiles(const Common& c)
{
    int64_t tiles = 0;
    for (int g = 0; g < c.r.G; ++g)
        tiles += (c.r.k_offs[g + 1] - c.r.k_offs[g] + kFusedTileM - 1) / kFusedTileM;
    return tiles;
}

// The host tile table: the tiles of a group go to one XCD (tile position
// y * kXcds + xcd), so that its A and B rows are fetched into one L2: groups,
// largest first, each to the XCD with the fewest tiles so far.  rows gets the
// grid height (tiles per XCD).  False when the table cannot hold the tiles.
bool fused_tile_table(const Common& c, FusedArgs& a, int64_t& rows)
{
    int order[LORA_MAX_HOST_GROUPS], cnt[kXcds] = {}, xcd_of[LORA_MAX_HOST_GROUPS];
    constexpr bool together = true;
    for (int g = 0; g < c.r.G; ++g)
        order[g] = g;
    auto gtiles = [&](int g) { return (c.r.k_offs[g + 1] - c.r.k_offs[g] + kFusedTileM - 1) / kFusedTileM; };
    rows = (fused_host_tiles(c) + kXcds - 1) / kXcds;
    if (together) {
        std::stable_sort(order, order + c.r.G, [&](int p, int q) { return gtiles(p) > gtiles(q); });
        for (int i = 0; i < c.r.G; ++i) {
            int best = 0;
            for (int x = 1; x < kXcds; ++x)
                if (cnt[x] < cnt[best])
                    best = x;
            xcd_of[order[i]] = best;
            cnt[best] += gtiles(order[i]);
        }
        rows = *std::max_element(cnt, cnt + kXcds);
    }
    if (rows * kXcds > kFusedHostTiles)
        return false;
    for (int i = 0; i < kFusedHostTiles; ++i)
        a.tt[i] = TileEntry{0, 0, 0, 0};
    int fill[kXcds] = {}, n = 0;
    for (int g = 0; g < c.r.G; ++g) {
        const int gs = c.r.k_offs[g], len = c.r.k_offs[g + 1] - gs;
        const int gnt = gtiles(g);
        for (int j = 0; j < gnt; ++j) {
            const int t0 = gs + (int)(((int64_t)len * j) / gnt);
            const int t1 = gs + (int)(((int64_t)len * (j + 1)) / gnt);
            const int pos = together ? fill[xcd_of[g]]++ * kXcds + xcd_of[g] : n++;
            a.tt[pos] = TileEntry{t0, t1 - t0, c.r.k_ids[g], len};
        }
    }
    return true;
}

lora_status_t run_fused(const Common& c, const void* x, int64_t ldx, const void* A_stack, const void* B_stack,
                        const void* bias, void* y, int64_t ldy, hipStream_t s)
{
    FusedArgs a;
    fused_common_args(c, a, x, ldx, A_stack, B_stack, bias, y, ldy);
    set_fused_feat(c, a, fused_widest_feat(c));
    const int steps = (c.fs.in_f + 31) / 32;
    a.wave_steps = (steps + kFusedWaves - 1) / kFusedWaves;
    // token tiles: exact count from the host routing, else a bound
    const int64_t tiles =
        c.r.kr ? fused_host_tiles(c) : ((int64_t)c.r.end + kFusedTileM - 1) / kFusedTileM + c.r.G;
    if (tiles == 0)
        return LORA_OK;
    if ((int64_t)(tiles + kXcds - 1) / kXcds * kXcds * a.nf > 2147483647LL || (tiles + kXcds - 1) / kXcds > 65535)
        return LORA_ERR_INVALID_ARGUMENT;
    int64_t rows = (tiles + kXcds - 1) / kXcds;  // grid rows (tiles per XCD)
    bool hostt = c.r.kr && a.nf <= kFusedHostFt && fused_tile_table(c, a, rows);
    if (!hostt)
        rows = (tiles + kXcds - 1) / kXcds;
    fused_feature_tiles(c, a, rows, hostt, true);
    // x through LDS when the wave's K range is one batch of 8 steps (K <= 4096)
    const bool xlds = a.wave_steps <= kXLdsSteps;
    const dim3 g((unsigned)(kXcds * a.nf), (unsigned)rows), blk(kFusedThreads);
    const bool gather = c.r.rows != nullptr;
#define LORA_FUSED(NH, ST, XL)                                                             \
    if (hostt && gather)                                                                   \
        hipLaunchKernelGGL((fused_delta_kernel<NH, ST, XL, true, true>), g, blk, 0, s, a); \
    else if (hostt)                                                                        \
        hipLaunchKernelGGL((fused_delta_kernel<NH, ST, XL, true, false>), g, blk, 0, s, a); \
    else if (gather)                                                                       \
        hipLaunchKernelGGL((fused_delta_kernel<NH, ST, XL, false, true>), g, blk, 0, s, a); \
    else                                                                                   \
        hipLaunchKernelGGL((fused_delta_kernel<NH, ST, XL, false, false>), g, blk, 0, s, a);
    if (c.fs.R == 16) {
        if (xlds) {
            LORA_FUSED(1, 8, true)
        } else {
            LORA_FUSED(1, 8, false)
        }
    } else {
        if (xlds) {
            LORA_FUSED(2, 8, true)
        } else {
            LORA_FUSED(2, 4, false)
        }
    }
#undef LORA_FUSED
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

// Short groups whose one-kernel delta would be slow: a K longer than 4096
// (each of that launch's workgroups reads its tile's x rows and its slice's
// A rows over all of K), or more than two of its workgroups per compute unit
// at the widest feature tile (a wide output: every feature tile recomputes
// the rank-space values).  On the Llama-3-8B decode batch: MLP down (K 14336)
// 20.9 -> 10.2 us, gate_up (28 672 outputs) 24.6 -> 16.9 us; the attention
// families stay on the one-kernel path (QKV 8.2 there, 10.3 us split).
// The splitk_short option (0/1) forces the choice.
bool splitk_short_wanted(const Common& c)
{
    if (c.t.splitk_short >= 0)
        return c.t.splitk_short > 0;
    if (c.fs.in_f > 4096)
        return true;
    int nf = 0;
    for (int sl = 0; sl < c.fs.n_s; ++sl)
        nf += c.fs.widths[sl] / fused_widest_feat(c);
    return fused_host_tiles(c) * nf > 2 * (int64_t)device_cus();
}

// The split-K delta for short groups: the one-kernel delta's shrink half with
// K split over workgroups (fp32 slabs in the workspace, one load round trip
// per workgroup), then its expand half, which loads every slab of its tile
// with y and B in one round and adds them in split order.
// Returns LORA_ERR_UNSPECIFIED, before any launch, when it does not apply
// (no host routing, too many tiles or splits for the launch tables, or too
// small a workspace); the caller then takes the one-kernel path.
lora_status_t run_splitk_short(const Common& c, const void* x, int64_t ldx, const void* A_stack,
                               const void* B_stack, const void* bias, void* y, int64_t ldy, void* workspace,
                               size_t workspace_bytes, int32_t path, hipStream_t s)
{
    if (!c.r.kr)
        return LORA_ERR_UNSPECIFIED;
    const int64_t tiles = fused_host_tiles(c);
    if (tiles == 0)
        return LORA_OK;
    // splits: about one workgroup per compute unit, each wave at least one
    // 32-element step and at most kXLdsSteps (x through LDS)
    constexpr int kWaveK = kFusedWaves * 32;  // K of one step of every wave
    const int units = (c.fs.in_f + kWaveK - 1) / kWaveK;
    int S = (int)std::max<int64_t>(1, (device_cus() + tiles * c.fs.n_s / 2) / (tiles * c.fs.n_s));
    S = std::min(std::max(S, (units + kXLdsSteps - 1) / kXLdsSteps), std::min(units, kFusedWaves));
    while (S > 1 && c.fs.n_s * S > kFusedHostFt)
        --S;
    const int per = (units + S - 1) / S;  // steps per wave
    if (per > kXLdsSteps)
        return LORA_ERR_UNSPECIFIED;
    S = (units + per - 1) / per;
    const int64_t slab = (int64_t)c.r.end * c.fs.C;
    if (!workspace || workspace_bytes < (size_t)S * slab * sizeof(float))
        return LORA_ERR_UNSPECIFIED;
    FusedArgs a;
    fused_common_args(c, a, x, ldx, A_stack, B_stack, bias, y, ldy);
    int64_t rows = 0;
    if (!fused_tile_table(c, a, rows))
        return LORA_ERR_UNSPECIFIED;
    a.F = 0;  // no feature tiles: nothing of y or B is touched
    for (int sl = 0; sl < 4; ++sl)
        a.nft[sl] = 0;
    a.nf = c.fs.n_s * S;
    a.wave_steps = per;
    a.kc = per * kWaveK;
    a.slabs = reinterpret_cast<float*>(workspace);
    a.slab = slab;
    int ft = 0;
    for (int sl = 0; sl < c.fs.n_s; ++sl)
        for (int sp = 0; sp < S; ++sp)
            a.fts[ft++] = make_int2(sl, sp);
    for (; ft < kFusedHostFt; ++ft)
        a.fts[ft] = make_int2(0, 0);
    const dim3 g((unsigned)(kXcds * a.nf), (unsigned)rows), blk(kFusedThreads);
    const bool gather = c.r.rows != nullptr;
    if (c.fs.R == 16) {
        if (gather)
            hipLaunchKernelGGL((fused_delta_kernel<1, 8, true, true, true, kPartShrink>), g, blk, 0, s, a);
        else
            hipLaunchKernelGGL((fused_delta_kernel<1, 8, true, true, false, kPartShrink>), g, blk, 0, s, a);
    } else {
        if (gather)
            hipLaunchKernelGGL((fused_delta_kernel<2, 8, true, true, true, kPartShrink>), g, blk, 0, s, a);
        else
            hipLaunchKernelGGL((fused_delta_kernel<2, 8, true, true, false, kPartShrink>), g, blk, 0, s, a);
    }
    if (hipGetLastError() != hipSuccess)
        return LORA_ERR_DEVICE;
    // the expand half: the same tiles, feature tiles as the one-kernel delta;
    // where 512-wide ones would put more than two workgroups on each compute
    // unit, 1024- or 2048-wide ones (two or four 32-feature pairs per wave):
    // the narrowest that puts at most one workgroup on each compute unit, so
    // that one round of workgroups covers the output
    FusedArgs b = a;
    const int F = fused_widest_feat(c);
    set_fused_feat(c, b, F);
    const int64_t per_xcd = device_cus() / kXcds;
    int pairs = 1;
    if (F == kFusedMaxFeat && rows * b.nf > 2 * per_xcd) {
        for (int p = 2; p <= 4; p *= 2) {
            bool fits = true;
            for (int sl = 0; sl < c.fs.n_s; ++sl)
                fits = fits && c.fs.widths[sl] % (p * kFusedMaxFeat) == 0;
            if (!fits)
                break;
            pairs = p;
            set_fused_feat(c, b, p * kFusedMaxFeat);
            if (rows * b.nf <= per_xcd)
                break;
        }
    }
    if (b.nf > kFusedHostFt)
        return run_expand(c, a.slabs, slab, S, B_stack, bias, y, ldy, path, s);
    fused_feature_tiles(c, b, rows, true, true);
    b.kc = 0;
    b.nsplit = S;
    const dim3 ge((unsigned)(kXcds * b.nf), (unsigned)rows);
#define LORA_EXPAND_HALF(NH, ST, PT)                                                                \
    if (gather)                                                                                     \
        hipLaunchKernelGGL((fused_delta_kernel<NH, ST, false, true, true, PT>), ge, blk, 0, s, b); \
    else                                                                                            \
        hipLaunchKernelGGL((fused_delta_kernel<NH, ST, false, true, false, PT>), ge, blk, 0, s, b);
    if (c.fs.R == 16) {
        if (pairs == 4) {
            LORA_EXPAND_HALF(1, 8, kPartExpand4)
        } else {
            LORA_EXPAND_HALF(1, 8, kPartExpand)
        }
    } else {
        if (pairs == 4) {
            LORA_EXPAND_HALF(2, 4, kPartExpand4)
        } else {
            LORA_EXPAND_HALF(2, 4, kPartExpand)
        }
    }
#undef LORA_EXPAND_HALF
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

bool row_ok(int64_t ld, int64_t width, int elem)
{
    return ld >= width && (ld * elem) % 16 == 0 && ld * elem <= kMaxRowBytes;
}

// Under per-token routing one buffer resource spans all of x or y, and row
// num_rows is the out-of-range row.  Masked lanes use offset kOOB = 2^31, so
// the resource, out-of-range row included, must end below it: otherwise a
// masked lane would read and write back a real row.
bool rows_fit(const Common& c, int64_t ld)
{
    return !c.r.rows || ((int64_t)c.r.nrows + 1) * ld * c.fs.elem <= (int64_t)kOOB;
}

// The one-kernel delta for long groups applies to bf16 families whose u has
// at most 64 columns (ranks 16 to 64), slice widths that are multiples of 64,
// and a host copy of the routing.
bool long_delta_ok(const Common& c)
{
    bool widths64 = true;
    for (int sl = 0; sl < c.fs.n_s; ++sl)
        widths64 = widths64 && c.fs.widths[sl] % 64 == 0;
    const int R = c.fs.R;
    return c.bf16 && c.r.kr && widths64 && c.fs.C <= kLongCols && (R == 16 || R == 32 || R == 64);
}

// AUTO takes it when the batch fills the chip without splitting K (the long
// shrink's plan has one K split), i.e. on prefill-sized batches, and either
// u has at most kLongDeltaAutoC columns or the call brings no workspace
// that the two-kernel path could use (ws_ok false).  With wider u the
// long-segment shrink and the expand in two launches measured faster
// (Llama-3-8B prefill QKV, C 48: 84.1 against 90.6 us; O, C 16: 63.7
// against 59.5 us).  The long_delta option forces it on or off.
constexpr int kLongDeltaAutoC = 16;
bool long_delta_wanted(const Common& c, const ShrinkChoice& ch, bool ws_ok)
{
    if (!long_delta_ok(c) || c.t.long_delta == 0)
        return false;
    return c.t.long_delta > 0 || (ch.lng && (c.fs.C <= kLongDeltaAutoC || !ws_ok));
}

template <int NB, int NH>
void launch_long_delta(bool gather, dim3 grid, hipStream_t s, const LongDeltaArgs& a)
{
    constexpr int D = NB <= 2 ? 3 : 2;
    constexpr int D2 = NH <= 2 ? 2 : 1;
    if (gather && a.bias)
        hipLaunchKernelGGL((delta_long_kernel<NB, NH, D, D2, true, true>), grid, dim3(kLsThreads), 0, s, a);
    else if (gather)
        hipLaunchKernelGGL((delta_long_kernel<NB, NH, D, D2, false, true>), grid, dim3(kLsThreads), 0, s, a);
    else if (a.bias)
        hipLaunchKernelGGL((delta_long_kernel<NB, NH, D, D2, true, false>), grid, dim3(kLsThreads), 0, s, a);
    else
        hipLaunchKernelGGL((delta_long_kernel<NB, NH, D, D2, false, false>), grid, dim3(kLsThreads), 0, s, a);
}

lora_status_t run_long_delta(const Common& c, const ShrinkChoice& ch, const void* x, int64_t ldx,
                             const void* A_stack, const void* B_stack, const void* bias, void* y, int64_t ldy,
                             hipStream_t s)
{
    LongDeltaArgs a;
    a.x = reinterpret_cast<const uint16_t*>(x);
    a.ldx = ldx;
    a.A = reinterpret_cast<const uint16_t*>(A_stack);
    a.a_slot = a_tiled_elems(c.fs.C, c.fs.in_f);
    a.B = reinterpret_cast<const uint16_t*>(B_stack);
    a.bias = reinterpret_cast<const uint16_t*>(bias);
    a.y = reinterpret_cast<uint16_t*>(y);
    a.ldy = ldy;
    a.in_f = c.fs.in_f;
    a.C = c.fs.C;
    a.out_f = c.fs.out_f;
    a.n_s = c.fs.n_s;
    for (int i = 0; i < 5; ++i)
        a.soff[i] = i <= c.fs.n_s ? c.fs.offs[i] : c.fs.out_f;
    a.kw = (c.fs.in_f + kLsKUnit - 1) / kLsKUnit * 32;
    a.fw = (c.fs.out_f + 64 * kLsWaves - 1) / (64 * kLsWaves) * 64;
    a.per_xcd = ch.per_xcd;
    a.pieces = ch.pieces;
    a.r = c.r;
    for (int g = 0; g <= LORA_MAX_HOST_GROUPS; ++g)
        a.k_piece0[g] = g <= c.r.G ? ch.k_piece0[g] : 0;
    const int64_t grid = (int64_t)kXcds * ch.per_xcd;
    if (grid == 0)
        return LORA_OK;
    if (grid > 2147483647LL)
        return LORA_ERR_INVALID_ARGUMENT;
    const bool gather = c.r.rows != nullptr;
    const dim3 g((unsigned)grid);
    const int NH = c.fs.R / 16, NB = c.fs.C / 16;
    if (NB == 1)
        launch_long_delta<1, 1>(gather, g, s, a);
    else if (NB == 2 && NH == 1)
        launch_long_delta<2, 1>(gather, g, s, a);
    else if (NB == 3)
        launch_long_delta<3, 1>(gather, g, s, a);
    else if (NB == 2)
        launch_long_delta<2, 2>(gather, g, s, a);
    else if (NH == 2)
        launch_long_delta<4, 2>(gather, g, s, a);
    else if (NH == 4)
        launch_long_delta<4, 4>(gather, g, s, a);
    else
        return LORA_ERR_UNSPECIFIED;
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

// The delta of one family once the common arguments are checked: the
// one-kernel path (or its split-K form, when a workspace is given and AUTO
// wants it) or the two-kernel path through the workspace.
lora_status_t run_delta(const Common& c, const void* x, int64_t ldx, const void* A_stack, const void* B_stack,
                        const void* bias_stack, void* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                        int32_t path, hipStream_t s)
{
    lora_status_t st;
    // the one-kernel path touches no workspace, so it may be NULL there
    const bool fused = path == LORA_PATH_FUSED || (path == LORA_PATH_AUTO && fused_auto(c));
    if (fused) {
        if (path == LORA_PATH_AUTO && workspace && splitk_short_wanted(c)) {
            st = run_splitk_short(c, x, ldx, A_stack, B_stack, bias_stack, y, ldy, workspace, workspace_bytes,
                                  path, s);
            if (st != LORA_ERR_UNSPECIFIED)
                return st;
        }
        return run_fused(c, x, ldx, A_stack, B_stack, bias_stack, y, ldy, s);
    }
    const ShrinkChoice ch = choose_shrink(c, path);
    if (path == LORA_PATH_AUTO &&
        long_delta_wanted(c, ch, workspace && workspace_bytes >= shrink_need(c, ch, true))) {
        st = run_long_delta(c, ch, x, ldx, A_stack, B_stack, bias_stack, y, ldy, s);
        if (st != LORA_ERR_UNSPECIFIED)
            return st;
    }
    if (!workspace)
        return LORA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < shrink_need(c, ch, true))
        return LORA_ERR_CAPACITY;
    float* slabs = reinterpret_cast<float*>(workspace);
    st = run_shrink_any(c, ch, x, ldx, A_stack, slabs, path, s);
    if (st != LORA_OK)
        return st;
    int S = ch.S();
    const int64_t n4 = (int64_t)c.r.end * c.fs.C / 4;
    // The fold_slabs option adds the slabs into slab 0 in a pass of its own
    // first; by default every feature tile of the expand adds the S slabs of
    // its token tile itself.  The fold paid on long batches while the
    // expand's slab loop waited on every load (32-layer stack, 3.6 K tokens:
    // -5 %); with the expand's batched slab loads it costs 1.7 % there (step
    // 2.535 -> 2.578 ms) and is no longer taken by default.
    if (S > 1 && c.t.fold > 0) {
        hipLaunchKernelGGL(reduce_slabs, dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads),
                           0, s, slabs, n4, S, slabs, n4);
        if (hipGetLastError() != hipSuccess)
            return LORA_ERR_DEVICE;
        S = 1;
    }
    return run_expand(c, slabs, (int64_t)c.r.end * c.fs.C, S, B_stack, bias_stack, y, ldy, path, s);
}

// Argument checks of both delta entry points (all before any launch).
lora_status_t check_delta(const lora_dims_t* dims, int32_t family, const void* x, int64_t ldx, const void* A_stack,
                          const void* B_stack, const void* bias_stack, const lora_routing_t* routing,
                          const void* y, int64_t ldy, int32_t path, const lora_options_t* options, Common* c)
{
    lora_status_t st = check_common(dims, family, path, routing, options, c);
    if (st != LORA_OK)
        return st;
    if ((path == LORA_PATH_MFMA && !(shrink_mfma_ok(*c) && expand_mfma_ok(*c))) ||
        (path == LORA_PATH_FUSED && !fused_ok(*c)))
        return LORA_ERR_INVALID_ARGUMENT;
    if (c->r.end == 0 || c->r.G == 0)
        return LORA_OK;
    if (!x || !A_stack || !B_stack || !y || !row_ok(ldx, c->fs.in_f, c->fs.elem) ||
        !row_ok(ldy, c->fs.out_f, c->fs.elem) || !rows_fit(*c, ldx) || !rows_fit(*c, ldy) || !aligned16(x) ||
        !aligned16(y) || !aligned16(A_stack) || !aligned16(B_stack) || !aligned16(bias_stack))
        return LORA_ERR_INVALID_ARGUMENT;
    return LORA_OK;
}

constexpr size_t kScratchBytes = kNoallocScratchBytes;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (null on failure).
void* scratch_address()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace lora

using namespace lora;

extern "C" {

lora_status_t lora_sgmv_shrink(const lora_dims_t* dims, int32_t family, const void* x, int64_t ldx,
                               const void* A_stack, const lora_routing_t* routing, float* u,
                               void* workspace, size_t workspace_bytes, int32_t path, void* stream)
{
    Common c;
    lora_status_t st = check_common(dims, family, path, routing, nullptr, &c);
    if (st != LORA_OK)
        return st;
    if ((path == LORA_PATH_MFMA && !shrink_mfma_ok(c)) || path == LORA_PATH_FUSED)
        return LORA_ERR_INVALID_ARGUMENT;
    if (c.r.end == 0 || c.r.G == 0)
        return LORA_OK;
    if (!x || !A_stack || !u || !row_ok(ldx, c.fs.in_f, c.fs.elem) || !rows_fit(c, ldx) || !aligned16(x) ||
        !aligned16(A_stack) || !aligned16(u))
        return LORA_ERR_INVALID_ARGUMENT;
    const ShrinkChoice ch = choose_shrink(c, path);
    const size_t need = shrink_need(c, ch, false);
    if (need > 0) {
        if (!workspace || !aligned16(workspace))
            return LORA_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < need)
            return LORA_ERR_CAPACITY;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int S = ch.S();
    float* out = S > 1 ? reinterpret_cast<float*>(workspace) : u;
    st = run_shrink_any(c, ch, x, ldx, A_stack, out, path, s);
    if (st != LORA_OK || S == 1)
        return st;
    const int64_t n4 = (int64_t)c.r.end * c.fs.C / 4;
    hipLaunchKernelGGL(reduce_slabs, dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       s, out, n4, S, u, n4);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

lora_status_t lora_sgmv_expand(const lora_dims_t* dims, int32_t family, const float* u,
                               const void* B_stack, const void* bias_stack, const lora_routing_t* routing,
                               void* y, int64_t ldy, int32_t path, void* stream)
{
    Common c;
    lora_status_t st = check_common(dims, family, path, routing, nullptr, &c);
    if (st != LORA_OK)
        return st;
    if ((path == LORA_PATH_MFMA && !expand_mfma_ok(c)) || path == LORA_PATH_FUSED)
        return LORA_ERR_INVALID_ARGUMENT;
    if (c.r.end == 0 || c.r.G == 0)
        return LORA_OK;
    if (!u || !B_stack || !y || !row_ok(ldy, c.fs.out_f, c.fs.elem) || !rows_fit(c, ldy) || !aligned16(u) ||
        !aligned16(B_stack) || !aligned16(y) || !aligned16(bias_stack))
        return LORA_ERR_INVALID_ARGUMENT;
    return run_expand(c, u, 0, 1, B_stack, bias_stack, y, ldy, path, reinterpret_cast<hipStream_t>(stream));
}

lora_status_t lora_sgmv_delta(const lora_dims_t* dims, int32_t family, const void* x, int64_t ldx,
                              const void* A_stack, const void* B_stack, const void* bias_stack,
                              const lora_routing_t* routing, void* y, int64_t ldy, void* workspace,
                              size_t workspace_bytes, int32_t path, const lora_options_t* options, void* stream)
{
    Common c;
    lora_status_t st =
        check_delta(dims, family, x, ldx, A_stack, B_stack, bias_stack, routing, y, ldy, path, options, &c);
    if (st != LORA_OK || c.r.end == 0 || c.r.G == 0)
        return st;
    if (!aligned16(workspace))
        return LORA_ERR_INVALID_ARGUMENT;
    return run_delta(c, x, ldx, A_stack, B_stack, bias_stack, y, ldy, workspace, workspace_bytes, path,
                     reinterpret_cast<hipStream_t>(stream));
}

size_t lora_sgmv_noalloc_scratch_bytes(void) { return kScratchBytes; }

lora_status_t lora_sgmv_delta_noalloc(const lora_dims_t* dims, int32_t family, const void* x, int64_t ldx,
                                      const void* A_stack, const void* B_stack, const void* bias_stack,
                                      const lora_routing_t* routing, void* y, int64_t ldy, int32_t path,
                                      const lora_options_t* options, void* stream)
{
    Common c;
    lora_status_t st =
        check_delta(dims, family, x, ldx, A_stack, B_stack, bias_stack, routing, y, ldy, path, options, &c);
    if (st != LORA_OK || c.r.end == 0 || c.r.G == 0)
        return st;
    // the two-kernel path's partial sums must fit the scratch array
    const bool fused = path == LORA_PATH_FUSED || (path == LORA_PATH_AUTO && fused_auto(c));
    if (!fused) {
        const ShrinkChoice ch = choose_shrink(c, path);
        const bool fits = shrink_need(c, ch, true) <= kScratchBytes;
        if (!(path == LORA_PATH_AUTO && long_delta_wanted(c, ch, fits)) && !fits)
            return LORA_ERR_CAPACITY;
    }
    void* ws = scratch_address();
    if (!ws)
        return LORA_ERR_DEVICE;
    return run_delta(c, x, ldx, A_stack, B_stack, bias_stack, y, ldy, ws, kScratchBytes, path,
                     reinterpret_cast<hipStream_t>(stream));
}

// Bytes of one slot of each stack: A_qkv, B_qkv, A_o, B_o.
static lora_status_t slot_bytes(const lora_dims_t* dims, size_t b[4])
{
    FamilyShape q, o;
    lora_status_t st = family_shape(dims, LORA_FAMILY_QKV, &q);
    if (st == LORA_OK)
        st = family_shape(dims, LORA_FAMILY_O, &o);
    if (st != LORA_OK)
        return st;
    b[0] = (size_t)a_tiled_elems(q.C, q.in_f) * q.elem;
    b[1] = (size_t)q.out_f * q.R * q.elem;
    b[2] = (size_t)a_tiled_elems(o.C, o.in_f) * o.elem;
    b[3] = (size_t)o.out_f * o.R * o.elem;
    return LORA_OK;
}

lora_status_t lora_write_slot(const lora_dims_t* dims, int32_t slot, const void* A_qkv, const void* B_qkv,
                              const void* A_o, const void* B_o, void* A_qkv_stack, void* B_qkv_stack,
                              void* A_o_stack, void* B_o_stack, void* stream)
{
    size_t b[4];
    const lora_status_t st = slot_bytes(dims, b);
    if (st != LORA_OK)
        return st;
    const void* src[4] = {A_qkv, B_qkv, A_o, B_o};
    void* dst[4] = {A_qkv_stack, B_qkv_stack, A_o_stack, B_o_stack};
    if (slot < 0 || slot >= dims->max_num_loras)
        return LORA_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < 4; ++i)
        if (!src[i] || !dst[i])
            return LORA_ERR_INVALID_ARGUMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int i = 0; i < 4; ++i)
        if (hipMemcpyAsync(reinterpret_cast<char*>(dst[i]) + (size_t)slot * b[i], src[i], b[i],
                           hipMemcpyHostToDevice, s) != hipSuccess)
            return LORA_ERR_DEVICE;
    return LORA_OK;
}

lora_status_t lora_reset_slot(const lora_dims_t* dims, int32_t slot, void* A_qkv_stack, void* B_qkv_stack,
                              void* A_o_stack, void* B_o_stack, void* stream)
{
    size_t b[4];
    const lora_status_t st = slot_bytes(dims, b);
    if (st != LORA_OK)
        return st;
    void* dst[4] = {A_qkv_stack, B_qkv_stack, A_o_stack, B_o_stack};
    if (slot < 0 || slot >= dims->max_num_loras)
        return LORA_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < 4; ++i)
        if (!dst[i] || !aligned16(dst[i]))
            return LORA_ERR_INVALID_ARGUMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int i = 0; i < 4; ++i) {
        // slot sizes are multiples of 16 bytes (widths and ranks are multiples of 8)
        const int64_t n = (int64_t)(b[i] / 16);
        const unsigned grid = (unsigned)std::min<int64_t>((n + kThreads - 1) / kThreads, 1024);
        hipLaunchKernelGGL(zero_words, dim3(grid), dim3(kThreads), 0, s,
                           reinterpret_cast<uint4*>(reinterpret_cast<char*>(dst[i]) + (size_t)slot * b[i]), n);
    }
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

}  // extern "C"
