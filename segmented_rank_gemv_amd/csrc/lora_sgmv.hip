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
#include <stdlib.h>

#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kThreads = 256;

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
// than 2^31 bytes and every masked offset is kOOB plus a small constant.
constexpr uint32_t kOOB = 0x80000000u;

struct Buf {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ Buf(const void* base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000))
    {
    }
    __device__ __forceinline__ uint4 ld16(uint32_t off) const
    {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    }
    __device__ __forceinline__ uint2 ld8(uint32_t off) const
    {
        return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    }
    __device__ __forceinline__ void st8(uint32_t off, uint2 v) const
    {
        typedef unsigned int u32x2 __attribute__((__vector_size__(8)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, 0);
    }
    __device__ __forceinline__ void st16(uint32_t off, uint4 v) const
    {
        typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 0);
    }
};

// 8 consecutive elements of T as fp32
template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
    typedef uint4 Raw;
    static __device__ __forceinline__ Raw load_raw(const Buf& b, uint32_t off) { return b.ld16(off); }
    static __device__ __forceinline__ void store_buf(const Buf& b, uint32_t off, const float* f)
    {
        uint4 v;
        v.x = f2bf_pair(f[0], f[1]);
        v.y = f2bf_pair(f[2], f[3]);
        v.z = f2bf_pair(f[4], f[5]);
        v.w = f2bf_pair(f[6], f[7]);
        b.st16(off, v);
    }
    static __device__ __forceinline__ Raw load_raw(const uint16_t* p) { return ld16(p); }
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
    static __device__ __forceinline__ Raw load_raw(const Buf& b, uint32_t off)
    {
        return Raw{b.ld16(off), b.ld16(off + 16)};
    }
    static __device__ __forceinline__ void store_buf(const Buf& b, uint32_t off, const float* f)
    {
        b.st16(off, make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                               __float_as_uint(f[3])));
        b.st16(off + 16, make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                                    __float_as_uint(f[7])));
    }
    static __device__ __forceinline__ Raw load_raw(const float* p) { return Raw{ld16(p), ld16(p + 4)}; }
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
};

// Locate token tile `tile`: groups are cut into kTileM-token tiles in group
// order.  Every lane takes one group, a wave-wide inclusive scan of the
// per-group tile counts gives each group's first tile and a ballot finds the
// group holding `tile`.  Offsets are clamped into [0, end] and made
// non-decreasing per group, so malformed routing cannot move accesses outside
// rows [0, end).  Returns false past the last tile or for a bad slot id.
__device__ bool locate_tile(const int* __restrict__ offs, const int* __restrict__ ids, int G,
                            int end, int L, int tile, TileInfo& ti)
{
    const int lane = threadIdx.x & 63;
    int base = 0;
    for (int c0 = 0; c0 < G; c0 += 64) {
        const int i = c0 + lane;
        int s = 0, e = 0;
        if (i < G) {
            s = min(max(offs[i], 0), end);
            e = min(max(offs[i + 1], s), end);
        }
        const int nt = (e - s + kTileM - 1) / kTileM;
        const int incl = wave_incl_scan(nt);
        const unsigned long long hit = __ballot(i < G && base + incl > tile);
        if (hit) {
            const int src = __ffsll((long long)hit) - 1;
            const int gs = __shfl(s, src, 64), ge = __shfl(e, src, 64);
            const int first = base + __shfl(incl, src, 64) - __shfl(nt, src, 64);
            // wave-uniform values: keep them in scalar registers
            ti.g = __builtin_amdgcn_readfirstlane(c0 + src);
            ti.t0 = __builtin_amdgcn_readfirstlane(gs + (tile - first) * kTileM);
            ti.n = __builtin_amdgcn_readfirstlane(min(kTileM, ge - gs - (tile - first) * kTileM));
            ti.slot = __builtin_amdgcn_readfirstlane(ids[ti.g]);
            return ti.slot >= 0 && ti.slot < L;
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
    const void* A;  // [L][C][in_f]
    float* out;     // slab s at out + s * slab, each [end][C]; S == 1: u itself
    int64_t slab;
    const int* ids;
    const int* offs;
    int in_f, C, L, G, end;
    int S, kc, nz, cb;
    int valu_max;  // tiles with at most this many tokens take the VALU path
};

// VALU path (decode-shaped tiles, and every fp32 tile).  A wave is four
// 16-lane groups; each group owns one output column at a time and its lanes
// walk K in 8-element runs (128 elements per pass), so a 16-lane wavefront
// reduction finishes every (token, column) dot product.  Columns are taken
// four per group per pass (16 per wave, 64 per workgroup) and tokens eight at
// a time: 12 independent 16-byte loads per pass.  Rows past the tile and
// columns past the group read as zero through the buffer resources.
template <typename T>
__device__ void shrink_valu(const ShrinkArgs& a, const TileInfo& ti, int k0, int k1, int c0,
                            int c1, float* res, int res_ld)
{
    constexpr int E = sizeof(T);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g16 = lane >> 4, l16 = lane & 15;
    const int slot_col = 4 * w + g16;  // 0..15
    const T* X = reinterpret_cast<const T*>(a.x) + (size_t)ti.t0 * a.ldx;
    const T* Ab = reinterpret_cast<const T*>(a.A) + ((size_t)ti.slot * a.C + c0) * a.in_f;
    const Buf xb(X, (uint32_t)(ti.n * a.ldx * E));
    const Buf ab(Ab, (uint32_t)((c1 - c0) * a.in_f * E));
    for (int tb = 0; tb < ti.n; tb += 8) {
        const int nt = min(8, ti.n - tb);
        for (int cb = 0; cb < c1 - c0; cb += 64) {
            float acc[4][8];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[j][i] = 0.f;
            for (int k = k0 + 8 * l16; k < k1; k += 128) {
                float av[4][8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t off = (uint32_t)((cb + slot_col + 16 * j) * a.in_f + k) * E;
                    Vec8<T>::unpack(Vec8<T>::load_raw(ab, off), av[j]);
                }
                typename Vec8<T>::Raw xr[8];  // rows past the tile read as zero
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    xr[i] = Vec8<T>::load_raw(xb, (uint32_t)((tb + i) * a.ldx + k) * E);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (i < nt) {
                        float xv[8];
                        Vec8<T>::unpack(xr[i], xv);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                acc[j][i] = fmaf(av[j][e], xv[e], acc[j][i]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = cb + slot_col + 16 * j;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float v = acc[j][i];
                    v += __shfl_xor(v, 8, 64);
                    v += __shfl_xor(v, 4, 64);
                    v += __shfl_xor(v, 2, 64);
                    v += __shfl_xor(v, 1, 64);
                    if (l16 == 0 && i < nt && c < c1 - c0)
                        res[(tb + i) * res_ld + c] = v;
                }
            }
        }
    }
}

template <int NB>
struct ShrinkFrags {
    uint4 x[4];
    uint4 a[NB];
};

// MFMA path (bf16): the 4 waves take interleaved 32-element K steps
// (k0 + 32 w + 128 j); each wave computes every 16-token x 16-column block
// of the tile with v_mfma_f32_16x16x32_bf16, x rows as the M operand and A
// rows as the N operand, both loaded straight from memory as 16-byte runs.
// Fragments of the next step are loaded before the current step's MFMAs so
// that two steps of loads are in flight per wave.  Wave partials land in
// red[w][token][column].
template <int NB>
__device__ void shrink_mfma(const ShrinkArgs& a, const TileInfo& ti, int k0, int k1, int c0,
                            int c1, float* red, int red_ld)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, q = lane >> 4;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x) + (size_t)ti.t0 * a.ldx;
    const uint16_t* Ab = reinterpret_cast<const uint16_t*>(a.A) + ((size_t)ti.slot * a.C + c0) * a.in_f;
    const Buf xb(X, (uint32_t)(ti.n * a.ldx * 2));
    const Buf ab(Ab, (uint32_t)((c1 - c0) * a.in_f * 2));
    const int mbn = (ti.n + 15) >> 4;

    uint32_t xrow[4], arow[NB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
        xrow[mb] = (uint32_t)((mb * 16 + l16) * a.ldx) * 2;  // rows >= n fall outside xb
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        arow[nb] = (uint32_t)((nb * 16 + l16) * a.in_f) * 2;  // columns >= c1 fall outside ab

    f32x4_t acc[4][NB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto load = [&](int kk, ShrinkFrags<NB>& f) {
        const bool kin = kk < k1;
        const uint32_t kb = 2u * (uint32_t)kk;
        // unconditional loads (rows past the tile read as zero) keep the
        // loop branch-free, so the wait before each MFMA covers only the
        // fragments it consumes
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            f.x[mb] = xb.ld16(kin ? xrow[mb] + kb : kOOB);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            f.a[nb] = ab.ld16(kin ? arow[nb] + kb : kOOB);
    };
    auto mma = [&](const ShrinkFrags<NB>& f) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            if (mb < mbn) {
                const bf16x8_t xv = __builtin_bit_cast(bf16x8_t, f.x[mb]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        xv, __builtin_bit_cast(bf16x8_t, f.a[nb]), acc[mb][nb], 0, 0, 0);
            }
        }
    };

    const int kw = k0 + 32 * w;
    const int steps = kw < k1 ? (k1 - kw + 127) / 128 : 0;
    const int kl = kw + 8 * q;
    // Two fragment sets in flight.  Loads past k1 (the tail of the last pair)
    // read zeros through kOOB, so the loop has no branches around its loads
    // and its MFMAs add nothing for them.
    ShrinkFrags<NB> fa, fb;
    load(kl, fa);
    for (int j = 0; j < steps; j += 2) {
        load(kl + 128 * (j + 1), fb);
        mma(fa);
        load(kl + 128 * (j + 2), fa);
        mma(fb);
    }
    // D[i][j]: lane holds column j = lane%16 and rows 4*(lane/16) + r
    float* my = red + (size_t)w * kTileM * red_ld;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        if (mb < mbn) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    my[(mb * 16 + 4 * q + r) * red_ld + nb * 16 + l16] = acc[mb][nb][r];
        }
    }
}

// One workgroup per (token tile, K split, column group).  With one split the
// result is u itself; with S splits each workgroup writes its split's slab
// and the sum over splits is taken later, in split order, by the expand or
// by reduce_slabs — there is no cross-workgroup synchronisation.
template <typename T, int NB>
__global__ __launch_bounds__(kThreads) void shrink_kernel(ShrinkArgs a)
{
    constexpr int CB = NB * 16;
    constexpr bool kMfma = sizeof(T) == 2;
    __shared__ float red[(kMfma ? 4 : 1) * kTileM * CB];

    const int lin = blockIdx.x;
    const int z = lin % a.nz;
    const int s = (lin / a.nz) % a.S;
    const int tile = lin / (a.nz * a.S);
    TileInfo ti;
    if (!locate_tile(a.offs, a.ids, a.G, a.end, a.L, tile, ti))
        return;
    const int k0 = s * a.kc, k1 = min(k0 + a.kc, a.in_f);
    const int c0 = z * a.cb, c1 = min(c0 + a.cb, a.C);
    const int cw = c1 - c0;

    bool use_mfma = false;
    if constexpr (kMfma) {
        use_mfma = ti.n > a.valu_max;
        if (use_mfma)
            shrink_mfma<NB>(a, ti, k0, k1, c0, c1, red, CB);
        else
            shrink_valu<T>(a, ti, k0, k1, c0, c1, red, CB);
    } else {
        shrink_valu<T>(a, ti, k0, k1, c0, c1, red, CB);
    }
    __syncthreads();

    float* dst = a.out + (size_t)s * a.slab + (size_t)ti.t0 * a.C + c0;
    for (int e = threadIdx.x; e < ti.n * cw; e += kThreads) {
        const int i = e / cw, c = e - i * cw;
        float v = red[i * CB + c];
        if (kMfma && use_mfma)
            v = ((v + red[1 * kTileM * CB + i * CB + c]) + red[2 * kTileM * CB + i * CB + c]) +
                red[3 * kTileM * CB + i * CB + c];
        dst[(size_t)i * a.C + c] = v;
    }
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
// expand

struct ExpandArgs {
    const float* u;  // slab s at u + s * slab, each [end][C]
    int64_t slab;
    int S;
    const void* B;  // [L][out_f][R]
    void* y;
    int64_t ldy;
    const int* ids;
    const int* offs;
    int C, R, L, G, end, n_s, out_f;
    int soff[5];  // slice offsets, soff[n_s] = out_f
    int ft;       // feature tile (divides every slice width)
    int n_ftiles;
    int valu_max;  // tiles with at most this many tokens take the VALU path
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

constexpr int kDeltaPad = 4;  // floats of padding per row of the LDS delta tile

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

// MFMA delta of the tile into LDS (bf16).  The tile's (16-token x 16-feature)
// blocks are dealt to the 4 waves round-robin.  For each block one
// v_mfma_f32_16x16x32_bf16 per 16 ranks computes B·u with K = 32 = 16 ranks
// of the high bf16 half of u followed by the same 16 ranks of its low half
// (u = hi + lo to ~2^-17 relative), so u keeps fp32 precision while the
// products run on the bf16 matrix cores.  B rows are the M operand
// (features), u the N operand (tokens).  bfr holds the B fragments, loaded
// before u was staged.
template <int NH>
__device__ __forceinline__ void mfma_delta(const ExpandArgs& a, const TileInfo& ti,
                                           const uint4 (&bfr)[8][NH], const float* us, float* dl,
                                           int dl_ld)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, q = lane >> 4;
    const int nfb = a.ft >> 4;
    const int nblk = ((ti.n + 15) >> 4) * nfb;
    int cur_tb = -1;
    bf16x8_t uf[NH];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int b = w + 4 * i;
        if (b < nblk) {
            const int tb = b / nfb, fb = b - tb * nfb;
            const int t = tb * 16 + l16;
            if (tb != cur_tb) {
                cur_tb = tb;
                // lanes q<2 carry hi(u[t][16h+8q..]), lanes q>=2 lo(u[t][16h+8(q-2)..])
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    float v[8];
                    const float* up = us + min(t, ti.n - 1) * a.R + 16 * h + 8 * (q & 1);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[e] = up[e];
                    uint32_t pk[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint32_t hi = f2bf_pair(v[2 * e], v[2 * e + 1]);
                        if (q >= 2)
                            hi = f2bf_pair(v[2 * e] - bf2f(hi & 0xFFFFu), v[2 * e + 1] - bf2f(hi >> 16));
                        pk[e] = hi;
                    }
                    uf[h] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
                }
            }
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int h = 0; h < NH; ++h)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bfr[i][h]), uf[h],
                                                             acc, 0, 0, 0);
            // D[i][j]: lane holds token j = lane%16, features 4*(lane/16) + r
            *reinterpret_cast<f32x4_t*>(dl + t * dl_ld + fb * 16 + 4 * q) = acc;
        }
    }
}

// One workgroup per (token tile, feature tile).  Thread (rr, fl) owns
// features f0 + 8 fl .. +8 of rows rr, rr + RP, ... (RP = rows per pass), so
// every y access is a 16-byte run and a wave covers whole row segments.  The
// y rows are loaded first, then u is staged; the delta comes from MFMA (long
// bf16 tiles, through an LDS tile) or from VALU FMAs in registers (short
// tiles and fp32); y + delta is rounded once and stored.
// NH = R / 16 when the MFMA path may run (bf16, R <= 64, slice widths multiple
// of 16); NH = 0 builds the VALU path alone.
template <typename T, int NH>
__global__ __launch_bounds__(kThreads) void expand_kernel(ExpandArgs a)
{
    constexpr int E = sizeof(T);
    constexpr int kRows = 4;  // row passes per thread (feature tile <= 128)
    extern __shared__ float smem[];
    float* us = smem;                                        // [kTileM][R]
    float4* part = reinterpret_cast<float4*>(us + kTileM * a.R);  // [kThreads] float4
    float* dl = reinterpret_cast<float*>(part + kThreads);        // [kTileM][ft + pad]
    const int dl_ld = a.ft + kDeltaPad;

    const int lin = blockIdx.x;
    const int ftile = lin % a.n_ftiles;
    const int tile = lin / a.n_ftiles;
    TileInfo ti;
    if (!locate_tile(a.offs, a.ids, a.G, a.end, a.L, tile, ti))
        return;
    const int f0 = ftile * a.ft;
    const int fgroups = a.ft >> 3;
    const int rp = kThreads / fgroups;
    const int fl = threadIdx.x % fgroups, rr = threadIdx.x / fgroups;
    const int f = f0 + 8 * fl;
    const Buf yb(reinterpret_cast<const T*>(a.y) + (size_t)ti.t0 * a.ldy, (uint32_t)(ti.n * a.ldy * E));

    typename Vec8<T>::Raw yraw[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int row = rr + i * rp;
        yraw[i] = Vec8<T>::load_raw(yb, row < ti.n ? (uint32_t)(row * a.ldy + f) * E : kOOB);
    }

    float delta[kRows][8];
#pragma unroll
    for (int i = 0; i < kRows; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            delta[i][e] = 0.f;

    const int ucol0 = slice_of(a, f0) * a.R;
    bool mfma_done = false;
    if constexpr (NH > 0) {
        if (ti.n > a.valu_max) {
            // B fragments of this wave's blocks: lane (l16, q) holds
            // B[fb*16 + l16][16h + 8(q&1) .. +8]
            const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
            const int l16 = lane & 15, q = lane >> 4;
            const int nfb = a.ft >> 4;
            const int nblk = ((ti.n + 15) >> 4) * nfb;
            const uint16_t* Bb = reinterpret_cast<const uint16_t*>(a.B) + ((size_t)ti.slot * a.out_f + f0) * a.R;
            uint4 bfr[8][NH];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int b = w + 4 * i;
                const int fb = (b < nblk ? b : 0) % nfb;
#pragma unroll
                for (int h = 0; h < NH; ++h)
                    bfr[i][h] = ld16(Bb + (size_t)(fb * 16 + l16) * a.R + 16 * h + 8 * (q & 1));
            }
            stage_u(a, ti, ucol0, us, part);
            __syncthreads();
            mfma_delta<NH>(a, ti, bfr, us, dl, dl_ld);
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kRows; ++i) {
                const int row = rr + i * rp;
                if (row < ti.n) {
                    const float* dp = dl + row * dl_ld + 8 * fl;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        delta[i][e] = dp[e];
                }
            }
            mfma_done = true;
        }
    }
    if (!mfma_done) {
        stage_u(a, ti, ucol0, us, part);
        __syncthreads();
        // VALU: delta[i][ff] = sum_j B[f + ff][j] * u[row_i][j], B read 8 ranks at a time
        const T* Bb = reinterpret_cast<const T*>(a.B) + ((size_t)ti.slot * a.out_f + f) * a.R;
        for (int j0 = 0; j0 < a.R; j0 += 8) {
            float bv[8][8];  // [feature][rank]
#pragma unroll
            for (int ff = 0; ff < 8; ++ff)
                Vec8<T>::load(Bb + (size_t)ff * a.R + j0, bv[ff]);
#pragma unroll
            for (int i = 0; i < kRows; ++i) {
                const int row = rr + i * rp;
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
    }
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int row = rr + i * rp;
        if (row < ti.n) {
            float out[8];
            Vec8<T>::unpack(yraw[i], out);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                out[e] += delta[i][e];
            Vec8<T>::store_buf(yb, (uint32_t)(row * a.ldy + f) * E, out);
        }
    }
}

// ---------------------------------------------------------------------------
// launch helpers

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Default VALU/MFMA split (tokens per tile); overridable for tuning through
// LORA_SGMV_VALU_MAX_SHRINK / LORA_SGMV_VALU_MAX_EXPAND.
int env_int(const char* name, int dflt)
{
    const char* v = getenv(name);
    if (!v || !*v)
        return dflt;
    return atoi(v);
}

int valu_max_for(int path, bool mfma_ok, int dflt_auto)
{
    if (!mfma_ok || path == LORA_PATH_VALU)
        return kTileM;  // every tile on the VALU path
    if (path == LORA_PATH_MFMA)
        return 0;
    return dflt_auto;
}

template <typename T>
hipError_t launch_shrink(const ShrinkArgs& a, int nb, int grid, hipStream_t st)
{
    switch (nb) {
    case 1: hipLaunchKernelGGL((shrink_kernel<T, 1>), dim3(grid), dim3(kThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((shrink_kernel<T, 2>), dim3(grid), dim3(kThreads), 0, st, a); break;
    case 3: hipLaunchKernelGGL((shrink_kernel<T, 3>), dim3(grid), dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((shrink_kernel<T, 4>), dim3(grid), dim3(kThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

struct Common {
    FamilyShape fs;
    bool bf16;
};

lora_status_t check_common(const lora_dims_t* dims, int32_t family, int32_t path, int32_t num_groups,
                           int64_t end, Common* c)
{
    lora_status_t st = family_shape(dims, family, &c->fs);
    if (st != LORA_OK)
        return st;
    if (path < LORA_PATH_AUTO || path > LORA_PATH_MFMA)
        return LORA_ERR_INVALID_ARGUMENT;
    c->bf16 = dims->dtype == LORA_DTYPE_BF16;
    if (end < 0 || end > 2147483647LL || num_groups < 0 || num_groups > c->fs.L)
        return LORA_ERR_INVALID_ARGUMENT;
    return LORA_OK;
}

bool shrink_mfma_ok(const Common& c) { return c.bf16; }

bool expand_mfma_ok(const Common& c)
{
    bool widths16 = true;
    for (int s = 0; s < c.fs.n_s; ++s)
        widths16 = widths16 && c.fs.widths[s] % 16 == 0;
    return c.bf16 && c.fs.R % 16 == 0 && c.fs.R <= 64 && widths16;
}

// shrink launch; `out` receives u (S == 1) or the S slabs
lora_status_t run_shrink(const Common& c, const ShrinkPlan& plan, const void* x, int64_t ldx,
                         const void* A_stack, const int32_t* ids, const int32_t* offs, int G,
                         int64_t end, float* out, int32_t path, hipStream_t s)
{
    ShrinkArgs a;
    a.x = x;
    a.ldx = ldx;
    a.A = A_stack;
    a.out = out;
    a.slab = end * c.fs.C;
    a.ids = ids;
    a.offs = offs;
    a.in_f = c.fs.in_f;
    a.C = c.fs.C;
    a.L = c.fs.L;
    a.G = G;
    a.end = (int)end;
    a.S = plan.S;
    a.kc = plan.kc;
    a.nz = plan.nz;
    a.cb = plan.cb;
    a.valu_max = valu_max_for(path, shrink_mfma_ok(c), env_int("LORA_SGMV_VALU_MAX_SHRINK", 8));
    const int64_t grid = (int64_t)plan.n_tiles * plan.S * plan.nz;
    if (grid > 2147483647LL)
        return LORA_ERR_INVALID_ARGUMENT;
    const hipError_t e = c.bf16 ? launch_shrink<uint16_t>(a, plan.cb / 16, (int)grid, s)
                                : launch_shrink<float>(a, plan.cb / 16, (int)grid, s);
    return e == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

bool nh_possible(const Common& c, const ExpandArgs& a) { return expand_mfma_ok(c) && a.valu_max < kTileM; }

lora_status_t run_expand(const Common& c, const float* u, int64_t slab, int S, const void* B_stack,
                         const int32_t* ids, const int32_t* offs, int G, int64_t end, void* y,
                         int64_t ldy, int32_t path, hipStream_t s)
{
    ExpandArgs a;
    a.u = u;
    a.slab = slab;
    a.S = S;
    a.B = B_stack;
    a.y = y;
    a.ldy = ldy;
    a.ids = ids;
    a.offs = offs;
    a.C = c.fs.C;
    a.R = c.fs.R;
    a.L = c.fs.L;
    a.G = G;
    a.end = (int)end;
    a.n_s = c.fs.n_s;
    a.out_f = c.fs.out_f;
    for (int i = 0; i < 5; ++i)
        a.soff[i] = i <= c.fs.n_s ? c.fs.offs[i] : c.fs.out_f;
    a.ft = expand_tile(c.fs);
    a.n_ftiles = c.fs.out_f / a.ft;
    a.valu_max = valu_max_for(path, expand_mfma_ok(c), env_int("LORA_SGMV_VALU_MAX_EXPAND", 8));
    const int64_t tiles = (end + kTileM - 1) / kTileM + G;
    const int64_t grid = tiles * a.n_ftiles;
    if (grid > 2147483647LL)
        return LORA_ERR_INVALID_ARGUMENT;
    const size_t lds = (size_t)kTileM * c.fs.R * sizeof(float) + kThreads * sizeof(float4) +
                       (nh_possible(c, a) ? (size_t)kTileM * (a.ft + kDeltaPad) * sizeof(float) : 0);
    const dim3 g((unsigned)grid), b(kThreads);
    const int nh = nh_possible(c, a) ? c.fs.R / 16 : 0;
    if (!c.bf16)
        hipLaunchKernelGGL((expand_kernel<float, 0>), g, b, lds, s, a);
    else if (nh == 1)
        hipLaunchKernelGGL((expand_kernel<uint16_t, 1>), g, b, lds, s, a);
    else if (nh == 2)
        hipLaunchKernelGGL((expand_kernel<uint16_t, 2>), g, b, lds, s, a);
    else if (nh == 3)
        hipLaunchKernelGGL((expand_kernel<uint16_t, 3>), g, b, lds, s, a);
    else if (nh == 4)
        hipLaunchKernelGGL((expand_kernel<uint16_t, 4>), g, b, lds, s, a);
    else
        hipLaunchKernelGGL((expand_kernel<uint16_t, 0>), g, b, lds, s, a);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

}  // namespace
}  // namespace lora

using namespace lora;

extern "C" {

lora_status_t lora_sgmv_shrink(const lora_dims_t* dims, int32_t family, const void* x, int64_t ldx,
                               const void* A_stack, const int32_t* lora_ids,
                               const int32_t* grouped_offsets, int32_t num_groups, int64_t end,
                               float* u, void* workspace, size_t workspace_bytes, int32_t path,
                               void* stream)
{
    Common c;
    lora_status_t st = check_common(dims, family, path, num_groups, end, &c);
    if (st != LORA_OK)
        return st;
    if (path == LORA_PATH_MFMA && !shrink_mfma_ok(c))
        return LORA_ERR_INVALID_ARGUMENT;
    if (end == 0 || num_groups == 0)
        return LORA_OK;
    if (!x || !A_stack || !lora_ids || !grouped_offsets || !u)
        return LORA_ERR_INVALID_ARGUMENT;
    if (ldx < c.fs.in_f || (ldx * c.fs.elem) % 16 || ldx * c.fs.elem > kMaxRowBytes || !aligned16(x) ||
        !aligned16(A_stack) || !aligned16(u))
        return LORA_ERR_INVALID_ARGUMENT;
    const ShrinkPlan plan = plan_shrink(c.fs, end, num_groups);
    const size_t need = shrink_workspace(plan);
    if (need > 0) {
        if (!workspace || !aligned16(workspace))
            return LORA_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < need)
            return LORA_ERR_CAPACITY;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    float* out = plan.S > 1 ? reinterpret_cast<float*>(workspace) : u;
    st = run_shrink(c, plan, x, ldx, A_stack, lora_ids, grouped_offsets, num_groups, end, out, path, s);
    if (st != LORA_OK || plan.S == 1)
        return st;
    const int64_t n4 = end * c.fs.C / 4;
    hipLaunchKernelGGL(reduce_slabs, dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       s, out, (int64_t)(end * c.fs.C / 4), plan.S, u, n4);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

lora_status_t lora_sgmv_expand(const lora_dims_t* dims, int32_t family, const float* u,
                               const void* B_stack, const int32_t* lora_ids,
                               const int32_t* grouped_offsets, int32_t num_groups, int64_t end,
                               void* y, int64_t ldy, int32_t path, void* stream)
{
    Common c;
    lora_status_t st = check_common(dims, family, path, num_groups, end, &c);
    if (st != LORA_OK)
        return st;
    if (path == LORA_PATH_MFMA && !expand_mfma_ok(c))
        return LORA_ERR_INVALID_ARGUMENT;
    if (end == 0 || num_groups == 0)
        return LORA_OK;
    if (!u || !B_stack || !lora_ids || !grouped_offsets || !y)
        return LORA_ERR_INVALID_ARGUMENT;
    if (ldy < c.fs.out_f || (ldy * c.fs.elem) % 16 || ldy * c.fs.elem > kMaxRowBytes || !aligned16(u) ||
        !aligned16(B_stack) || !aligned16(y))
        return LORA_ERR_INVALID_ARGUMENT;
    return run_expand(c, u, 0, 1, B_stack, lora_ids, grouped_offsets, num_groups, end, y, ldy, path,
                      reinterpret_cast<hipStream_t>(stream));
}

lora_status_t lora_sgmv_delta(const lora_dims_t* dims, int32_t family, const void* x, int64_t ldx,
                              const void* A_stack, const void* B_stack, const int32_t* lora_ids,
                              const int32_t* grouped_offsets, int32_t num_groups, int64_t end,
                              void* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                              int32_t path, void* stream)
{
    Common c;
    lora_status_t st = check_common(dims, family, path, num_groups, end, &c);
    if (st != LORA_OK)
        return st;
    if (path == LORA_PATH_MFMA && !(shrink_mfma_ok(c) && expand_mfma_ok(c)))
        return LORA_ERR_INVALID_ARGUMENT;
    if (end == 0 || num_groups == 0)
        return LORA_OK;
    if (!x || !A_stack || !B_stack || !lora_ids || !grouped_offsets || !y || !workspace)
        return LORA_ERR_INVALID_ARGUMENT;
    if (ldx < c.fs.in_f || (ldx * c.fs.elem) % 16 || ldy < c.fs.out_f || (ldy * c.fs.elem) % 16 ||
        ldx * c.fs.elem > kMaxRowBytes || ldy * c.fs.elem > kMaxRowBytes || !aligned16(x) ||
        !aligned16(y) || !aligned16(A_stack) || !aligned16(B_stack) || !aligned16(workspace))
        return LORA_ERR_INVALID_ARGUMENT;
    const ShrinkPlan plan = plan_shrink(c.fs, end, num_groups);
    if (workspace_bytes < delta_workspace(plan))
        return LORA_ERR_CAPACITY;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    float* slabs = reinterpret_cast<float*>(workspace);
    st = run_shrink(c, plan, x, ldx, A_stack, lora_ids, grouped_offsets, num_groups, end, slabs, path, s);
    if (st != LORA_OK)
        return st;
    int S = plan.S;
    if (S > 1 && env_int("LORA_SGMV_DELTA_REDUCE", 0)) {
        // fold the slabs into slab 0 first (tuning switch: one extra launch,
        // the expand then stages a single slab)
        const int64_t n4 = end * c.fs.C / 4;
        hipLaunchKernelGGL(reduce_slabs, dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads),
                           0, s, slabs, n4, S, slabs, n4);
        if (hipGetLastError() != hipSuccess)
            return LORA_ERR_DEVICE;
        S = 1;
    }
    return run_expand(c, slabs, end * c.fs.C, S, B_stack, lora_ids, grouped_offsets, num_groups, end,
                      y, ldy, path, s);
}

}  // extern "C"
