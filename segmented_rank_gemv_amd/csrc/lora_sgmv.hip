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
// shrink streams one A row per wave with lanes along K and finishes with
// wavefront reductions; the expand keeps B rows in registers and streams
// y.  Longer bf16 tiles are real dense contractions and use
// v_mfma_f32_16x16x32_bf16.  Both read x, A, B and y with 16-byte vector loads.
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

// 8 consecutive elements of T as fp32
template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
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

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        v += __shfl_xor(v, d, 64);
    return v;
}

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
            ti.g = c0 + src;
            ti.t0 = gs + (tile - first) * kTileM;
            ti.n = min(kTileM, ge - ti.t0);
            ti.slot = ids[ti.g];
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
    const void* A;       // [L][C][in_f]
    float* u;            // [end][C]
    float* partial;      // [n_tiles][S][kTileM][C]   (S > 1)
    uint32_t* counters;  // [n_tiles][nz]             (S > 1)
    const int* ids;
    const int* offs;
    int in_f, C, L, G, end;
    int S, kc, nz, cb, n_tiles;
    int valu_max;  // tiles with at most this many tokens take the VALU path
};

// VALU path: wave w owns columns c0+w, c0+w+4, ...; lanes cover 8 consecutive
// k each (512 per wave step); tokens in groups of 8; one wavefront reduction
// per (token, column).  Results go to res[token][column - c0].
template <typename T>
__device__ void shrink_valu(const ShrinkArgs& a, const TileInfo& ti, int k0, int k1, int c0,
                            int c1, float* res, int res_ld)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const T* X = reinterpret_cast<const T*>(a.x);
    const T* Ab = reinterpret_cast<const T*>(a.A) + (size_t)ti.slot * a.C * a.in_f;
    for (int tb = 0; tb < ti.n; tb += 8) {
        const int nt = min(8, ti.n - tb);
        for (int c = c0 + w; c < c1; c += 4) {
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = 0.f;
            for (int k = k0 + 8 * lane; k < k1; k += 512) {
                float av[8];
                Vec8<T>::load(Ab + (size_t)c * a.in_f + k, av);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (i < nt) {
                        float xv[8];
                        Vec8<T>::load(X + (size_t)(ti.t0 + tb + i) * a.ldx + k, xv);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[i] = fmaf(av[e], xv[e], acc[i]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i < nt) {
                    const float v = wave_sum(acc[i]);
                    if (lane == 0)
                        res[(tb + i) * res_ld + (c - c0)] = v;
                }
            }
        }
    }
}

// MFMA path (bf16): the 4 waves take interleaved 32-element K steps; each
// wave computes every 16-token block x 16-column block of the tile with
// v_mfma_f32_16x16x32_bf16 (x rows as the M operand, A rows as the N
// operand, both loaded straight from HBM as 16-byte K runs).  Wave partials
// land in red[w][token][column].
template <int NB>
__device__ void shrink_mfma(const ShrinkArgs& a, const TileInfo& ti, int k0, int k1, int c0,
                            int c1, float* red, int red_ld)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, q = lane >> 4;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* Ab = reinterpret_cast<const uint16_t*>(a.A) + (size_t)ti.slot * a.C * a.in_f;
    const int mbn = (ti.n + 15) >> 4;
    f32x4_t acc[4][NB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint4 zero = make_uint4(0, 0, 0, 0);
    for (int k = k0 + 32 * w; k < k1; k += 128) {
        const int kk = k + 8 * q;
        const bool kin = kk < k1;
        bf16x8_t xf[4], af[NB];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int i = mb * 16 + l16;
            uint4 v = zero;
            if (mb < mbn && i < ti.n && kin)
                v = ld16(X + (size_t)(ti.t0 + i) * a.ldx + kk);
            xf[mb] = __builtin_bit_cast(bf16x8_t, v);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int c = c0 + nb * 16 + l16;
            uint4 v = zero;
            if (c < c1 && kin)
                v = ld16(Ab + (size_t)c * a.in_f + kk);
            af[nb] = __builtin_bit_cast(bf16x8_t, v);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            if (mb < mbn) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[mb], af[nb], acc[mb][nb],
                                                                         0, 0, 0);
            }
        }
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

template <typename T, int NB>
__global__ __launch_bounds__(kThreads) void shrink_kernel(ShrinkArgs a)
{
    constexpr int CB = NB * 16;
    constexpr bool kMfma = sizeof(T) == 2;
    __shared__ float red[(kMfma ? 4 : 1) * kTileM * CB];
    __shared__ int s_last;

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

    const bool use_mfma = kMfma && ti.n > a.valu_max;
    if constexpr (kMfma) {
        if (use_mfma)
            shrink_mfma<NB>(a, ti, k0, k1, c0, c1, red, CB);
        else
            shrink_valu<T>(a, ti, k0, k1, c0, c1, red, CB);
    } else {
        shrink_valu<T>(a, ti, k0, k1, c0, c1, red, CB);
    }
    __syncthreads();

    // the tile's [n][cw] result: u directly, or this split's partial
    float* dst;
    int64_t dst_ld;
    if (a.S == 1) {
        dst = a.u + (size_t)ti.t0 * a.C + c0;
        dst_ld = a.C;
    } else {
        dst = a.partial + ((size_t)(tile * a.S + s) * kTileM) * a.C + c0;
        dst_ld = a.C;
    }
    for (int e = threadIdx.x; e < ti.n * cw; e += kThreads) {
        const int i = e / cw, c = e - i * cw;
        float v = red[i * CB + c];
        if (kMfma && use_mfma)
            v = ((v + red[1 * kTileM * CB + i * CB + c]) + red[2 * kTileM * CB + i * CB + c]) +
                red[3 * kTileM * CB + i * CB + c];
        dst[(size_t)i * dst_ld + c] = v;
    }
    if (a.S == 1)
        return;

    // split-K: the last split to arrive sums the S partials in split order
    // (deterministic) and re-arms the counter for the next call
    __threadfence();
    __syncthreads();
    uint32_t* ctr = a.counters + (size_t)tile * a.nz + z;
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(a.S - 1);
    }
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();
    const float* part = a.partial + (size_t)tile * a.S * kTileM * a.C + c0;
    const size_t split_stride = (size_t)kTileM * a.C;
    float* u = a.u + (size_t)ti.t0 * a.C + c0;
    for (int e = threadIdx.x; e < ti.n * cw; e += kThreads) {
        const int i = e / cw, c = e - i * cw;
        const float* p = part + (size_t)i * a.C + c;
        float v = 0.f;
#pragma unroll 8
        for (int ss = 0; ss < a.S; ++ss)
            v += p[ss * split_stride];
        u[(size_t)i * a.C + c] = v;
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// expand

struct ExpandArgs {
    const float* u;  // [end][C]
    const void* B;   // [L][out_f][R]
    void* y;
    int64_t ldy;
    const int* ids;
    const int* offs;
    int C, R, L, G, end, n_s, out_f;
    int soff[5];  // slice offsets, soff[n_s] = out_f
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

// VALU path: thread (tg, fl) owns features f0+8*fl .. +8 and tokens
// tg, tg+8, ... of the tile.  B is read 8 ranks at a time into registers and
// reused for every token; u rows are broadcast loads.
template <typename T>
__device__ void expand_valu(const ExpandArgs& a, const TileInfo& ti, int f0, int f1)
{
    const int fl = threadIdx.x & 31, tg = threadIdx.x >> 5;
    const int f = f0 + 8 * fl;
    if (f >= f1)
        return;
    const int sl = slice_of(a, f);
    const T* Bb = reinterpret_cast<const T*>(a.B) + ((size_t)ti.slot * a.out_f + f) * a.R;
    T* Y = reinterpret_cast<T*>(a.y);
    const float* U = a.u + (size_t)ti.t0 * a.C + sl * a.R;

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = 0.f;

    for (int j0 = 0; j0 < a.R; j0 += 8) {
        float bv[8][8];  // [feature][rank]
#pragma unroll
        for (int ff = 0; ff < 8; ++ff)
            Vec8<T>::load(Bb + (size_t)ff * a.R + j0, bv[ff]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = tg + 8 * i;
            if (t < ti.n) {
                float uv[8];
                Vec8<float>::load(U + (size_t)t * a.C + j0, uv);
#pragma unroll
                for (int ff = 0; ff < 8; ++ff)
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
                        acc[i][ff] = fmaf(bv[ff][jj], uv[jj], acc[i][ff]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = tg + 8 * i;
        if (t < ti.n) {
            T* yp = Y + (size_t)(ti.t0 + t) * a.ldy + f;
            float yv[8];
            Vec8<T>::load(yp, yv);
#pragma unroll
            for (int ff = 0; ff < 8; ++ff)
                yv[ff] += acc[i][ff];
            Vec8<T>::store(yp, yv);
        }
    }
}

// MFMA path (bf16): wave w owns tokens 16w..16w+15 of the tile and walks the
// feature tile in 16-feature blocks.  Per 16 ranks one
// v_mfma_f32_16x16x32_bf16 computes B·u with K = 32 = 16 ranks of the high
// bf16 part of u followed by the same 16 ranks of its low part
// (u = hi + lo to ~2^-17 relative), so fp32 u keeps its precision while the
// products run on bf16 matrix cores.  B rows are the M operand (features),
// u the N operand (tokens); the C operand is y itself, so the accumulator
// layout (4 consecutive features of one token per lane) is also the y access
// pattern.
template <int NH>
__device__ void expand_mfma(const ExpandArgs& a, const TileInfo& ti, int f0, int f1)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, q = lane >> 4;
    if (16 * w >= ti.n)
        return;
    const int t = 16 * w + l16;
    const bool tval = t < ti.n;
    const uint16_t* Bb = reinterpret_cast<const uint16_t*>(a.B) + (size_t)ti.slot * a.out_f * a.R;
    uint16_t* Y = reinterpret_cast<uint16_t*>(a.y);
    int cur = -1;
    bf16x8_t uf[NH];  // one fragment per 16 ranks
    for (int fb = f0; fb < f1; fb += 16) {
        const int sl = slice_of(a, fb);
        if (sl != cur) {
            cur = sl;
            // u fragment: lanes q<2 carry hi(u[t][16h+8q..]), q>=2 lo(u[t][16h+8(q-2)..])
            const float* up = a.u + (size_t)(ti.t0 + t) * a.C + sl * a.R + 8 * (q & 1);
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                float v[8];
                if (tval)
                    Vec8<float>::load(up + 16 * h, v);
                else
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[e] = 0.f;
                uint32_t p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t hi = f2bf_pair(v[2 * e], v[2 * e + 1]);
                    if (q >= 2) {
                        const float r0 = v[2 * e] - bf2f(hi & 0xFFFFu);
                        const float r1 = v[2 * e + 1] - bf2f(hi >> 16);
                        hi = f2bf_pair(r0, r1);
                    }
                    p[e] = hi;
                }
                uf[h] = __builtin_bit_cast(bf16x8_t, make_uint4(p[0], p[1], p[2], p[3]));
            }
        }
        // y: 4 consecutive features of token t
        uint16_t* yp = Y + (size_t)(ti.t0 + t) * a.ldy + fb + 4 * q;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (tval) {
            uint2 yv = *reinterpret_cast<const uint2*>(yp);
            acc[0] = bf2f(yv.x & 0xFFFFu);
            acc[1] = bf2f(yv.x >> 16);
            acc[2] = bf2f(yv.y & 0xFFFFu);
            acc[3] = bf2f(yv.y >> 16);
        }
        const uint16_t* bp = Bb + (size_t)(fb + l16) * a.R + 8 * (q & 1);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, ld16(bp + 16 * h));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, uf[h], acc, 0, 0, 0);
        }
        if (tval) {
            uint2 o;
            o.x = f2bf_pair(acc[0], acc[1]);
            o.y = f2bf_pair(acc[2], acc[3]);
            *reinterpret_cast<uint2*>(yp) = o;
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void expand_kernel(ExpandArgs a)
{
    const int lin = blockIdx.x;
    const int ft = lin % a.n_ftiles;
    const int tile = lin / a.n_ftiles;
    TileInfo ti;
    if (!locate_tile(a.offs, a.ids, a.G, a.end, a.L, tile, ti))
        return;
    const int f0 = ft * kExpandCols, f1 = min(f0 + kExpandCols, a.out_f);
    if constexpr (sizeof(T) == 2) {
        if (ti.n > a.valu_max) {
            switch (a.R >> 4) {
            case 1: expand_mfma<1>(a, ti, f0, f1); break;
            case 2: expand_mfma<2>(a, ti, f0, f1); break;
            case 3: expand_mfma<3>(a, ti, f0, f1); break;
            default: expand_mfma<4>(a, ti, f0, f1); break;
            }
            return;
        }
    }
    expand_valu<T>(a, ti, f0, f1);
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

int valu_max_for(int path, bool bf16, int dflt_auto)
{
    if (!bf16 || path == LORA_PATH_VALU)
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
    FamilyShape fs;
    lora_status_t st = family_shape(dims, family, &fs);
    if (st != LORA_OK)
        return st;
    if (path < LORA_PATH_AUTO || path > LORA_PATH_MFMA)
        return LORA_ERR_INVALID_ARGUMENT;
    const bool bf16 = dims->dtype == LORA_DTYPE_BF16;
    if (path == LORA_PATH_MFMA && (!bf16 || fs.R % 16))
        return LORA_ERR_INVALID_ARGUMENT;
    if (end < 0 || end > 2147483647LL || num_groups < 0 || num_groups > fs.L)
        return LORA_ERR_INVALID_ARGUMENT;
    if (end == 0 || num_groups == 0)
        return LORA_OK;
    if (!x || !A_stack || !lora_ids || !grouped_offsets || !u)
        return LORA_ERR_INVALID_ARGUMENT;
    if (ldx < fs.in_f || (ldx * fs.elem) % 16 || !aligned16(x) || !aligned16(A_stack) ||
        !aligned16(u))
        return LORA_ERR_INVALID_ARGUMENT;
    ShrinkPlan plan = plan_shrink(fs, end, num_groups);
    const size_t need = plan.counter_bytes + plan.partial_bytes;
    if (need > 0) {
        if (!workspace || !aligned16(workspace))
            return LORA_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < need)
            return LORA_ERR_CAPACITY;
    }
    ShrinkArgs a;
    a.x = x;
    a.ldx = ldx;
    a.A = A_stack;
    a.u = u;
    a.counters = reinterpret_cast<uint32_t*>(workspace);
    a.partial = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + plan.counter_bytes);
    a.ids = lora_ids;
    a.offs = grouped_offsets;
    a.in_f = fs.in_f;
    a.C = fs.C;
    a.L = fs.L;
    a.G = num_groups;
    a.end = (int)end;
    a.S = plan.S;
    a.kc = plan.kc;
    a.nz = plan.nz;
    a.cb = plan.cb;
    a.n_tiles = plan.n_tiles;
    a.valu_max = valu_max_for(path, bf16, env_int("LORA_SGMV_VALU_MAX_SHRINK", 8));
    const int64_t grid = (int64_t)plan.n_tiles * plan.S * plan.nz;
    if (grid > 2147483647LL)
        return LORA_ERR_INVALID_ARGUMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = bf16 ? launch_shrink<uint16_t>(a, plan.cb / 16, (int)grid, s)
                              : launch_shrink<float>(a, plan.cb / 16, (int)grid, s);
    return e == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

lora_status_t lora_sgmv_expand(const lora_dims_t* dims, int32_t family, const float* u,
                               const void* B_stack, const int32_t* lora_ids,
                               const int32_t* grouped_offsets, int32_t num_groups, int64_t end,
                               void* y, int64_t ldy, int32_t path, void* stream)
{
    FamilyShape fs;
    lora_status_t st = family_shape(dims, family, &fs);
    if (st != LORA_OK)
        return st;
    if (path < LORA_PATH_AUTO || path > LORA_PATH_MFMA)
        return LORA_ERR_INVALID_ARGUMENT;
    const bool bf16 = dims->dtype == LORA_DTYPE_BF16;
    bool widths16 = true;
    for (int s = 0; s < fs.n_s; ++s)
        widths16 = widths16 && fs.widths[s] % 16 == 0;
    const bool mfma_ok = bf16 && fs.R % 16 == 0 && fs.R <= 64 && widths16;
    if (path == LORA_PATH_MFMA && !mfma_ok)
        return LORA_ERR_INVALID_ARGUMENT;
    if (end < 0 || end > 2147483647LL || num_groups < 0 || num_groups > fs.L)
        return LORA_ERR_INVALID_ARGUMENT;
    if (end == 0 || num_groups == 0)
        return LORA_OK;
    if (!u || !B_stack || !lora_ids || !grouped_offsets || !y)
        return LORA_ERR_INVALID_ARGUMENT;
    if (ldy < fs.out_f || (ldy * fs.elem) % 16 || !aligned16(u) || !aligned16(B_stack) ||
        !aligned16(y))
        return LORA_ERR_INVALID_ARGUMENT;
    ExpandArgs a;
    a.u = u;
    a.B = B_stack;
    a.y = y;
    a.ldy = ldy;
    a.ids = lora_ids;
    a.offs = grouped_offsets;
    a.C = fs.C;
    a.R = fs.R;
    a.L = fs.L;
    a.G = num_groups;
    a.end = (int)end;
    a.n_s = fs.n_s;
    a.out_f = fs.out_f;
    for (int s = 0; s < 5; ++s)
        a.soff[s] = s <= fs.n_s ? fs.offs[s] : fs.out_f;
    a.n_ftiles = (fs.out_f + kExpandCols - 1) / kExpandCols;
    a.valu_max = mfma_ok ? valu_max_for(path, bf16, env_int("LORA_SGMV_VALU_MAX_EXPAND", 8)) : kTileM;
    const int64_t tiles = (end + kTileM - 1) / kTileM + num_groups;
    const int64_t grid = tiles * a.n_ftiles;
    if (grid > 2147483647LL)
        return LORA_ERR_INVALID_ARGUMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (bf16)
        hipLaunchKernelGGL((expand_kernel<uint16_t>), dim3((int)grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((expand_kernel<float>), dim3((int)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_DEVICE;
}

}  // extern "C"
