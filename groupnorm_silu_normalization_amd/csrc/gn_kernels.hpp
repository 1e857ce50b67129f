// gn_kernels.hpp -- gfx950 (CDNA4) kernels of the channels-last GroupNorm(+SiLU)
// path: partial statistics (with the finalize fused into its tail), a
// separate finalize for many groups, and the fused apply (+SiLU).
//
// The three steps are the ones of "FLUX.2 VAE decoder fast path behind
// quality=high", Modifications section 1 "Kernel"; the kernels below are a
// fresh design for wave64 CDNA4, not a translation of the Triton kernel the
// pages describe.
//
// Element types: bf16, IEEE fp16 or fp32 in and out (the same type for x and
// y); all arithmetic is fp32, and y is rounded once to its type (round to
// nearest even).
//
// Data layout: one sample is E = L*C values, channel fastest.  A "tile" is
// kThreads*VEC consecutive elements of a sample (2048 for VEC = 8).  Lane
// `tid` owns VEC slots of every tile at fixed offsets o(tid, j) (Pack::
// slot_offset): 8*tid + j for 16-bit types, whose 8 values are one 16-byte
// access; 4*tid + j and 1024 + 4*tid + (j - 4) for fp32, two 16-byte
// accesses, so that each wave instruction still covers 1 KiB of contiguous
// memory.  C is a power of two <= 2048, so every tile starts on a row
// boundary and slot j always holds channel o(tid, j) mod C: the lane's
// channel parameters and partial sums stay in registers for the whole chunk.
//
// Numerics: each thread accumulates x - p_g, where the pivot p_g is the first
// element of its group in row 0 of the sample (x[n, 0, g*Cg]).  Shifting by a
// value of the group keeps the fp32 sum of squares from cancelling when a
// group's mean is large against its spread; in exact arithmetic the result is
// unchanged (mean = p + S/M, var = Q/M - (S/M)^2).  Every reduction runs in an
// order fixed by (N, L, C, G) alone, so results are bitwise reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gnsilu {

constexpr int kThreads = 256;  // 4 waves of 64

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---- element types ---------------------------------------------------------
// storage: the in-memory type; to_f32 widens exactly; pack2 rounds two fp32
// values to the type (round to nearest even: v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32 on gfx950) and packs them, lower address first.
struct Bf16 {
    using storage = uint16_t;
    __device__ __forceinline__ static float to_f32(uint16_t b) {
        return __uint_as_float(static_cast<uint32_t>(b) << 16);
    }
    __device__ __forceinline__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ __forceinline__ static float hi(uint32_t w) {
        return __uint_as_float(w & 0xffff0000u);
    }
    __device__ __forceinline__ static uint32_t pack2(float a, float b) {
        f32x2 v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    }
    __device__ __forceinline__ static uint16_t from_f32(float f) {
        return static_cast<uint16_t>(pack2(f, 0.0f) & 0xffffu);
    }
};

struct Fp16 {
    using storage = uint16_t;
    __device__ __forceinline__ static float to_f32(uint16_t b) {
        return static_cast<float>(__builtin_bit_cast(_Float16, b));
    }
    __device__ __forceinline__ static float lo(uint32_t w) {
        return to_f32(static_cast<uint16_t>(w & 0xffffu));
    }
    __device__ __forceinline__ static float hi(uint32_t w) {
        return to_f32(static_cast<uint16_t>(w >> 16));
    }
    __device__ __forceinline__ static uint32_t pack2(float a, float b) {
        f32x2 v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
    __device__ __forceinline__ static uint16_t from_f32(float f) {
        return static_cast<uint16_t>(pack2(f, 0.0f) & 0xffffu);
    }
};

struct F32 {
    using storage = float;
    __device__ __forceinline__ static float to_f32(float v) { return v; }
    __device__ __forceinline__ static float from_f32(float f) { return f; }
};

// SiLU(t) = t * sigmoid(t) = t / (1 + e^-t), with e^-t = 2^(-t*log2 e):
// one v_exp_f32 and one v_rcp_f32.  t << 0 gives 2^(+big) = inf, 1/inf = 0,
// t*0 = -0, the limit; t >> 0 gives t.
__device__ __forceinline__ float silu_f32(float t) {
    const float e = __builtin_amdgcn_exp2f(t * -1.4426950408889634f);
    return t * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---- a lane's VEC consecutive values ----------------------------------------
// NT: the access carries the nontemporal hint (streaming cache policy), for
// data the pass touches once.
template <bool NT, class T>
__device__ __forceinline__ T ld(const T *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}
template <bool NT, class T>
__device__ __forceinline__ void st(T *p, T v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

template <class D, int VEC> struct Pack;

// Each Pack is loaded from / stored to a tile (its first element) by lane
// `tid`; slot_offset(tid, j) is the element of the tile held in slot j.

// 16-bit types: 8 values in one 16-byte access.
template <class D> struct Pack16 {
    u32x4 w;
    __device__ __forceinline__ static int slot_offset(int tid, int j) { return tid * 8 + j; }
    __device__ __forceinline__ float get(int j) const {
        const uint32_t word = w[j >> 1];
        return (j & 1) ? D::hi(word) : D::lo(word);
    }
    template <bool NT = false>
    __device__ __forceinline__ static void store(uint16_t *tile, int tid, const float (&o)[8]) {
        u32x4 v;
        v[0] = D::pack2(o[0], o[1]);
        v[1] = D::pack2(o[2], o[3]);
        v[2] = D::pack2(o[4], o[5]);
        v[3] = D::pack2(o[6], o[7]);
        st<NT>(reinterpret_cast<u32x4 *>(tile + tid * 8), v);
    }
};
template <> struct Pack<Bf16, 8> : Pack16<Bf16> {
    template <bool NT = false>
    __device__ __forceinline__ static Pack load(const uint16_t *tile, int tid) {
        Pack v;
        v.w = ld<NT>(reinterpret_cast<const u32x4 *>(tile + tid * 8));
        return v;
    }
};
template <> struct Pack<Fp16, 8> : Pack16<Fp16> {
    template <bool NT = false>
    __device__ __forceinline__ static Pack load(const uint16_t *tile, int tid) {
        Pack v;
        v.w = ld<NT>(reinterpret_cast<const u32x4 *>(tile + tid * 8));
        return v;
    }
};

// fp32: slots 0-3 are elements 4*tid .. 4*tid+3 of the tile, slots 4-7 the
// same four one half-tile (kThreads*4 elements) further on.
template <> struct Pack<F32, 8> {
    static constexpr int kHalf = kThreads * 4;
    u32x4 a, b;
    __device__ __forceinline__ static int slot_offset(int tid, int j) {
        return (j < 4 ? 0 : kHalf - 4) + tid * 4 + j;
    }
    template <bool NT = false>
    __device__ __forceinline__ static Pack load(const float *tile, int tid) {
        Pack v;
        v.a = ld<NT>(reinterpret_cast<const u32x4 *>(tile + tid * 4));
        v.b = ld<NT>(reinterpret_cast<const u32x4 *>(tile + kHalf + tid * 4));
        return v;
    }
    __device__ __forceinline__ float get(int j) const {
        return __uint_as_float(j < 4 ? a[j] : b[j - 4]);
    }
    template <bool NT = false>
    __device__ __forceinline__ static void store(float *tile, int tid, const float (&o)[8]) {
        u32x4 va, vb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            va[j] = __float_as_uint(o[j]);
            vb[j] = __float_as_uint(o[j + 4]);
        }
        st<NT>(reinterpret_cast<u32x4 *>(tile + tid * 4), va);
        st<NT>(reinterpret_cast<u32x4 *>(tile + kHalf + tid * 4), vb);
    }
};

// One value per lane (C < 8 with L*C not a multiple of 8).
template <class D> struct Pack<D, 1> {
    typename D::storage b;
    __device__ __forceinline__ static int slot_offset(int tid, int) { return tid; }
    template <bool NT = false>
    __device__ __forceinline__ static Pack load(const typename D::storage *tile, int tid) {
        Pack v;
        v.b = ld<NT>(tile + tid);
        return v;
    }
    __device__ __forceinline__ float get(int) const { return D::to_f32(b); }
    template <bool NT = false>
    __device__ __forceinline__ static void store(typename D::storage *tile, int tid,
                                                 const float (&o)[1]) {
        st<NT>(tile + tid, D::from_f32(o[0]));
    }
};

// Arguments shared by the kernels; the host fills it from the plan.
struct Geometry {
    int64_t E;         // elements per sample, L*C
    int64_t tiles;     // tiles per sample, ceil(E / tile)
    int64_t full;      // tiles per sample lying entirely inside the sample
    int64_t tpc;       // tiles per chunk (one workgroup's share)
    int64_t K;         // chunks per sample
    int C;             // channels (power of two)
    int cg_shift;      // log2(C / G)
    int G;             // groups
};

// Where the statistics go.
struct StatsOut {
    float *part_s;        // [N][K][G] pivot-shifted sum of each group over chunk k
    float *part_q;        // [N][K][G] pivot-shifted sum of squares
    unsigned *arrivals;   // [N] statistics workgroups of sample n finished (fused
                          // finalize only); zero between calls
    float *mean;          // [N][G]
    float *rstd;          // [N][G]
    double inv_m;         // 1 / (L*Cg)
    float eps;
};

// mean = p + S/M, var = max(Q/M - (S/M)^2, 0), rstd = 1/sqrt(var + eps); the
// few scalar operations in fp64, results stored as fp32.
__device__ __forceinline__ void group_moments(float S, float Q, float pivot, double inv_m,
                                              float eps, float *mean, float *rstd) {
    const double ms = static_cast<double>(S) * inv_m;
    double var = static_cast<double>(Q) * inv_m - ms * ms;
    if (var < 0.0) var = 0.0;
    *mean = static_cast<float>(static_cast<double>(pivot) + ms);
    *rstd = static_cast<float>(1.0 / sqrt(var + static_cast<double>(eps)));
}

// A partial written by step 1.  When the finalize is fused, the partials are
// agent-scope atomic stores: write-through (sc1), so they are visible to a
// workgroup on any XCD once the store has completed, without writing back the
// whole L2 as an agent-scope release fence would.
template <bool COHERENT>
__device__ __forceinline__ void store_partial(float *p, float v) {
    if constexpr (COHERENT)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

// ---------------------------------------------------------------------------
// Pieces of steps 1-3, kept as functions so the order of every
// floating-point operation is written down once.
// ---------------------------------------------------------------------------

// Pivots p_g of the lane's VEC channel slots; zeroed running sums.
template <class D, int VEC>
__device__ __forceinline__ void init_slots(const typename D::storage *xs, const Geometry &geo,
                                           int tid, float (&piv)[VEC], float (&s)[VEC],
                                           float (&q)[VEC]) {
    const int cmask = geo.C - 1;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        const int c = Pack<D, VEC>::slot_offset(tid, j) & cmask;
        piv[j] = D::to_f32(xs[(c >> geo.cg_shift) << geo.cg_shift]);
        s[j] = 0.0f;
        q[j] = 0.0f;
    }
}

template <class D, int VEC>
__device__ __forceinline__ void accumulate(const Pack<D, VEC> &v, const float (&piv)[VEC],
                                           float (&s)[VEC], float (&q)[VEC]) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        const float d = v.get(j) - piv[j];
        s[j] += d;
        q[j] = fmaf(d, d, q[j]);
    }
}

__device__ __forceinline__ void accumulate1(float v, float piv, float &s, float &q) {
    const float d = v - piv;
    s += d;
    q = fmaf(d, d, q);
}

// Tiles [t_begin, t_end) of a chunk; the first t_full_end - t_begin of them
// lie wholly inside the sample, the one after that (if any) is the sample's
// partial last tile.
struct ChunkRange {
    int64_t t_begin, t_end, t_full_end;
};
__device__ __forceinline__ ChunkRange chunk_range(const Geometry &geo, int64_t k) {
    ChunkRange r;
    r.t_begin = k * geo.tpc;
    r.t_end = r.t_begin + geo.tpc < geo.tiles ? r.t_begin + geo.tpc : geo.tiles;
    r.t_full_end = r.t_end < geo.full ? r.t_end : geo.full;
    if (r.t_full_end < r.t_begin) r.t_full_end = r.t_begin;
    return r;
}

// Workgroup reduction of the lanes' slot sums to per-group partials of chunk
// k, written to out.part_s / out.part_q at [(n*K + k)*G + g].  Slot j of
// lane tid goes to red_*[i], i = slot_offset(tid, j), which holds channel
// i mod C; the P = TILE/G entries of group g are i = r*C + g*Cg + u.
template <class D, int VEC, bool COHERENT>
__device__ __forceinline__ void write_group_partials(const float (&s)[VEC], const float (&q)[VEC],
                                                     float *red_s, float *red_q,
                                                     const Geometry &geo, int64_t n, int64_t k,
                                                     const StatsOut &out, int tid) {
    constexpr int TILE = kThreads * VEC;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        const int i = Pack<D, VEC>::slot_offset(tid, j);
        red_s[i] = s[j];
        red_q[i] = q[j];
    }
    __syncthreads();
    const int G = geo.G;
    const int cgm = (1 << geo.cg_shift) - 1;
    if (G <= kThreads) {
        const int tg = kThreads / G;  // threads per group
        const int g = tid / tg;
        const int part = tid - g * tg;
        float as = 0.0f, aq = 0.0f;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const int e = part * VEC + j;
            const int i = (e >> geo.cg_shift) * geo.C + (g << geo.cg_shift) + (e & cgm);
            as += red_s[i];
            aq += red_q[i];
        }
        __syncthreads();
        red_s[tid] = as;
        red_q[tid] = aq;
        __syncthreads();
        for (int stride = tg >> 1; stride > 0; stride >>= 1) {
            if (part < stride) {
                red_s[tid] += red_s[tid + stride];
                red_q[tid] += red_q[tid + stride];
            }
            __syncthreads();
        }
        if (part == 0) {
            const int64_t o = (n * geo.K + k) * G + g;
            store_partial<COHERENT>(out.part_s + o, red_s[tid]);
            store_partial<COHERENT>(out.part_q + o, red_q[tid]);
        }
    } else {
        const int P = TILE / G;  // < VEC slots per group
        for (int g = tid; g < G; g += kThreads) {
            float as = 0.0f, aq = 0.0f;
            for (int e = 0; e < P; ++e) {
                const int i = (e >> geo.cg_shift) * geo.C + (g << geo.cg_shift) + (e & cgm);
                as += red_s[i];
                aq += red_q[i];
            }
            const int64_t o = (n * geo.K + k) * G + g;
            store_partial<COHERENT>(out.part_s + o, as);
            store_partial<COHERENT>(out.part_q + o, aq);
        }
    }
}

// Counts this workgroup's arrival for sample n once its (write-through)
// partial stores have completed; true, uniformly, in the last of the K.
__device__ __forceinline__ bool arrive_is_last(const StatsOut &out, int64_t n, int64_t K,
                                               int tid) {
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(0);  // this lane's stores have completed ...
    __syncthreads();                // ... in every lane, before the arrival is counted
    if (tid == 0) {
        const unsigned before =
            __hip_atomic_fetch_add(out.arrivals + n, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = (before == static_cast<unsigned>(K - 1));
    }
    __syncthreads();
    return last != 0;
}

// Step 2 for sample n, run by the last workgroup to arrive (G <= kThreads):
// thread tid = g + G*j sums the chunks k = j, j + tpg, ... in increasing
// order (coalesced along g; loads issued kBatch at a time so their round
// trips overlap -- one round trip for K <= 16*tpg), a fixed tree over j
// follows, and mean/rstd are written.  The arrival counter is reset to zero
// for the next call.
template <class D>
__device__ __forceinline__ void finalize_sample(const typename D::storage *xs,
                                                const Geometry &geo, int64_t n,
                                                const StatsOut &out, float *red_s, float *red_q,
                                                int tid) {
    const int G = geo.G;
    const int tpg = kThreads / G;
    const int g = tid & (G - 1);
    const int j = tid / G;
    constexpr int kBatch = 16;
    const float *ps = out.part_s + n * geo.K * G + g;
    const float *pq = out.part_q + n * geo.K * G + g;
    float as = 0.0f, aq = 0.0f;
    int64_t kk = j;
    for (; kk + (kBatch - 1) * tpg < geo.K; kk += kBatch * tpg) {
        float vs[kBatch], vq[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int64_t o = (kk + b * tpg) * G;
            vs[b] = __hip_atomic_load(ps + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            vq[b] = __hip_atomic_load(pq + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            as += vs[b];
            aq += vq[b];
        }
    }
    for (; kk < geo.K; kk += tpg) {
        as += __hip_atomic_load(ps + kk * G, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        aq += __hip_atomic_load(pq + kk * G, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    red_s[tid] = as;
    red_q[tid] = aq;
    __syncthreads();
    for (int stride = tpg >> 1; stride > 0; stride >>= 1) {
        if (j < stride) {
            red_s[tid] += red_s[tid + stride * G];
            red_q[tid] += red_q[tid + stride * G];
        }
        __syncthreads();
    }
    if (j == 0) {
        const float pivot = D::to_f32(xs[static_cast<int64_t>(g) << geo.cg_shift]);
        group_moments(red_s[tid], red_q[tid], pivot, out.inv_m, out.eps, out.mean + n * G + g,
                      out.rstd + n * G + g);
    }
    if (tid == 0)
        __hip_atomic_store(out.arrivals + n, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// scale = gamma*rstd, shift = beta - mean*scale for the lane's VEC channels.
template <class D, int VEC>
__device__ __forceinline__ void fold_affine(const float *mean, const float *rstd,
                                            const float *gamma, const float *beta,
                                            const Geometry &geo, int64_t n, int tid,
                                            float (&sc)[VEC], float (&sh)[VEC]) {
    const int cmask = geo.C - 1;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        const int c = Pack<D, VEC>::slot_offset(tid, j) & cmask;
        const int64_t gi = n * geo.G + (c >> geo.cg_shift);
        const float ga = gamma ? gamma[c] : 1.0f;
        const float be = beta ? beta[c] : 0.0f;
        sc[j] = ga * rstd[gi];
        sh[j] = fmaf(-mean[gi], sc[j], be);
    }
}

template <bool SILU>
__device__ __forceinline__ float transform1(float x, float sc, float sh) {
    const float t = fmaf(x, sc, sh);
    if constexpr (SILU) {
        return silu_f32(t);
    } else {
        return t;
    }
}

template <class D, int VEC, bool SILU>
__device__ __forceinline__ void transform(const Pack<D, VEC> &v, const float (&sc)[VEC],
                                          const float (&sh)[VEC], float (&o)[VEC]) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) o[j] = transform1<SILU>(v.get(j), sc[j], sh[j]);
}

// ---------------------------------------------------------------------------
// Step 1: partial statistics.  One workgroup per (sample n, chunk k); writes
// the pivot-shifted sum and sum of squares of each group over its chunk to
// part_s / part_q at [(n*K + k)*G + g].
// FUSED (requires G <= kThreads): the last workgroup of sample n to finish,
// found with an agent-scope atomic counter, also performs step 2 for that
// sample -- a fixed-order reduction over the K chunk partials of each group,
// whichever workgroup happens to be last -- and resets the counter to zero.
// Ordering: every lane waits for its write-through partial stores to
// complete (s_waitcnt vmcnt(0)), the workgroup barrier follows, and only then
// is the arrival counted; the last workgroup reads the partials with
// agent-scope (coherent) loads.
// ---------------------------------------------------------------------------
template <class D, int VEC, int UNROLL, bool NTL, bool FUSED>
__global__ __launch_bounds__(kThreads) void gn_partial_stats(
    const typename D::storage *__restrict__ x, Geometry geo, StatsOut out) {
    constexpr int TILE = kThreads * VEC;
    __shared__ float red_s[TILE];
    __shared__ float red_q[TILE];

    const int tid = threadIdx.x;
    const int64_t wg = blockIdx.x;
    const int64_t n = wg / geo.K;
    const int64_t k = wg - n * geo.K;
    const typename D::storage *xs = x + n * geo.E;

    float piv[VEC], s[VEC], q[VEC];
    init_slots<D, VEC>(xs, geo, tid, piv, s, q);

    const ChunkRange cr = chunk_range(geo, k);
    const typename D::storage *p = xs + cr.t_begin * TILE;  // current tile
    int64_t tt = cr.t_begin;
    for (; tt + UNROLL <= cr.t_full_end; tt += UNROLL) {
        Pack<D, VEC> v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            v[u] = Pack<D, VEC>::template load<NTL>(p + u * TILE, tid);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) accumulate<D, VEC>(v[u], piv, s, q);
        p += UNROLL * TILE;
    }
    for (; tt < cr.t_full_end; ++tt) {
        accumulate<D, VEC>(Pack<D, VEC>::template load<NTL>(p, tid), piv, s, q);
        p += TILE;
    }
    if (tt < cr.t_end) {
        // The sample's last tile is partial: slot by slot, in bounds only.
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const int64_t off = tt * TILE + Pack<D, VEC>::slot_offset(tid, j);
            if (off < geo.E) accumulate1(D::to_f32(xs[off]), piv[j], s[j], q[j]);
        }
    }

    write_group_partials<D, VEC, FUSED>(s, q, red_s, red_q, geo, n, k, out, tid);
    if constexpr (FUSED) {
        if (arrive_is_last(out, n, geo.K, tid))
            finalize_sample<D>(xs, geo, n, out, red_s, red_q, tid);
    }
}

// ---------------------------------------------------------------------------
// Step 2 as its own kernel, used when G > kThreads (too many groups for one
// workgroup to finish quickly): one workgroup per (n, g), a fixed-order tree
// over the K chunk partials.
// ---------------------------------------------------------------------------
template <class D>
__global__ __launch_bounds__(kThreads) void gn_finalize_stats(
    const typename D::storage *__restrict__ x, Geometry geo, StatsOut out) {
    __shared__ float rs[kThreads];
    __shared__ float rq[kThreads];
    const int tid = threadIdx.x;
    const int64_t ng = blockIdx.x;
    const int64_t n = ng / geo.G;
    const int g = static_cast<int>(ng - n * geo.G);
    float s = 0.0f, q = 0.0f;
    for (int64_t k = tid; k < geo.K; k += kThreads) {
        const int64_t o = (n * geo.K + k) * geo.G + g;
        s += out.part_s[o];
        q += out.part_q[o];
    }
    rs[tid] = s;
    rq[tid] = q;
    __syncthreads();
    for (int stride = kThreads / 2; stride > 0; stride >>= 1) {
        if (tid < stride) {
            rs[tid] += rs[tid + stride];
            rq[tid] += rq[tid + stride];
        }
        __syncthreads();
    }
    if (tid == 0) {
        const float pivot = D::to_f32(x[n * geo.E + (static_cast<int64_t>(g) << geo.cg_shift)]);
        group_moments(rs[0], rq[0], pivot, out.inv_m, out.eps, out.mean + ng, out.rstd + ng);
    }
}

// Zero-fill for the arrival counters of a fresh scratch buffer (a kernel, so
// the clearing is ordinary stream work).
__global__ __launch_bounds__(kThreads) void gn_zero_u32(unsigned *p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Step 3: fused apply.  One workgroup per (n, chunk); each lane folds
// gamma/beta and the group statistics of its VEC channels into scale/shift
// registers once (scale = gamma*rstd, shift = beta - mean*scale), then
// streams its chunk: y = SiLU(x*scale + shift), rounded once to D.
// x and y may be the same buffer (each element is read, then written, by one
// lane), so they carry no __restrict__.
// ---------------------------------------------------------------------------
template <class D, int VEC, int UNROLL, bool SILU, bool NTL, bool NTS>
__global__ __launch_bounds__(kThreads) void gn_apply(
    const typename D::storage *x, typename D::storage *y, Geometry geo, int reverse,
    const float *__restrict__ mean, const float *__restrict__ rstd,
    const float *__restrict__ gamma, const float *__restrict__ beta) {
    constexpr int TILE = kThreads * VEC;
    const int tid = threadIdx.x;
    const int64_t wg = reverse ? static_cast<int64_t>(gridDim.x) - 1 - blockIdx.x
                               : static_cast<int64_t>(blockIdx.x);
    const int64_t n = wg / geo.K;
    const int64_t k = wg - n * geo.K;

    float sc[VEC], sh[VEC];
    fold_affine<D, VEC>(mean, rstd, gamma, beta, geo, n, tid, sc, sh);

    const int64_t base = n * geo.E;
    const ChunkRange cr = chunk_range(geo, k);
    int64_t off = base + cr.t_begin * TILE;  // current tile
    int64_t tt = cr.t_begin;
    for (; tt + UNROLL <= cr.t_full_end; tt += UNROLL) {
        Pack<D, VEC> v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            v[u] = Pack<D, VEC>::template load<NTL>(x + off + u * TILE, tid);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float o[VEC];
            transform<D, VEC, SILU>(v[u], sc, sh, o);
            Pack<D, VEC>::template store<NTS>(y + off + u * TILE, tid, o);
        }
        off += UNROLL * TILE;
    }
    for (; tt < cr.t_full_end; ++tt) {
        float o[VEC];
        transform<D, VEC, SILU>(Pack<D, VEC>::template load<NTL>(x + off, tid), sc, sh, o);
        Pack<D, VEC>::template store<NTS>(y + off, tid, o);
        off += TILE;
    }
    if (tt < cr.t_end) {
        // The sample's last tile is partial: slot by slot, in bounds only.
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const int64_t rel = tt * TILE + Pack<D, VEC>::slot_offset(tid, j);
            if (rel < geo.E)
                y[base + rel] = D::from_f32(transform1<SILU>(D::to_f32(x[base + rel]), sc[j], sh[j]));
        }
    }
}

}  // namespace gnsilu
