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
// R whole rows, T = R*C elements, worked by the first A lanes of a 256-lane
// workgroup; lane `tid` owns S = W*NV slots of every tile, NV accesses of W
// consecutive elements (W = 8 for 16-bit types and W = 4 for fp32: one
// 16-byte access; W = 1 when rows are not 16-byte multiples).  Access a of
// lane tid covers elements (a*A + tid)*W .. +W-1, so each wave instruction
// covers contiguous memory, and slot j sits at the fixed offset
// o(tid, j) = ((j / W)*A + tid)*W + j % W.  Because a tile starts on a row
// boundary, slot j always holds channel o(tid, j) mod C: the lane's channel
// parameters and partial sums stay in registers for the whole chunk.  The
// host picks (W, NV, R) with A*S = T; for power-of-two C <= 2048 in 16-bit
// types that is W = 8, NV = 1, T = 2048, A = 256.
//
// Numerics: each thread accumulates x - p_g, where the pivot p_g is the first
// element of its group in row 0 of the sample (x[n, 0, g*Cg]).  Shifting by a
// value of the group keeps the fp32 sum of squares from cancelling when a
// group's mean is large against its spread; in exact arithmetic the result is
// unchanged (mean = p + S/M, var = Q/M - (S/M)^2).  Every reduction runs in an
// order fixed by (N, L, C, G) and the element type alone, so results are
// bitwise reproducible.
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

// ---- one access of W consecutive elements -----------------------------------
template <class D, int W> struct Vec;

template <class D> struct Vec16x8 {  // 8 16-bit values, one 16-byte access
    u32x4 w;
    __device__ __forceinline__ float get(int j) const {
        const uint32_t word = w[j >> 1];
        return (j & 1) ? D::hi(word) : D::lo(word);
    }
    template <bool NT>
    __device__ __forceinline__ void load(const uint16_t *p) {
        w = ld<NT>(reinterpret_cast<const u32x4 *>(p));
    }
    template <bool NT>
    __device__ __forceinline__ static void store(uint16_t *p, const float *o) {
        u32x4 v;
        v[0] = D::pack2(o[0], o[1]);
        v[1] = D::pack2(o[2], o[3]);
        v[2] = D::pack2(o[4], o[5]);
        v[3] = D::pack2(o[6], o[7]);
        st<NT>(reinterpret_cast<u32x4 *>(p), v);
    }
};
template <> struct Vec<Bf16, 8> : Vec16x8<Bf16> {};
template <> struct Vec<Fp16, 8> : Vec16x8<Fp16> {};

template <> struct Vec<F32, 4> {  // 4 fp32 values, one 16-byte access
    u32x4 w;
    __device__ __forceinline__ float get(int j) const { return __uint_as_float(w[j]); }
    template <bool NT>
    __device__ __forceinline__ void load(const float *p) {
        w = ld<NT>(reinterpret_cast<const u32x4 *>(p));
    }
    template <bool NT>
    __device__ __forceinline__ static void store(float *p, const float *o) {
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __float_as_uint(o[j]);
        st<NT>(reinterpret_cast<u32x4 *>(p), v);
    }
};

template <class D> struct Vec<D, 1> {  // one value
    typename D::storage b;
    __device__ __forceinline__ float get(int) const { return D::to_f32(b); }
    template <bool NT>
    __device__ __forceinline__ void load(const typename D::storage *p) { b = ld<NT>(p); }
    template <bool NT>
    __device__ __forceinline__ static void store(typename D::storage *p, const float *o) {
        st<NT>(p, D::from_f32(o[0]));
    }
};

// ---- a lane's S = W*NV slots of one tile -------------------------------------
template <class D, int W, int NV> struct Lane {
    static constexpr int kSlots = W * NV;
    static constexpr int kW = W;
    static constexpr int kNV = NV;
    using T = typename D::storage;
    Vec<D, W> v[NV];
    __device__ __forceinline__ static int slot_offset(int A, int tid, int j) {
        return ((j / W) * A + tid) * W + j % W;
    }
    template <bool NT>
    __device__ __forceinline__ static Lane load(const T *tile, int A, int tid) {
        Lane l;
#pragma unroll
        for (int a = 0; a < NV; ++a) l.v[a].template load<NT>(tile + (a * A + tid) * W);
        return l;
    }
    __device__ __forceinline__ float get(int j) const { return v[j / W].get(j % W); }
    template <bool NT>
    __device__ __forceinline__ static void store(T *tile, int A, int tid, const float (&o)[kSlots]) {
#pragma unroll
        for (int a = 0; a < NV; ++a) Vec<D, W>::template store<NT>(tile + (a * A + tid) * W, o + a * W);
    }
};

// Arguments shared by the kernels; the host fills it from the plan.
struct Geometry {
    int64_t E;      // elements per sample, L*C
    int64_t T;      // elements per tile: R whole rows, a multiple of C (T = A*S)
    int64_t tiles;  // tiles per sample, ceil(E / T)
    int64_t full;   // tiles per sample lying entirely inside the sample
    int64_t tpc;    // tiles per chunk (one workgroup's share) ...
    int64_t rem;    // ... plus one for the first `rem` chunks of a sample (step 3;
                    // step 1's chunks are tpc tiles, the last one cut at the end)
    int64_t K;      // chunks per sample
    int C;          // channels
    int G;          // groups
    int Cg;         // channels per group, C / G
    int A;          // active lanes per tile (<= kThreads)
    int cg_shift;   // log2(Cg) when C is a power of two, else 0
    int64_t plain_tail;  // step 1: the last plain_tail tiles of each chunk use plain
                         // loads, the tiles before them nontemporal ones
};

// The tile geometry as one kernel sees it.  All 256 lanes are busy exactly
// when C is a power of two (A is the largest multiple of C / gcd(C, W*NV)
// not above 256, and W*NV is a power of two).  POW2 kernels are compiled for
// that case: the tile is the compile-time 256*S elements, and channel and
// group indices are masks and shifts; the general kernels take T and A from
// the plan and divide.
template <bool POW2, int S> struct TileGeo {
    int64_t T_;
    int A_, C, Cg, cg_shift;
    __device__ __forceinline__ explicit TileGeo(const Geometry &g)
        : T_(g.T), A_(g.A), C(g.C), Cg(g.Cg), cg_shift(g.cg_shift) {}
    __device__ __forceinline__ int64_t tile() const {
        if constexpr (POW2)
            return int64_t{kThreads} * S;
        else
            return T_;
    }
    __device__ __forceinline__ int lanes() const {
        if constexpr (POW2)
            return kThreads;
        else
            return A_;
    }
    __device__ __forceinline__ int channel(int o) const {  // o mod C
        if constexpr (POW2)
            return o & (C - 1);
        else
            return o % C;
    }
    __device__ __forceinline__ int group_of(int c) const {  // c / Cg
        if constexpr (POW2)
            return c >> cg_shift;
        else
            return c / Cg;
    }
};

// Where the statistics go.
struct StatsOut {
    float *part_s;        // [N][K][G] pivot-shifted sum of each group over chunk k
    float *part_q;        // [N][K][G] pivot-shifted sum of squares
    unsigned *arrivals;   // [N][arrival_stride(K)] arrival counters of sample n
                          // (fused finalize only); zero between calls
    float *mean;          // [N][G]
    float *rstd;          // [N][G]
    float *pivot;         // [N][G] or null: the group pivots x[n, 0, g*Cg], saved by
                          // chunk 0 of each sample for the late finalize (which must
                          // not read x: with y == x step 3 overwrites row 0)
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

// Fixed-order tree over the `count` entries red[base + i*step], i < count,
// whatever count is: strides halve from the power of two below count, entry
// i adds entry i + stride when that exists; entry 0 ends up holding the sum.
// Every thread of the workgroup calls it (it contains barriers, and count is
// uniform); `idx` is the calling thread's i, or -1 for a thread that holds no
// entry.
__device__ __forceinline__ void tree_sum(float *red_s, float *red_q, int base, int step, int idx,
                                         int count) {
    int p2 = 1;
    while (p2 < count) p2 <<= 1;
    for (int stride = p2 >> 1; stride > 0; stride >>= 1) {
        if (idx >= 0 && idx < stride && idx + stride < count) {
            red_s[base + idx * step] += red_s[base + (idx + stride) * step];
            red_q[base + idx * step] += red_q[base + (idx + stride) * step];
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Pieces of steps 1-3, kept as functions so the order of every
// floating-point operation is written down once.
// ---------------------------------------------------------------------------

template <class L>
__device__ __forceinline__ void accumulate(const L &v, const float (&piv)[L::kSlots],
                                           float (&s)[L::kSlots], float (&q)[L::kSlots]) {
#pragma unroll
    for (int j = 0; j < L::kSlots; ++j) {
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
// Step 3's chunks: the sample's tiles split evenly, the first geo.rem chunks
// one tile longer.
__device__ __forceinline__ ChunkRange chunk_range_even(const Geometry &geo, int64_t k) {
    ChunkRange r;
    r.t_begin = k * geo.tpc + (k < geo.rem ? k : geo.rem);
    const int64_t end = r.t_begin + geo.tpc + (k < geo.rem ? 1 : 0);
    r.t_end = end < geo.tiles ? end : geo.tiles;
    r.t_full_end = r.t_end < geo.full ? r.t_end : geo.full;
    if (r.t_full_end < r.t_begin) r.t_full_end = r.t_begin;
    return r;
}

// Workgroup reduction of the lanes' slot sums to per-group partials of chunk
// k, written to out.part_s / out.part_q at [(n*K + k)*G + g].  Slot j of
// active lane tid goes to red_*[i], i = o(tid, j), which holds channel
// i mod C; the P = R*Cg entries of group g are i = r*C + g*Cg + u.
// G <= kThreads: tg = kThreads / G threads per group, thread (g, part) sums
// the entries e = part, part + tg, ... of its group, then a fixed tree over
// the parts.  G > kThreads: each thread sums whole groups.
// The same reduction for the power-of-two 16-byte layouts of 16-bit types
// (256 lanes, lane tid holding the 8 consecutive channels
// c0 = 8 * (tid mod C/8) ... c0 + 7 of row tid / (C/8) of the tile) whose
// groups are at least 8 channels wide (Cg >= 8, so a lane's slots lie in one
// group), G <= kThreads, without the LDS passes: each lane adds its 8 slots
// (j in increasing order); an xor butterfly over the lane bits that keep the
// group (the bits below Cg/8: the lanes of one row sharing the group; the
// bits from C/8 up: the rows of the wave) leaves every lane of a group with
// the same sum; one lane per (wave, group) writes it to LDS, and thread g
// adds the entries of the waves that hold channels of group g in wave order.
// A fixed order, so the partials are reproducible; every mode of the path
// (fused tail, late finalize, separate finalize, steps 1-2 alone) reads the
// same partials.  Measured on MI355X against the LDS reduction below, in one
// process: 4% less at (1,512,128,128), 1.5% at 64 MiB, 5.5% at
// (2,4096,256).
template <bool COHERENT>
__device__ __forceinline__ void write_group_partials_wave(const float (&s)[8], const float (&q)[8],
                                                          float *red_s, float *red_q,
                                                          const Geometry &geo, int64_t n,
                                                          int64_t k, const StatsOut &out,
                                                          int tid) {
    const int G = geo.G, Cg = geo.Cg;
    const int cb = geo.C >> 3;       // lanes per row of the tile (channel blocks)
    const int gb = Cg >> 3;          // blocks per group
    const int lane = tid & 63, wave = tid >> 6;
    const int blk = tid & (cb - 1);  // the lane's channel block
    float vs = 0.0f, vq = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        vs += s[j];
        vq += q[j];
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        if (m < gb || m >= cb) {  // uniform: the same for every lane
            vs += __shfl_xor(vs, m, 64);
            vq += __shfl_xor(vq, m, 64);
        }
    }
    if ((lane & (gb - 1)) == 0 && (cb >= 64 || lane < cb)) {
        red_s[wave * G + blk / gb] = vs;
        red_q[wave * G + blk / gb] = vq;
    }
    __syncthreads();
    if (tid < G) {
        // channel blocks [b0, b1) of group tid; wave w holds blocks [lo, lo + 64)
        // (all of them when a row is at most 64 blocks)
        const int b0 = tid * gb, b1 = b0 + gb;
        float ts = 0.0f, tq = 0.0f;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) {
            const int lo = cb <= 64 ? 0 : (w * 64) & (cb - 1);
            const int hi = cb <= 64 ? cb : lo + 64;
            if (b0 < hi && b1 > lo) {
                ts += red_s[w * G + tid];
                tq += red_q[w * G + tid];
            }
        }
        const int64_t o = (n * geo.K + k) * G + tid;
        store_partial<COHERENT>(out.part_s + o, ts);
        store_partial<COHERENT>(out.part_q + o, tq);
    }
}

// The same for groups narrower than a lane's 8 channels (Cg = 8 / PER, PER
// groups per lane, Cg consecutive slots each): the lane adds the slots of
// each of its groups, the butterfly runs over the row bits of the wave only,
// and the lanes of the first row of each wave write their PER sums.  PER is
// a template parameter: with Cg known only at run time the per-group sums
// were indexed dynamically, and that version was 3% slower than the LDS
// reduction at (1,128,64,64); this one is 6% faster there (3.5% at Cg = 4
// and 2% at Cg = 2 for 8 MiB shapes).
template <bool COHERENT, int PER>
__device__ __forceinline__ void write_group_partials_wave_narrow(
    const float (&s)[8], const float (&q)[8], float *red_s, float *red_q, const Geometry &geo,
    int64_t n, int64_t k, const StatsOut &out, int tid) {
    constexpr int CG = 8 / PER;
    const int G = geo.G;
    const int cb = geo.C >> 3;
    const int lane = tid & 63, wave = tid >> 6;
    const int blk = tid & (cb - 1);
    float vs[PER], vq[PER];
#pragma unroll
    for (int h = 0; h < PER; ++h) {
        vs[h] = 0.0f;
        vq[h] = 0.0f;
#pragma unroll
        for (int u = 0; u < CG; ++u) {
            vs[h] += s[h * CG + u];
            vq[h] += q[h * CG + u];
        }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        if (m >= cb) {
#pragma unroll
            for (int h = 0; h < PER; ++h) {
                vs[h] += __shfl_xor(vs[h], m, 64);
                vq[h] += __shfl_xor(vq[h], m, 64);
            }
        }
    }
    if (cb >= 64 || lane < cb) {
#pragma unroll
        for (int h = 0; h < PER; ++h) {
            red_s[wave * G + blk * PER + h] = vs[h];
            red_q[wave * G + blk * PER + h] = vq[h];
        }
    }
    __syncthreads();
    if (tid < G) {
        const int b = tid / PER;  // the group's channel block
        float ts = 0.0f, tq = 0.0f;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) {
            const int lo = cb <= 64 ? 0 : (w * 64) & (cb - 1);
            const int hi = cb <= 64 ? cb : lo + 64;
            if (b >= lo && b < hi) {
                ts += red_s[w * G + tid];
                tq += red_q[w * G + tid];
            }
        }
        const int64_t o = (n * geo.K + k) * G + tid;
        store_partial<COHERENT>(out.part_s + o, ts);
        store_partial<COHERENT>(out.part_q + o, tq);
    }
}

template <class L, bool POW2, bool COHERENT, int NT = kThreads>
__device__ __forceinline__ void write_group_partials(const float (&s)[L::kSlots],
                                                     const float (&q)[L::kSlots], float *red_s,
                                                     float *red_q, const Geometry &geo,
                                                     const TileGeo<POW2, L::kSlots> &tg_,
                                                     int64_t n, int64_t k, const StatsOut &out,
                                                     int tid) {
    if constexpr (POW2 && L::kW == 8 && L::kNV == 1 && NT == kThreads) {
        if (geo.Cg >= 8 && geo.G <= kThreads) {
            write_group_partials_wave<COHERENT>(s, q, red_s, red_q, geo, n, k, out, tid);
            return;
        }
        if (geo.G <= kThreads && geo.C >= 8) {
            if (geo.Cg == 4) {
                write_group_partials_wave_narrow<COHERENT, 2>(s, q, red_s, red_q, geo, n, k, out, tid);
                return;
            }
            if (geo.Cg == 2) {
                write_group_partials_wave_narrow<COHERENT, 4>(s, q, red_s, red_q, geo, n, k, out, tid);
                return;
            }
            if (geo.Cg == 1) {
                write_group_partials_wave_narrow<COHERENT, 8>(s, q, red_s, red_q, geo, n, k, out, tid);
                return;
            }
        }
    }
    const int A = tg_.lanes();
    if (tid < A) {
#pragma unroll
        for (int j = 0; j < L::kSlots; ++j) {
            const int i = L::slot_offset(A, tid, j);
            red_s[i] = s[j];
            red_q[i] = q[j];
        }
    }
    __syncthreads();
    const int G = geo.G, C = geo.C, Cg = geo.Cg;
    const int P = static_cast<int>(tg_.tile() / G);  // entries of one group in the tile
    if (G <= kThreads) {
        // tg threads per group; thread (g, part) sums the contiguous entries
        // e in [part*per, (part+1)*per) of its group, a fixed tree over the
        // parts follows.
        const int tg = kThreads / G;
        const int per = (P + tg - 1) / tg;
        const bool has = tid < tg * G;
        const int g = has ? tid / tg : 0;
        const int part = has ? tid - g * tg : 0;
        float as = 0.0f, aq = 0.0f;
        if (has) {
            const int e0 = part * per;
            const int e1 = e0 + per < P ? e0 + per : P;
            int r = tg_.group_of(e0), u = e0 - r * Cg;  // entry e = row r, channel g*Cg + u
            for (int e = e0; e < e1; ++e) {
                const int i = r * C + g * Cg + u;
                as += red_s[i];
                aq += red_q[i];
                if (++u == Cg) {
                    u = 0;
                    ++r;
                }
            }
        }
        __syncthreads();
        red_s[tid] = as;
        red_q[tid] = aq;
        __syncthreads();
        tree_sum(red_s, red_q, g * tg, 1, has ? part : -1, tg);
        if (has && part == 0) {
            const int64_t o = (n * geo.K + k) * G + g;
            store_partial<COHERENT>(out.part_s + o, red_s[tid]);
            store_partial<COHERENT>(out.part_q + o, red_q[tid]);
        }
    } else {
        // Each thread sums whole groups, entries in increasing order.
        for (int g = tid; g < G; g += NT) {
            float as = 0.0f, aq = 0.0f;
            int r = 0, u = 0;
            for (int e = 0; e < P; ++e) {
                const int i = r * C + g * Cg + u;
                as += red_s[i];
                aq += red_q[i];
                if (++u == Cg) {
                    u = 0;
                    ++r;
                }
            }
            const int64_t o = (n * geo.K + k) * G + g;
            store_partial<COHERENT>(out.part_s + o, as);
            store_partial<COHERENT>(out.part_q + o, aq);
        }
    }
}

// Arrival counters of a sample.  With fewer than kArrivalTwoLevelMinK chunks
// a sample has one counter word.  With more, the arrivals of its chunks
// queue at the memory on one word, and a two-level count is faster (measured
// on MI355X: 1-1.6 us less for step 1 at 32-64 MiB, no change from 256 MiB
// up): word 0 counts finished groups of chunks, and word kArrivalLine*(1+s),
// s < kArrivalSubs, the chunks k with k % kArrivalSubs == s, each counter on
// a 128-byte line of its own.  (A sample with that many chunks is large, so
// the wider stride costs little scratch.)
constexpr int kArrivalSubs = 8;
constexpr int kArrivalLine = 32;  // 32-bit words per 128 bytes
constexpr int64_t kArrivalTwoLevelMinK = 64;
__host__ __device__ constexpr int64_t arrival_stride(int64_t K) {
    return K >= kArrivalTwoLevelMinK ? int64_t{kArrivalSubs + 1} * kArrivalLine : 1;
}

// Counts this workgroup's arrival (chunk k of sample n) once its
// (write-through) partial stores have completed; true, uniformly, in the last
// of the K.  In the two-level count the last arrival of a group of chunks
// resets that group's counter and counts the group on word 0.
__device__ __forceinline__ bool arrive_is_last(const StatsOut &out, int64_t n, int64_t K,
                                               int64_t k, int tid) {
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(0);  // this lane's stores have completed ...
    __syncthreads();                // ... in every lane, before the arrival is counted
    if (tid == 0) {
        unsigned *top = out.arrivals + n * arrival_stride(K);
        if (K < kArrivalTwoLevelMinK) {
            const unsigned before =
                __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = (before == static_cast<unsigned>(K - 1));
        } else {
            const int sub = static_cast<int>(k % kArrivalSubs);
            const unsigned in_sub =
                static_cast<unsigned>((K - sub + kArrivalSubs - 1) / kArrivalSubs);
            unsigned *sc = top + (1 + sub) * kArrivalLine;
            const unsigned before =
                __hip_atomic_fetch_add(sc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int is_last = 0;
            if (before == in_sub - 1) {
                __hip_atomic_store(sc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const unsigned groups =
                    __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                is_last = (groups == static_cast<unsigned>(kArrivalSubs - 1));
            }
            last = is_last;
        }
    }
    __syncthreads();
    // The last workgroup reads the other workgroups' partials next: an
    // agent-scope acquire (invalidating what this CU's caches hold that is not
    // coherent at agent scope) so those reads see every partial whose arrival
    // was counted.  Paid once per sample.
    if (last != 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return last != 0;
}

// Partials the fused finalize loads per thread in one batch, and how far past
// the end of a partials array a batch may read; the partial squares are
// followed by that much padding.
constexpr int kFinalizeBatch = 16;
constexpr int64_t kFinalizeOverread = int64_t{kFinalizeBatch - 1} * kThreads;

// One batch of the finalize's partial loads for the thread of (group g, part
// j): chunks kk + b*tpg, b < kFinalizeBatch, issued together so their round
// trips overlap.  A slot past K reads up to (kFinalizeBatch-1)*tpg*G floats
// beyond the sample's partials -- the next sample's, the partial squares
// after the sums, or the kFinalizeOverread floats of padding after the
// squares -- and is not added.  COHERENT: agent-scope loads (the partials
// were written by other workgroups of the same kernel).
// B: slots per batch (kFinalizeBatch, or fewer for the late finalize of a
// sample with few chunks: every load instruction counts in its latency).
template <bool COHERENT, int B = kFinalizeBatch> struct FinalizeBatch {
    static_assert(B >= 1 && B <= kFinalizeBatch, "the over-read bound assumes B <= 16");
    float vs[B], vq[B];
    __device__ __forceinline__ void load(const float *ps, const float *pq, int64_t kk, int tpg,
                                         int G) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int64_t o = (kk + b * tpg) * G;
            if constexpr (COHERENT) {
                vs[b] = __hip_atomic_load(ps + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                vq[b] = __hip_atomic_load(pq + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                vs[b] = ps[o];
                vq[b] = pq[o];
            }
        }
    }
    // Adds the batch's chunks below K, in increasing order.
    __device__ __forceinline__ void add(int64_t kk, int tpg, int64_t K, float &as,
                                       float &aq) const {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (kk + b * tpg < K) {
                as += vs[b];
                aq += vq[b];
            }
        }
    }
};

// The end of step 2 for one sample, every thread of the workgroup taking
// part: thread tid = g + G*j holds its sum (as, aq) over the chunks
// k = j, j + tpg, ...; a fixed tree over j follows and the thread j = 0 of
// each group writes mean/rstd through mean_g/rstd_g (global memory or LDS).
__device__ __forceinline__ void finalize_groups(float as, float aq, bool has, int j, int g,
                                                int G, int tpg, float pivot, double inv_m,
                                                float eps, float *red_s, float *red_q, int tid,
                                                float *mean_g, float *rstd_g) {
    red_s[tid] = as;
    red_q[tid] = aq;
    __syncthreads();
    tree_sum(red_s, red_q, g, G, has ? j : -1, tpg);
    if (has && j == 0) group_moments(red_s[tid], red_q[tid], pivot, inv_m, eps, mean_g, rstd_g);
}

// Step 2 for sample n, run by the last workgroup to arrive (G <= kThreads):
// tpg = kThreads / G threads per group; thread tid = g + G*j (j < tpg) sums
// the chunks k = j, j + tpg, ... in increasing order (coalesced along g;
// loads issued kFinalizeBatch at a time), a fixed tree over j follows, and
// mean/rstd are written.  The arrival counter is reset to zero for the next
// call.  Every batch, the last one included, issues all its loads before the
// first add, so a short tail costs one round trip, not one per chunk.
template <class D>
__device__ __forceinline__ void finalize_sample(const typename D::storage *xs,
                                                const Geometry &geo, int64_t n,
                                                const StatsOut &out, float *red_s, float *red_q,
                                                int tid) {
    const int G = geo.G;
    const int tpg = kThreads / G;
    const bool has = tid < tpg * G;
    const int g = tid % G;
    const int j = tid / G;
    float as = 0.0f, aq = 0.0f;
    if (has) {
        const float *ps = out.part_s + n * geo.K * G + g;
        const float *pq = out.part_q + n * geo.K * G + g;
        for (int64_t kk = j; kk < geo.K; kk += kFinalizeBatch * tpg) {
            FinalizeBatch<true> fb;
            fb.load(ps, pq, kk, tpg, G);
            __builtin_amdgcn_sched_barrier(0);  // all loads issued before the adds
            fb.add(kk, tpg, geo.K, as, aq);
        }
    }
    const float pivot = has && j == 0 ? D::to_f32(xs[static_cast<int64_t>(g) * geo.Cg]) : 0.0f;
    finalize_groups(as, aq, has, j, g, G, tpg, pivot, out.inv_m, out.eps, red_s, red_q, tid,
                    out.mean + n * G + g, out.rstd + n * G + g);
    if (tid == 0)
        __hip_atomic_store(out.arrivals + n * arrival_stride(geo.K), 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Step 2 folded into step 3 (the "late" finalize, for samples whose chunk
// partials one batch covers: K1 <= kFinalizeBatch * (kThreads / G)): step 1
// only writes its partials, and every step-3 workgroup reduces its sample's
// partials itself, with the loads, the order of the adds and the tree of the
// fused finalize, so mean/rstd are bitwise the same.
struct LateStats {
    const float *part_s;  // [N][K1][G] from step 1
    const float *part_q;
    const float *pivot;   // [N][G], the pivots step 1 used (StatsOut::pivot)
    int64_t K1;           // chunks per sample of step 1
    double inv_m;         // 1 / (L*Cg)
    float eps;
    // Not the late finalize: the arrival counters step 1 of the same call
    // used (or null), arrival_words per sample.  Workgroup 0 of each sample
    // sets them to zero, so a counter left non-zero by calls that overlapped
    // on the same scratch cannot disturb the calls after this one.
    unsigned *arrivals;
    int64_t arrival_words;
};

// gamma and beta: C values each, or null (1 and 0), of element type kF32,
// kBf16 or kF16; widened exactly to fp32 before the fold.
struct Affine {
    enum : int { kF32 = 0, kBf16 = 1, kF16 = 2 };
    const void *gamma;
    const void *beta;
    int type;
};

// A lane's channel parameters as loaded: the 32-bit words holding gamma and
// beta (of the Affine type; a 16-bit value starts at bit hg[j] / hb[j] of its
// word) and its groups' mean and rstd.  They are widened and combined only
// later, in fold_affine, so no instruction between the loads waits for them.
template <int S> struct SlotParams {
    uint32_t g[S], b[S];
    uint32_t hg[S], hb[S];
    float mu[S], rs[S];
};

// Reads gamma and beta of one channel.  An absent one is read from
// `fallback` (any valid 4-byte-aligned address, offset 0) and replaced by 1 or
// 0 in fold_affine.  Every element type is read with the same 32-bit load of
// the aligned word that holds the value, so no branch on the type separates
// the loads (at the end of such a branch the compiler waits for the loads
// issued in it).  A 16-bit value shares its word with a neighbour that may lie
// just outside the array; an aligned 32-bit word never crosses a page.
struct AffineReader {
    const char *gw, *bw;  // each array's start rounded down to 4 bytes
    uint32_t g2, b2;      // start mod 4 (0 or 2)
    uint32_t gm, bm;      // channel mask: all ones, or 0 for an absent parameter
    int es;               // log2 of the element size
    __device__ __forceinline__ AffineReader(const Affine &af, const void *fallback) {
        const char *g = static_cast<const char *>(af.gamma ? af.gamma : fallback);
        const char *b = static_cast<const char *>(af.beta ? af.beta : fallback);
        g2 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(g)) & 2u;
        b2 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(b)) & 2u;
        gw = g - g2;
        bw = b - b2;
        gm = af.gamma ? ~0u : 0u;
        bm = af.beta ? ~0u : 0u;
        es = af.type == Affine::kF32 ? 2 : 1;
    }
    // t: the value's byte offset from the rounded-down start.
    __device__ __forceinline__ static uint32_t word(const char *w, uint32_t t, uint32_t &h) {
        h = (t & 2u) * 8;  // 0 or 16; 0 for fp32
        return *reinterpret_cast<const uint32_t *>(w + (t & ~3u));
    }
    template <int S>
    __device__ __forceinline__ void load(int c, int j, SlotParams<S> &pr) const {
        pr.g[j] = word(gw, ((static_cast<uint32_t>(c) & gm) << es) + g2, pr.hg[j]);
        pr.b[j] = word(bw, ((static_cast<uint32_t>(c) & bm) << es) + b2, pr.hb[j]);
    }
};

// Issues the loads of the lane's parameters; their round trips overlap.  An
// absent gamma or beta is read from `mean` (AffineReader).
// STATS: also load mean/rstd of the slots' groups from mean[n*G + g] (else
// the caller fills pr.mu / pr.rs; `mean` is then only a valid address).
template <class L, bool POW2, bool STATS>
__device__ __forceinline__ void load_slot_params(const float *mean, const float *rstd,
                                                 const Affine &af, const Geometry &geo,
                                                 const TileGeo<POW2, L::kSlots> &tg_, int64_t n,
                                                 int tid, SlotParams<L::kSlots> &pr) {
    constexpr int S = L::kSlots;
    int c[S];
#pragma unroll
    for (int j = 0; j < S; ++j) {
        c[j] = tg_.channel(L::slot_offset(tg_.lanes(), tid, j));
        if constexpr (STATS) {
            const int64_t gi = n * geo.G + tg_.group_of(c[j]);
            pr.mu[j] = mean[gi];
            pr.rs[j] = rstd[gi];
        }
    }
    const AffineReader rd(af, mean);
#pragma unroll
    for (int j = 0; j < S; ++j) rd.load(c[j], j, pr);
}

// gamma or beta bits of the Affine type for the lane's slots, widened exactly
// to fp32 (`absent` where the parameter is null).  Presence and type are the
// same for the whole launch, so they are decided once, outside the slots: a
// choice per slot and value compiles to a chain of scalar branches for each
// of them, which the fold runs after the statistics are known.
template <int S>
__device__ __forceinline__ void widen_affine(const uint32_t (&bits)[S], const uint32_t (&h)[S],
                                             const void *p, int type, float absent,
                                             float (&out)[S]) {
    if (p == nullptr) {
#pragma unroll
        for (int j = 0; j < S; ++j) out[j] = absent;
    } else if (type == Affine::kBf16) {
#pragma unroll
        for (int j = 0; j < S; ++j) out[j] = Bf16::to_f32(static_cast<uint16_t>(bits[j] >> h[j]));
    } else if (type == Affine::kF16) {
#pragma unroll
        for (int j = 0; j < S; ++j) out[j] = Fp16::to_f32(static_cast<uint16_t>(bits[j] >> h[j]));
    } else {
#pragma unroll
        for (int j = 0; j < S; ++j) out[j] = __uint_as_float(bits[j]);
    }
}

// scale = gamma*rstd, shift = beta - mean*scale for the lane's slots.
template <int S>
__device__ __forceinline__ void fold_affine(const SlotParams<S> &pr, const Affine &af,
                                            float (&sc)[S], float (&sh)[S]) {
    float ga[S], be[S];
    widen_affine<S>(pr.g, pr.hg, af.gamma, af.type, 1.0f, ga);
    widen_affine<S>(pr.b, pr.hb, af.beta, af.type, 0.0f, be);
#pragma unroll
    for (int j = 0; j < S; ++j) {
        sc[j] = ga[j] * pr.rs[j];
        sh[j] = fmaf(-pr.mu[j], sc[j], be[j]);
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

// ---------------------------------------------------------------------------
// Step 1: partial statistics.  One workgroup per (sample n, chunk k); writes
// the pivot-shifted sum and sum of squares of each group over its chunk to
// part_s / part_q at [(n*K + k)*G + g].
// Cache policy: step 3 reads x again, and whatever of x is still in the
// 256 MB Infinity Cache when step 3 starts is served from there.  The last
// geo.plain_tail tiles of every chunk -- together about one cache's worth,
// the part read last -- use plain loads, which allocate in that cache; the
// tiles before them use nontemporal loads, which would only be evicted again
// before step 3 and cost bandwidth to allocate.
// FUSED (requires G <= kThreads): the last workgroup of sample n to finish,
// found with an agent-scope atomic counter, also performs step 2 for that
// sample -- a fixed-order reduction over the K chunk partials of each group,
// whichever workgroup happens to be last -- and resets the counter to zero.
// Ordering: every lane waits for its write-through partial stores to
// complete (s_waitcnt vmcnt(0)), the workgroup barrier follows, and only then
// is the arrival counted; the last workgroup reads the partials with
// agent-scope (coherent) loads.
// ---------------------------------------------------------------------------
// Step 1 launches about one workgroup per CU, so its occupancy target is one
// or two waves per SIMD: with that, the compiler keeps a whole batch of
// UNROLL tiles in flight and starts accumulating as the first arrives, where
// a higher target made it interleave waits into the loads (fully serialized
// for 16-bit wide tiles) to save registers.
// NT: lanes per workgroup, kThreads or more for the wide-channel layouts
// (the group reduction and the fused finalize keep their 256-thread mapping;
// the other threads of a wider workgroup hold no entry there).
template <class D, int W, int NV, bool POW2, int UNROLL, bool FUSED, int NT = kThreads>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 2))) void
gn_partial_stats(
    const typename D::storage *__restrict__ x, Geometry geo, StatsOut out) {
    static_assert(NT == kThreads || !POW2, "power-of-two tiles take 256-lane workgroups");
    using L = Lane<D, W, NV>;
    constexpr int S = L::kSlots;
    __shared__ float red_s[NT * S];
    __shared__ float red_q[NT * S];

    const TileGeo<POW2, S> tg(geo);
    const int64_t T = tg.tile();
    const int A = tg.lanes();
    const int tid = threadIdx.x;
    const int64_t wg = blockIdx.x;
    const int64_t n = wg / geo.K;
    const int64_t k = wg - n * geo.K;
    const typename D::storage *xs = x + n * geo.E;
    const bool active = POW2 || tid < A;  // power-of-two tiles: every lane

    float piv[S], s[S], q[S];
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const int c = tg.channel(L::slot_offset(A, active ? tid : 0, j));
        piv[j] = D::to_f32(xs[tg.group_of(c) * geo.Cg]);
        s[j] = 0.0f;
        q[j] = 0.0f;
    }

    if (!FUSED && out.pivot != nullptr && k == 0) {
        for (int g = tid; g < geo.G; g += NT)
            out.pivot[n * geo.G + g] = D::to_f32(xs[static_cast<int64_t>(g) * geo.Cg]);
    }

    const ChunkRange cr = chunk_range(geo, k);
    if (active) {
        const typename D::storage *p = xs + cr.t_begin * T;  // current tile
        int64_t tt = cr.t_begin;
        int64_t t_plain = cr.t_end - geo.plain_tail;  // first tile read with plain loads
        if (t_plain > cr.t_full_end) t_plain = cr.t_full_end;
        // Each batch issues all its loads before the first add.  Where the
        // compiler did not do so by itself, a scheduling barrier keeps it
        // from moving adds, and the waits they need, in between: in the
        // 320-lane fp16 build it had waited for every load before issuing the
        // next, and some builds with two or four accesses per lane and tile
        // waited part-way.  (One access per lane in 256-lane workgroups
        // already issued whole batches, and is left as it was.)
        constexpr bool kPin = NT != kThreads || NV > 1;
        for (; tt + UNROLL <= t_plain; tt += UNROLL) {
            L v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) v[u] = L::template load<true>(p + u * T, A, tid);
            if constexpr (kPin) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) accumulate<L>(v[u], piv, s, q);
            p += UNROLL * T;
        }
        for (; tt + UNROLL <= cr.t_full_end; tt += UNROLL) {
            L v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) v[u] = L::template load<false>(p + u * T, A, tid);
            if constexpr (kPin) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) accumulate<L>(v[u], piv, s, q);
            p += UNROLL * T;
        }
        if (tt < cr.t_full_end) {
            // Fewer than UNROLL whole tiles left: one batch all the same, its
            // surplus loads re-reading the last whole tile and not accumulated.
            const int rem = static_cast<int>(cr.t_full_end - tt);
            L v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                v[u] = L::template load<false>(p + (u < rem ? u : rem - 1) * T, A, tid);
            if constexpr (kPin) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                if (u < rem) accumulate<L>(v[u], piv, s, q);
            tt += rem;
        }
        if (tt < cr.t_end) {
            // The sample's last tile is partial: slot by slot, in bounds only.
#pragma unroll
            for (int j = 0; j < S; ++j) {
                const int64_t off = tt * T + L::slot_offset(A, tid, j);
                if (off < geo.E) accumulate1(D::to_f32(xs[off]), piv[j], s[j], q[j]);
            }
        }
    }

    write_group_partials<L, POW2, FUSED, NT>(s, q, red_s, red_q, geo, tg, n, k, out, tid);
    if constexpr (FUSED) {
        if (arrive_is_last(out, n, geo.K, k, tid))
            finalize_sample<D>(xs, geo, n, out, red_s, red_q, tid);
    }
}

// ---------------------------------------------------------------------------
// Step 2 as its own kernel (G > kThreads: too many groups for one workgroup
// to finish quickly; and from 16 to 160 MiB, where it measured faster than
// the fused tail): one workgroup per (n, g).  Thread t sums chunks t,
// t + kThreads, ... in increasing order; each wave reduces its 64 sums with
// an xor butterfly (every lane ends with the same bits), and thread 0 adds
// the four wave sums in wave order -- a fixed order, so the statistics are
// reproducible.  The group's pivot is loaded with the partials (by every
// thread, see below), so the kernel waits for one memory round trip, not two.
// ---------------------------------------------------------------------------
template <class D>
__global__ __launch_bounds__(kThreads) void gn_finalize_stats(
    const typename D::storage *__restrict__ x, Geometry geo, StatsOut out) {
    constexpr int kWaves = kThreads / 64;
    __shared__ float ws[kWaves], wq[kWaves];
    const int tid = threadIdx.x;
    const int64_t ng = blockIdx.x;
    const int64_t n = ng / geo.G;
    const int g = static_cast<int>(ng - n * geo.G);
    // Every thread loads the pivot's raw bits (one address for the
    // workgroup), converted only at the end: loaded under a branch on tid,
    // the compiler waited for it at the branch's end, before issuing the
    // partial loads, so the kernel waited for two round trips.
    const typename D::storage praw = x[n * geo.E + static_cast<int64_t>(g) * geo.Cg];
    float s = 0.0f, q = 0.0f;
    for (int64_t k = tid; k < geo.K; k += kThreads) {
        const int64_t o = (n * geo.K + k) * geo.G + g;
        s += out.part_s[o];
        q += out.part_q[o];
    }
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
        s += __shfl_xor(s, m, 64);
        q += __shfl_xor(q, m, 64);
    }
    if ((tid & 63) == 0) {
        ws[tid >> 6] = s;
        wq[tid >> 6] = q;
    }
    __syncthreads();
    if (tid == 0) {
        float ts = ws[0], tq = wq[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            ts += ws[w];
            tq += wq[w];
        }
        group_moments(ts, tq, D::to_f32(praw), out.inv_m, out.eps, out.mean + ng,
                      out.rstd + ng);
    }
}

// Zero-fill for the arrival counters of a fresh scratch buffer (a kernel, so
// the clearing is ordinary stream work).
__global__ __launch_bounds__(kThreads) void gn_zero_u32(unsigned *p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Step 3: fused apply.  One workgroup per (n, chunk); each active lane folds
// gamma/beta and the group statistics of its slots into scale/shift
// registers once (scale = gamma*rstd, shift = beta - mean*scale), then
// streams its chunk: y = SiLU(x*scale + shift), rounded once to D.
// x and y may be the same buffer (each element is read, then written, by one
// lane), so they carry no __restrict__.
// ---------------------------------------------------------------------------
// FIN: the late finalize -- the workgroup first reduces its sample's step-1
// partials (ls) to mean/rstd in LDS, every thread taking part, and `mean` /
// `rstd` are not read.  NT: lanes per workgroup (kThreads, or more for the
// wide-channel layouts whose tiles need more lanes to keep all of them busy).
// FIN: 0, or the late finalize with batches of FIN slots (4, 8 or 16: the
// fewest that cover the sample's chunks, K1 <= FIN * kThreads / G; the same
// chunks, added in the same order, whatever FIN is).
template <class D, int W, int NV, bool POW2, int UNROLL, bool SILU, bool NTL, bool NTS, int FIN,
          int NT = kThreads>
__global__ __launch_bounds__(NT) void gn_apply(
    const typename D::storage *x, typename D::storage *y, Geometry geo,
    const float *__restrict__ mean, const float *__restrict__ rstd, Affine af, LateStats ls) {
    static_assert(NT == kThreads || (!FIN && !POW2), "the late finalize and the power-of-two "
                                                   "tiles take 256-lane workgroups");
    using L = Lane<D, W, NV>;
    constexpr int S = L::kSlots;
    const TileGeo<POW2, S> tg(geo);
    const int64_t T = tg.tile();
    const int A = tg.lanes();
    const int tid = threadIdx.x;
    const bool active = POW2 || tid < A;  // power-of-two tiles: every lane
    const int64_t wg = blockIdx.x;
    const int64_t n = wg / geo.K;
    const int64_t k = wg - n * geo.K;
    const int64_t base = n * geo.E;
    if (ls.arrivals != nullptr && k == 0) {
        for (int64_t w = tid; w < ls.arrival_words; w += NT)
            __hip_atomic_store(ls.arrivals + n * ls.arrival_words + w, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if constexpr (!FIN) {
        if (!active) return;
    }

    // Late finalize, first its loads: the partials of (group g, part j) --
    // K1 <= kFinalizeBatch*tpg, so the fused finalize's first (only) batch;
    // a thread with no part (j >= K1) loads part 0's, which stays within the
    // same bound, and adds none -- and the group's pivot x[n, 0, g*Cg] as
    // step 1 saved it (x itself may already hold y here).
    const int G = geo.G;
    const int tpg = kThreads / G;
    const bool fin_has = FIN && tid < tpg * G;
    const int fg = tid % G;
    const int fj = tid / G;
    FinalizeBatch<false, (FIN > 0 ? FIN : 1)> fb;
    // No load of the prologue sits under a branch on the thread index: at the
    // end of such a branch the compiler waits for the loads issued in it (or
    // for an add it moved in there), before the loads after it are issued.
    // So every thread loads its group's pivot (only the part j = 0 uses it)
    // and a batch of partials.
    const bool fin_part = fin_has && fj < ls.K1;
    float pivot = 0.0f;
    if constexpr (FIN) {
        pivot = ls.pivot[n * G + fg];
        fb.load(ls.part_s + n * ls.K1 * G + fg, ls.part_q + n * ls.K1 * G + fg,
                fin_part ? fj : 0, tpg, G);
        __builtin_amdgcn_sched_barrier(0);  // these first: the finalize waits for them only
    }

    // The parameter loads are issued next and the chunk's first batch of x
    // right after them; the fold then waits for the parameters only (loads
    // return in order), so the round trips overlap.
    SlotParams<S> pr;
    if (active) load_slot_params<L, POW2, !FIN>(mean, rstd, af, geo, tg, n, tid, pr);

    const ChunkRange cr = chunk_range_even(geo, k);
    int64_t off = base + cr.t_begin * T;  // current tile
    int64_t tt = cr.t_begin;
    const int64_t nb = (cr.t_full_end - tt) / UNROLL;  // whole batches
    L a[UNROLL], b[UNROLL];
    auto load_batch = [&](L (&v)[UNROLL], int64_t o0) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = L::template load<NTL>(x + o0 + u * T, A, tid);
    };
    // A chunk with fewer than UNROLL whole tiles has one batch, the tail batch
    // (its surplus slots re-reading the last whole tile): it is issued here
    // too, so that its round trip also overlaps the parameters'.
    auto load_tail = [&](L (&v)[UNROLL], int64_t o0, int rem) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            v[u] = L::template load<NTL>(x + o0 + (u < rem ? u : rem - 1) * T, A, tid);
    };
    const int first = nb > 0 ? UNROLL : static_cast<int>(cr.t_full_end - tt);
    if (active && first > 0) load_tail(a, off, first);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FIN) {
        __shared__ float red_s[kThreads], red_q[kThreads];
        __shared__ float s_mean[kThreads], s_rstd[kThreads];
        float as = 0.0f, aq = 0.0f;
        fb.add(fin_part ? fj : 0, tpg, fin_part ? ls.K1 : 0, as, aq);
        finalize_groups(as, aq, fin_has, fj, fg, G, tpg, pivot, ls.inv_m, ls.eps, red_s, red_q,
                        tid, s_mean + fg, s_rstd + fg);
        __syncthreads();
        if (!active) return;
#pragma unroll
        for (int j = 0; j < S; ++j) {
            const int g = tg.group_of(tg.channel(L::slot_offset(A, tid, j)));
            pr.mu[j] = s_mean[g];
            pr.rs[j] = s_rstd[g];
        }
    }
    float sc[S], sh[S];
    fold_affine<S>(pr, af, sc, sh);
    auto apply_batch = [&](const L (&v)[UNROLL], int64_t o0) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float o[S];
#pragma unroll
            for (int j = 0; j < S; ++j) o[j] = transform1<SILU>(v[u].get(j), sc[j], sh[j]);
            L::template store<NTS>(y + o0 + u * T, A, tid, o);
        }
    };
    // Whole batches, software-pipelined in two register sets.  One in-order
    // counter covers loads and stores, so waiting for a batch's loads also
    // waits for every older store; loading batch i+1 before storing batch i
    // keeps the stores out of that wait.  The last one or two batches are
    // peeled, so no batch is loaded twice; in place (x == y) every tile is
    // still loaded before it is stored.  Measured on MI355X against the plain
    // load-then-store loop: 2-5% faster step 3 for 16-bit data from 32 MiB to
    // 1 GiB, 3-15% on wide tiles, 0-3% in fp32, 2% slower at C = 1280.
    if (nb > 0) {  // batch 0 is in flight in a
        const int64_t step = UNROLL * T;
        int64_t i = 0;
        for (; i + 3 <= nb; i += 2) {  // batches i, i+1 and i+2 exist
            load_batch(b, off + step);
            __builtin_amdgcn_sched_barrier(0);
            apply_batch(a, off);
            load_batch(a, off + 2 * step);
            __builtin_amdgcn_sched_barrier(0);
            apply_batch(b, off + step);
            off += 2 * step;
        }
        if (i + 2 <= nb) {  // two batches left, the first in a
            load_batch(b, off + step);
            __builtin_amdgcn_sched_barrier(0);
            apply_batch(a, off);
            apply_batch(b, off + step);
            off += 2 * step;
        } else {  // one batch left, in a
            apply_batch(a, off);
            off += step;
        }
        tt += nb * UNROLL;
    }
    if (tt < cr.t_full_end) {
        // Fewer than UNROLL whole tiles left: one batch of loads (the surplus
        // re-reading the last whole tile, before any store of the batch; in
        // a chunk with no whole batch, loaded ahead of the fold), and stores
        // for the real tiles only.
        const int rem = static_cast<int>(cr.t_full_end - tt);
        if (nb > 0) load_tail(a, off, rem);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if (u < rem) {
                float o[S];
#pragma unroll
                for (int j = 0; j < S; ++j) o[j] = transform1<SILU>(a[u].get(j), sc[j], sh[j]);
                L::template store<NTS>(y + off + u * T, A, tid, o);
            }
        }
        tt += rem;
    }
    if (tt < cr.t_end) {
        // The sample's last tile is partial: slot by slot, in bounds only.
#pragma unroll
        for (int j = 0; j < S; ++j) {
            const int64_t rel = tt * T + L::slot_offset(A, tid, j);
            if (rel < geo.E)
                y[base + rel] = D::from_f32(transform1<SILU>(D::to_f32(x[base + rel]), sc[j], sh[j]));
        }
    }
}

// ---------------------------------------------------------------------------
// Single launch for small tensors: steps 1-3 in one kernel with no
// communication between workgroups.  A workgroup owns a strip of gpw whole,
// consecutive groups of one sample -- every row of those gpw*Cg channels --
// so it finishes their statistics alone: it loads the strip once into
// registers (at most kStripPieces 16-byte pieces per lane), reduces each
// group in a fixed order, folds gamma/beta and applies from the registers.
// Nothing waits on another workgroup, so no co-residency is needed and no
// partials go through memory.
//
// Where it pays: a strip row is narrower than a cache line, so every row a
// workgroup reads costs a whole line fill of its CU's L1 -- the strip's rows,
// not its bytes, set the time, and one workgroup per group cannot spread a
// long group over more CUs.  The host takes this path only for short strips
// (at most kStripPieces pieces per lane) and at most one workgroup per CU;
// larger tensors take the three-step path.
//
// Layout: the strip's rows are P 16-byte pieces wide (P = gpw*Cg / W, a power
// of two <= 64); lane tid always takes piece p = tid % P of rows
// tid / P + k*(NT/P), k < kStripPieces, so its W slots keep the channels
// cs + p*W + j (cs: the strip's first channel) and its scale/shift stay in
// registers.  SUB = min(Cg, W): a piece holds W/SUB whole groups (Cg <= W) or
// a W-channel part of one group (Cg > W).
// Reduction, fixed order: each lane sums its pieces per slot (pivot-shifted,
// as in step 1), its slots per group part, then a butterfly over the lanes
// of its wave with the same p; per (wave, piece, part) one LDS entry; per
// group a tree over its entries (waves x pieces of the group).
// ---------------------------------------------------------------------------
constexpr int kStripThreads = 1024;  // 16 waves: one workgroup per CU
constexpr int kStripPieces = 2;      // 16-byte pieces per lane, at most

struct StripGeo {
    int64_t L;        // rows per sample
    int64_t E;        // elements per sample, L*C
    int C, G, Cg;
    int gpw;          // groups per strip
    int P;            // 16-byte pieces per strip row (power of two, <= 64)
    int S;            // strips per sample, G / gpw
    int xcd;          // 1: workgroup b takes strip (b % 8) * (blocks / 8) + b / 8
    int64_t blocks;   // N * S
    double inv_m;     // 1 / (L*Cg)
    float eps;
};

// v summed over the lanes of the wave whose lane index agrees with this
// lane's in the bits below `low` (a power of two): xor butterfly, fixed
// order, every such lane ends with the same total.
__device__ __forceinline__ float wave_sum_same_low(float v, int low) {
    const int lane = static_cast<int>(threadIdx.x) & 63;
    for (int m = 32; m >= low; m >>= 1) {
        const int o = __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __float_as_int(v));
        v += __int_as_float(o);
    }
    return v;
}

// stats_only (uniform, at run time): write the strip's groups' mean/rstd to
// mean_out/rstd_out [N][G] and stop (steps 1-2 alone; the apply kernel then
// gives the same y as the full single launch, bit for bit: the same fold and
// transform of the same fp32 statistics).
template <class D, int SUB, bool SILU>
__global__ __launch_bounds__(kStripThreads) void gn_strip(
    const typename D::storage *x, typename D::storage *y, StripGeo geo, Affine af,
    int stats_only, float *__restrict__ mean_out, float *__restrict__ rstd_out) {
    using T = typename D::storage;
    constexpr int W = static_cast<int>(16 / sizeof(T));
    constexpr int NT = kStripThreads;
    constexpr int NW = NT / 64;
    constexpr int NS = W / SUB;  // group parts per piece
    using V = Vec<D, W>;
    static_assert(W % SUB == 0, "SUB divides the piece");
    __shared__ float ent_s[NW * 64 * NS], ent_q[NW * 64 * NS];  // per (wave, piece, part)
    __shared__ float red_s[NT], red_q[NT];
    __shared__ float s_mean[64 * NS], s_rstd[64 * NS];

    const int tid = threadIdx.x;
    int64_t b = blockIdx.x;
    if (geo.xcd) b = (b % 8) * (geo.blocks / 8) + b / 8;
    const int64_t n = b / geo.S;
    const int strip = static_cast<int>(b - n * geo.S);
    const int cs = strip * geo.gpw * geo.Cg;
    const T *xs = x + n * geo.E + cs;
    T *ys = y + n * geo.E + cs;
    const int P = geo.P;
    const int p = tid & (P - 1);
    const int64_t r0 = tid / P;
    const int64_t rstep = NT / P;
    const int cw = p * W;  // the piece's first channel within the strip
    const int64_t C = geo.C;

    // the strip's pieces, issued first
    V v[kStripPieces];
#pragma unroll
    for (int k = 0; k < kStripPieces; ++k) {
        const int64_t r = r0 + k * rstep;
        if (r < geo.L) v[k].template load<false>(xs + r * C + cw);
    }
    // pivots: the group's first element in row 0 (as step 1 takes them)
    float piv[W], s[W], q[W];
#pragma unroll
    for (int j = 0; j < W; ++j) {
        const int lg = (cw + j) / geo.Cg;
        piv[j] = D::to_f32(xs[lg * geo.Cg]);
        s[j] = 0.0f;
        q[j] = 0.0f;
    }
    // gamma / beta of the lane's channels: issued now, used after the reduction.
    // The loads of x are already in flight and the sums wait for them anyway,
    // so here a branch on the element type costs little, and the typed loads
    // take fewer address instructions than AffineReader's (measured faster).
    SlotParams<W> pr;
    {
        const void *gp = af.gamma ? af.gamma : static_cast<const void *>(x);
        const void *bp = af.beta ? af.beta : static_cast<const void *>(x);
        const int gs = af.gamma ? 1 : 0, bs = af.beta ? 1 : 0;
        const int c0 = cs + cw;
        if (af.type == Affine::kF32) {
#pragma unroll
            for (int j = 0; j < W; ++j) {
                pr.g[j] = static_cast<const uint32_t *>(gp)[(c0 + j) * gs];
                pr.b[j] = static_cast<const uint32_t *>(bp)[(c0 + j) * bs];
            }
        } else {
#pragma unroll
            for (int j = 0; j < W; ++j) {
                pr.g[j] = static_cast<const uint16_t *>(gp)[(c0 + j) * gs];
                pr.b[j] = static_cast<const uint16_t *>(bp)[(c0 + j) * bs];
            }
        }
#pragma unroll
        for (int j = 0; j < W; ++j) pr.hg[j] = pr.hb[j] = 0;  // each value at bit 0
    }
#pragma unroll
    for (int k = 0; k < kStripPieces; ++k) {
        if (r0 + k * rstep < geo.L) {
#pragma unroll
            for (int j = 0; j < W; ++j) accumulate1(v[k].get(j), piv[j], s[j], q[j]);
        }
    }

    // slots -> group parts (SUB consecutive slots each), then the wave's
    // lanes with the same piece
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        float ps = 0.0f, pq = 0.0f;
#pragma unroll
        for (int j = u * SUB; j < (u + 1) * SUB; ++j) {
            ps += s[j];
            pq += q[j];
        }
        ps = wave_sum_same_low(ps, P);
        pq = wave_sum_same_low(pq, P);
        if (lane < P) {
            ent_s[(wave * P + lane) * NS + u] = ps;
            ent_q[(wave * P + lane) * NS + u] = pq;
        }
    }
    __syncthreads();

    // Entries of local group lg: Cg <= W: one per wave, piece lg*Cg / W,
    // part (lg*Cg % W) / SUB; Cg > W: Cg/W per wave, the group's pieces.
    // Entry e = wave*EPW + k, EPW = max(1, Cg/W): EPW*NW entries per group, a
    // power of two; thread lg*EN + e holds entry e of group lg, a fixed tree
    // over e follows.
    const int EPW = geo.Cg > W ? geo.Cg / W : 1;
    const int EN = EPW * NW;
    {
        const int lg = tid / EN, e = tid - lg * EN;
        const bool has = lg < geo.gpw;
        float as = 0.0f, aq = 0.0f;
        if (has) {
            const int w = e / EPW, k = e - w * EPW;
            int pc, part;
            if (geo.Cg > W) {
                pc = lg * EPW + k;
                part = 0;
            } else {
                pc = (lg * geo.Cg) / W;
                part = ((lg * geo.Cg) % W) / SUB;
            }
            as = ent_s[(w * P + pc) * NS + part];
            aq = ent_q[(w * P + pc) * NS + part];
        }
        red_s[tid] = as;
        red_q[tid] = aq;
        __syncthreads();
        tree_sum(red_s, red_q, lg * EN, 1, has ? e : -1, EN);
        if (has && e == 0) {
            float mu, rs;
            group_moments(red_s[tid], red_q[tid], D::to_f32(xs[lg * geo.Cg]), geo.inv_m,
                          geo.eps, &mu, &rs);
            s_mean[lg] = mu;
            s_rstd[lg] = rs;
            if (stats_only) {
                const int64_t gi = n * geo.G + static_cast<int64_t>(strip) * geo.gpw + lg;
                mean_out[gi] = mu;
                rstd_out[gi] = rs;
            }
        }
    }
    if (stats_only) return;
    __syncthreads();

#pragma unroll
    for (int j = 0; j < W; ++j) {
        const int lg = (cw + j) / geo.Cg;
        pr.mu[j] = s_mean[lg];
        pr.rs[j] = s_rstd[lg];
    }
    float sc[W], sh[W];
    fold_affine<W>(pr, af, sc, sh);
#pragma unroll
    for (int k = 0; k < kStripPieces; ++k) {
        const int64_t r = r0 + k * rstep;
        if (r < geo.L) {
            float o[W];
#pragma unroll
            for (int j = 0; j < W; ++j) o[j] = transform1<SILU>(v[k].get(j), sc[j], sh[j]);
            V::template store<true>(ys + r * C + cw, o);
        }
    }
}

}  // namespace gnsilu
