// gn_conv.hpp -- gfx950 (CDNA4) 3x3 NHWC convolution with the GroupNorm(+SiLU)
// of its input fused into the prologue and the statistics of its output for
// the next GroupNorm fused into the epilogue.
//
// The fusion is the one the decoder's ResnetBlock2D invites ("FLUX.2 VAE
// decoder fast path behind quality=high", Modifications section 2: the
// ResnetBlock2D norm1/norm2 + SiLU chains around its Conv2d(3x3, p1)): the
// normalised activation y = SiLU(GroupNorm(x)) exists only in LDS, on its way
// into the matrix cores, and the output's per-group moments are taken while
// the output tile is still on chip, so the two elementwise passes of the
// GroupNorm between two convolutions disappear.
//
//   z[n,h,w,co] = bias[co] + res[n,h,w,co]
//               + sum_{kh,kw,ci} wt[co,kh,kw,ci] * y[n,h+kh-1,w+kw-1,ci]   (y = 0 outside)
//   y = SiLU?(gamma[ci] * (x - mean[n,g]) * rstd[n,g] + beta[ci])          (or y = x)
//
// Implicit GEMM on the matrix cores: M = output pixels, N = output channels,
// K = 9 taps x Ci.  A workgroup of 256 lanes owns an 8 x 16 pixel output tile
// and 256 output channels, each of its four waves 128 pixels x 64 channels as
// 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (when Co is not a multiple of 256:
// 128 channels, each wave 64 pixels x 64 channels as 2 x 2 blocks).  Per
// chunk of 32 input channels:
//   * the 10 x 18 pixel halo of the tile is normalised (+SiLU) with
//     per-channel scale/shift held in LDS, rounded to bf16 and stored to one
//     of two LDS halo buffers -- every input value is transformed once per
//     chunk, not once per tap.  The halo of chunk k+1 is loaded into
//     registers at tap 4 of chunk k-1 and normalised into the other buffer
//     at taps 1-3 of chunk k, so the loads have most of a chunk to arrive
//     and the VALU work overlaps the matrix-core work; one barrier per chunk;
//   * the nine taps run against it.  Each wave reads its weight fragments
//     straight from global memory (the weight slice of a workgroup stays in
//     its XCD's L2) into a ring of registers, two taps ahead of their use, so
//     no weight tile passes through LDS and no tap needs a barrier; its A
//     fragments come from LDS one tap ahead (64-pixel waves: into a second
//     register set; 128-pixel waves: each k-step's right after its products
//     are issued, which keeps the wave within 256 registers, two waves per
//     SIMD).
// LDS rows are 80 bytes (32 bf16 + 8 padding), so the 16-byte fragment reads
// of 16 consecutive lanes fall on distinct banks.
//
// Epilogue: the accumulators (+ bias) are staged as fp32 through LDS, 64
// output channels at a time, so that every lane adds the residual and writes
// z with 16-byte accesses; the bf16-rounded values (what the next GroupNorm
// reads) give, per tile and per output group, the count, mean and sum of
// squared deviations (M2), in a fixed order.  gn_conv_stats_finalize merges
// the tiles of each (n, group) in fp64 (pivot-shifted sums, one pass), in a
// fixed order, so the statistics are reproducible bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace gnconv {

constexpr int kThreads = 256;
constexpr int TH = 8, TW = 16;                 // output tile, pixels
constexpr int HH = TH + 2, HWD = TW + 2;       // halo tile
constexpr int BM = TH * TW;                    // 128 output pixels
constexpr int BN = 128;                        // output channels per workgroup
constexpr int BK = 32;                         // input channels per chunk
constexpr int KS = BK + 8;                     // LDS row stride of A and B, bf16 elements
constexpr int A_ELEMS = HH * HWD * KS;         // 7200 bf16 per halo buffer
constexpr int OS = 72;                         // epilogue fp32 row stride (64 + 8)
constexpr int kMaxCi = 1024;                   // scale/shift table in LDS
// Packed weights: per (output-channel block, step = chunk * 9 + tap) one run
// of kPackStep bf16 = 2 k-steps x 2 wave columns x 2 block columns x 64 lanes
// x 8 values; lane l of block column ni, wave column wn, k-step ks holds
// wt[cb*128 + wn*64 + ni*32 + l%32][tap][chunk*32 + ks*16 + 8*(l/32) + 0..7].
constexpr int kPackStep = 2 * 2 * 2 * 64 * 8;  // 4096 bf16 = 8 KiB
constexpr int kLdsBytesMain = 2 * A_ELEMS * 2;              // 28800: two halo buffers
constexpr int kLdsBytesEpi = BM * OS * 4;                    // 36864
constexpr int kLdsBytes = kLdsBytesMain > kLdsBytesEpi ? kLdsBytesMain : kLdsBytesEpi;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct ConvArgs {
    const uint16_t *x;      // [N][H][W][Ci] bf16
    const float *mean;      // [N][G] or null: no normalisation (y = SiLU?(x))
    const float *rstd;      // [N][G]
    const float *gamma;     // [Ci] or null (ones)
    const float *beta;      // [Ci] or null (zeros)
    const uint16_t *wt;     // weights packed by gn_conv_pack_weights (fragment order)
    const float *bias;      // [Co] or null
    const uint16_t *res;    // [N][H][W][Co] bf16 or null
    uint16_t *z;            // [N][H][W][Co] bf16
    float *part;            // [N][tiles][G2][4]: count, mean, M2, 0 (statistics only)
    int N, H, W, Ci, Co, G, G2;
    int tiles_h, tiles_w;   // ceil(H/8), ceil(W/16)
    int nb;                 // Co / (64*WN) output-channel blocks
    int xcd_map;            // 1: XCD-aware block order (nb divides 8)
    int64_t blocks;         // N * tiles_h * tiles_w * nb (real workgroups)
};

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float silu(float t) {
    const float e = __builtin_amdgcn_exp2f(t * -1.4426950408889634f);
    return t * __builtin_amdgcn_rcpf(1.0f + e);
}

// Workgroup -> (sample, tile, output-channel block).  Dispatch hands
// consecutive workgroups to the 8 XCDs in turn; with xcd_map, the XCDs are
// split into nb sets, each set working on one output-channel block (so each
// XCD's L2 holds one slice of the weights: 128 or 256 channels) and all sets walking
// the pixel tiles in the same order (so the nb reads of an input tile fall
// close together in time and share the Infinity Cache).
__device__ __forceinline__ bool map_block(const ConvArgs &a, int64_t b, int64_t *tile,
                                          int *cb) {
    if (a.xcd_map) {
        const int xcd = static_cast<int>(b & 7);
        const int64_t j = b >> 3;
        const int reps = 8 / a.nb;  // XCDs per output-channel block
        *cb = xcd % a.nb;
        *tile = j * reps + xcd / a.nb;
        return *tile < a.blocks / a.nb;
    }
    *cb = static_cast<int>(b % a.nb);
    *tile = b / a.nb;
    return b < a.blocks;
}

// ---------------------------------------------------------------------------
// SILU: apply SiLU after the normalisation; STATS: output moments; RES: add
// the residual.  The prologue always runs: without statistics it is the
// identity scale 1, shift 0 (fmaf(x, 1, 0) == x for every finite x), which
// costs one fma per input value and keeps every variant on the same
// instruction schedule -- without the transform between the halo load and
// its LDS store the compiler drains all outstanding loads at each store.
// ---------------------------------------------------------------------------
// WM x WN waves: WM along the tile's 128 pixels, WN along the output
// channels; a workgroup of 64*WM*WN lanes owns 64*WN output channels and each
// wave 128/WM pixels x 64 channels, as MI x 2 blocks of 32 x 32 (MI = 4/WM).
// WM = 2, WN = 2: 128 channels, 4 waves of 64 pixels.  WM = 1, WN = 4: 256
// channels, 4 waves of 128 pixels -- each weight fragment a wave pulls from
// L2 feeds twice the matrix-core work, and the normalised halo of a chunk
// serves twice as many outputs, so the prologue's loads and transcendentals
// per output halve.
// Two waves per SIMD (at most 256 registers a lane): one wave stalls on its
// loads while the other keeps the matrix core busy; left to itself the
// compiler gives the 128-pixel waves 384 registers and one wave per SIMD,
// measured 5-18% slower at the decoder shapes.  WPE = 1 is for grids of at
// most one workgroup per CU, where no second wave shares a SIMD anyway and the
// compiler may use the whole register file (measured at (1,512,128,128):
// 1-5% faster; with more workgroups 3-11% slower).
template <int WM, int WN, bool SILU, bool STATS, bool RES, int WPE = 2>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void
gn_conv3x3(ConvArgs a) {
    static_assert(WM == 1 || WM == 2, "a wave owns 128 or 64 pixels");
    constexpr bool PRO = true;
    constexpr int MI = 4 / WM;               // 32-pixel blocks per wave
    constexpr int NT = 64 * WM * WN;         // lanes
    constexpr int BNW = 64 * WN;             // output channels of the workgroup
    constexpr int ROWS = NT / 8;             // epilogue: lanes per 8-channel piece
    constexpr int PIX = BM / ROWS;           // epilogue: pixels per lane
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
    __shared__ float s_scale[kMaxCi];
    __shared__ float s_shift[kMaxCi];
    __shared__ __attribute__((aligned(16))) float s_stat[STATS ? 512 : 4];  // [2][4 waves][64]
    uint16_t *sA = reinterpret_cast<uint16_t *>(smem);  // two halo buffers of A_ELEMS
    float *sO = reinterpret_cast<float *>(smem);

    int64_t tile;
    int cb;
    if (!map_block(a, blockIdx.x, &tile, &cb)) return;  // padding workgroup: uniform exit
    const int tiles_per_sample = a.tiles_h * a.tiles_w;
    const int n = static_cast<int>(tile / tiles_per_sample);
    const int tin = static_cast<int>(tile - static_cast<int64_t>(n) * tiles_per_sample);
    const int h0 = (tin / a.tiles_w) * TH;
    const int w0 = (tin % a.tiles_w) * TW;
    const int co0 = cb * BNW;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int Ci = a.Ci;

    if constexpr (PRO) {
        if (a.mean) {
            const int Cg = Ci / a.G;
            for (int c = tid; c < Ci; c += NT) {
                const int gi = n * a.G + c / Cg;
                const float sc = (a.gamma ? a.gamma[c] : 1.0f) * a.rstd[gi];
                s_scale[c] = sc;
                s_shift[c] = fmaf(-a.mean[gi], sc, a.beta ? a.beta[c] : 0.0f);
            }
        } else {
            for (int c = tid; c < Ci; c += NT) {
                s_scale[c] = 1.0f;
                s_shift[c] = 0.0f;
            }
        }
        __syncthreads();
    }

    // Lane constants of the fragment reads: pixel p = lane % 32 of a 32-pixel
    // block (2 rows of 16), k offset 8 * (lane / 32); output channel
    // co0 + wn*64 + ni*32 + lane % 32 for the weights.
    const int fp = lane & 31, fk = 8 * (lane >> 5);
    const int frow = fp >> 4, fcol = fp & 15;
    const int nchunks = Ci / BK;
    const int nsteps = nchunks * 9;  // (chunk, tap) steps

    // Weight fragments come straight from global memory (L2) into registers,
    // two steps ahead of their use.  The packed layout puts the 64 lanes'
    // 16-byte fragments of one (block, step, k-step, wave column, block
    // column) next to each other, so each load is one contiguous 1 KiB.
    // (packed in 128-channel blocks: wave column wn reads block co0/128 + wn/2)
    const uint16_t *wwave = a.wt + static_cast<int64_t>(co0 / BN + wn / 2) * nsteps * kPackStep +
                            (wn % 2) * 2 * 512 + lane * 8;
    auto load_w = [&](int step, bf16x8 (&w)[2][2]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                w[ks][ni] = *reinterpret_cast<const bf16x8 *>(
                    wwave + static_cast<int64_t>(step) * kPackStep + ks * 4 * 512 + ni * 512);
    };

    // The halo tile of a chunk: 180 pixels x 4 pieces of 8 channels, PP
    // pieces per lane (a lane whose last piece would lie past the last one
    // redoes the last piece: the same value, written twice).  Loaded into
    // registers, then normalised and stored to one of the two LDS halo
    // buffers.  No branches: pixels outside the image load from a clamped
    // address and become zero by a select, so the whole chunk -- taps,
    // loads and the transform -- is one basic block the scheduler can
    // interleave with the matrix-core instructions.
    constexpr int kPieces = HH * HWD * 4;  // 720
    constexpr int PP = (kPieces + NT - 1) / NT;  // 3 (256 lanes) or 2 (512)
    int hoff[PP], hq[PP];
    bool hin[PP];
#pragma unroll
    for (int i = 0; i < PP; ++i) {
        const int v = min(tid + i * NT, kPieces - 1);
        const int p = v >> 2, q = v & 3;
        const int ih = h0 - 1 + p / HWD, iw = w0 - 1 + p % HWD;
        hin[i] = ih >= 0 && ih < a.H && iw >= 0 && iw < a.W;
        const int ihc = min(max(ih, 0), a.H - 1), iwc = min(max(iw, 0), a.W - 1);
        hoff[i] = p * KS + 8 * q;           // LDS offset
        hq[i] = (ihc * a.W + iwc) * Ci + 8 * q;  // element offset within the sample
    }
    const uint16_t *xs = a.x + static_cast<int64_t>(n) * a.H * a.W * Ci;
    auto load_halo = [&](int k, u32x4 (&raw)[PP]) {
#pragma unroll
        for (int i = 0; i < PP; ++i)
            raw[i] = *reinterpret_cast<const u32x4 *>(xs + hq[i] + k * BK);
    };
    auto store_piece = [&](int k, uint16_t *dst, const u32x4 &raw, int i) {
        u32x4 out;
        if constexpr (PRO) {
            const int c = k * BK + (hoff[i] % KS);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float lo = bf16_to_f32(raw[e] & 0xffffu);
                float hi = bf16_to_f32(raw[e] >> 16);
                lo = fmaf(lo, s_scale[c + 2 * e], s_shift[c + 2 * e]);
                hi = fmaf(hi, s_scale[c + 2 * e + 1], s_shift[c + 2 * e + 1]);
                if constexpr (SILU) {
                    lo = silu(lo);
                    hi = silu(hi);
                }
                out[e] = pack_bf16x2(lo, hi);
            }
        } else {
            out = raw;
        }
        const u32x4 zero = u32x4{0u, 0u, 0u, 0u};  // zero padding of y
        *reinterpret_cast<u32x4 *>(dst + hoff[i]) = hin[i] ? out : zero;
    };

    // Bias of the wave's output channels (co0 + wn*64 + ni*32 + lane % 32),
    // read once here rather than in the epilogue, where each read would wait
    // behind the stores before it.
    float bias_v[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
        bias_v[ni] = a.bias ? a.bias[co0 + wn * 64 + ni * 32 + (lane & 31)] : 0.0f;

    f32x16 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    bf16x8 wq[3][2][2];  // ring of weight fragments: step s in slot s % 3
    // A fragments of a tap from the current halo buffer: rows of the wave's
    // 32*MI pixels shifted by the tap, k-steps ks, pixel blocks mi.
    // With 64 pixels per wave the next tap's fragments go to a second
    // register set; with 128 there is one set, and each k-step's fragments of
    // the next tap are read as soon as that k-step's products are issued.
    constexpr int ASETS = MI == 2 ? 2 : 1;
    bf16x8 afr[ASETS][2][MI];  // [tap parity][ks][mi]
    // (the lane's part of the address is added once; the rest is a constant
    // offset of the LDS read)
    const int alane = ((wm * 2 * MI + frow) * HWD + fcol) * KS + fk;
    auto read_a_ks = [&](const uint16_t *abuf, int t, int ks, bf16x8 (&af)[MI]) {
        const int kh = t / 3, kw = t % 3;
        const uint16_t *ab = abuf + alane;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            af[mi] = *reinterpret_cast<const bf16x8 *>(ab + ((mi * 2 + kh) * HWD + kw) * KS + 16 * ks);
    };
    auto read_a = [&](const uint16_t *abuf, int t, bf16x8 (&af)[2][MI]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) read_a_ks(abuf, t, ks, af[ks]);
    };
    // raw holds the halo of the chunk after the current one: stored to LDS
    // early in the current chunk, then reloaded with the chunk after that.
    u32x4 raw[PP];
    load_halo(0, raw);
    load_w(0, wq[0]);
    load_w(min(1, nsteps - 1), wq[1]);
#pragma unroll
    for (int i = 0; i < PP; ++i) store_piece(0, sA, raw[i], i);
    load_halo(min(1, nchunks - 1), raw);
    __syncthreads();

    for (int k = 0; k < nchunks; ++k) {
        const uint16_t *a_cur = sA + (k & 1) * A_ELEMS;
        uint16_t *a_next = sA + ((k + 1) & 1) * A_ELEMS;
        // raw holds chunk kn's halo and is reloaded with chunk kl's at tap 4
        // (past the end the last chunk is reloaded and stored again, to the
        // buffer no one reads any more: harmless).
        const int kn = min(k + 1, nchunks - 1);
        const int kl = min(k + 2, nchunks - 1);
        // A fragments of tap 0; later taps' are read one tap ahead.
        read_a(a_cur, 0, afr[0]);
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const int s = k * 9 + t;
            // slots rotate with t; 9 is a multiple of 3, so slot = t % 3.
            // Past the last step the last step's weights are reloaded.
            load_w(min(s + 2, nsteps - 1), wq[(t + 2) % 3]);
            if constexpr (ASETS == 2) {
                if (t < 8) read_a(a_cur, t + 1, afr[(t + 1) & 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 (&af)[MI] = afr[ASETS == 2 ? (t & 1) : 0][ks];
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            af[mi], wq[t % 3][ks][ni], acc[mi][ni], 0, 0, 0);
                if constexpr (ASETS == 1) {
                    if (t < 8) read_a_ks(a_cur, t + 1, ks, af);
                }
            }
            // the next chunk's pieces are normalised and stored early, at
            // taps 1-3 (three pieces) or 1-2 (two), which frees raw for the
            // reload at tap 4
            if constexpr (PP == 3) {
                if (t >= 1 && t <= 3) store_piece(kn, a_next, raw[t - 1], t - 1);
            } else {
                if (t >= 1 && t <= 2) store_piece(kn, a_next, raw[t - 1], t - 1);
            }
            if (t == 4) {
                load_halo(kl, raw);
                // Keep the loads where they are issued: left to itself the
                // scheduler sinks them next to their first use to save
                // registers, which turns the prefetch into a stall.
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();  // a_next written by all lanes; a_cur no longer read
    }

    // ---- epilogue, 64 output channels at a time
    const int q = tid & 7;          // 8-channel piece of the pass
    const int prow = tid >> 3;      // pixels prow + ROWS * i
    float vals[PIX][8];
    bool valid[PIX];
    int cnt = 0;                    // valid pixels of the tile
    {
        const int rows = min(TH, a.H - h0), cols = min(TW, a.W - w0);
        cnt = rows * cols;
    }
    const int Cg2 = STATS ? a.Co / a.G2 : 1;
    for (int half = 0; half < WN; ++half) {  // passes of 64 channels
        if (wn == half) {
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int cl = ni * 32 + fp;  // channel within the half
                    const float bv = bias_v[ni];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        const int pix = wm * 32 * MI + mi * 32 + m;
                        sO[pix * OS + cl] = acc[mi][ni][r] + bv;
                    }
                }
        }
        __syncthreads();
        // Output offsets of the lane's pixels; with a residual, all of its
        // values are loaded before the first store of z (waiting for a load
        // also waits for every older store, one counter covering both), and
        // before any z of the half is written, so res may alias z. A tile
        // with every pixel inside the image takes a copy of this code with
        // no per-pixel branch: a load or store inside one makes the compiler
        // wait for all outstanding memory operations at each store.
        int64_t offs[PIX];
        u32x4 rr[PIX];
        auto emit = [&](auto checked) {
            constexpr bool CHECK = decltype(checked)::value;
#pragma unroll
            for (int i = 0; i < PIX; ++i) {
                const int pix = prow + ROWS * i;
                const int oh = h0 + pix / TW, ow = w0 + pix % TW;
                valid[i] = !CHECK || (oh < a.H && ow < a.W);
                offs[i] = ((static_cast<int64_t>(n) * a.H + oh) * a.W + ow) * a.Co + co0 +
                          half * 64 + 8 * q;
                if constexpr (RES) {
                    if (!CHECK || valid[i]) rr[i] = *reinterpret_cast<const u32x4 *>(a.res + offs[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < PIX; ++i) {
                const int pix = prow + ROWS * i;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = sO[pix * OS + 8 * q + e];
                if (!CHECK || valid[i]) {
                    if constexpr (RES) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[2 * e] += bf16_to_f32(rr[i][e] & 0xffffu);
                            v[2 * e + 1] += bf16_to_f32(rr[i][e] >> 16);
                        }
                    }
                    u32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        o[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
                        // the stored (rounded) values, for the statistics
                        vals[i][2 * e] = bf16_to_f32(o[e] & 0xffffu);
                        vals[i][2 * e + 1] = bf16_to_f32(o[e] >> 16);
                    }
                    *reinterpret_cast<u32x4 *>(a.z + offs[i]) = o;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) vals[i][e] = 0.0f;
                }
            }
        };
        if (cnt == BM)
            emit(std::false_type{});
        else
            emit(std::true_type{});
        if constexpr (!STATS) {
            __syncthreads();  // sO fully read: free for the next half
        } else {
            // Per output group of the pass (Cg2 channels: a run of the lane's
            // 8 when Cg2 < 8, else Cg2/8 consecutive pieces), sums in a fixed
            // order: per lane over its valid pixels; within the lane over the
            // group's channels (pairs, then pairs of pairs); an xor butterfly
            // over the lanes of the wave holding the same piece (lane bits
            // 3-5) and, for Cg2 > 8, over the group's pieces (lane bits 0-2);
            // then the four waves' sums in wave order.  Every step adds two
            // equal-ranked operands in either order, so all lanes and
            // channels of a group hold the same bits, and every lane forms the
            // group's mean itself.
            static_assert(NT == 256, "four waves in the statistics");
            const int wave = tid >> 6;
            const float count = static_cast<float>(cnt * Cg2);
            auto reduce = [&](float (&t)[8]) {
                if (Cg2 >= 8) {
                    float v = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
#pragma unroll
                    for (int m = 8; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
#pragma unroll
                    for (int m = 1; m < 8; m <<= 1)
                        if (8 * m < Cg2) v += __shfl_xor(v, m, 64);  // uniform
#pragma unroll
                    for (int e = 0; e < 8; ++e) t[e] = v;
                } else {
                    if (Cg2 >= 2) {
#pragma unroll
                        for (int e = 0; e < 8; e += 2) t[e] = t[e + 1] = t[e] + t[e + 1];
                    }
                    if (Cg2 >= 4) {
#pragma unroll
                        for (int h = 0; h < 8; h += 4)
#pragma unroll
                            for (int e = h; e < h + 2; ++e) t[e] = t[e + 2] = t[e] + t[e + 2];
                    }
#pragma unroll
                    for (int m = 8; m < 64; m <<= 1)
#pragma unroll
                        for (int e = 0; e < 8; ++e) t[e] += __shfl_xor(t[e], m, 64);
                }
            };
            auto publish = [&](float *dst, const float (&t)[8]) {
                if (lane < 8) {  // the wave's first row: q == lane
                    *reinterpret_cast<float4 *>(dst + wave * 64 + 8 * q) =
                        make_float4(t[0], t[1], t[2], t[3]);
                    *reinterpret_cast<float4 *>(dst + wave * 64 + 8 * q + 4) =
                        make_float4(t[4], t[5], t[6], t[7]);
                }
            };
            auto wave_sum = [](const float *src, int c) {
                return ((src[c] + src[64 + c]) + src[128 + c]) + src[192 + c];
            };
            float t8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = 0.0f;
#pragma unroll
                for (int i = 0; i < PIX; ++i) v += valid[i] ? vals[i][e] : 0.0f;
                t8[e] = v;
            }
            reduce(t8);
            publish(s_stat, t8);
            __syncthreads();
            float mg[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) mg[e] = wave_sum(s_stat, 8 * q + e) / count;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = 0.0f;
#pragma unroll
                for (int i = 0; i < PIX; ++i) {
                    const float d = vals[i][e] - mg[e];
                    v = valid[i] ? fmaf(d, d, v) : v;
                }
                t8[e] = v;
            }
            reduce(t8);
            publish(s_stat + 256, t8);
            __syncthreads();
            const int ngroups = 64 / Cg2;
            if (tid < ngroups) {
                const int c0 = tid * Cg2;
                const int g2 = (co0 + half * 64) / Cg2 + tid;
                float *dst = a.part + ((static_cast<int64_t>(n) * tiles_per_sample + tin) *
                                           a.G2 + g2) * 4;
                dst[0] = count;
                dst[1] = wave_sum(s_stat, c0) / count;
                dst[2] = wave_sum(s_stat + 256, c0);
                dst[3] = 0.0f;
            }
            __syncthreads();  // sO and s_stat free for the next half
        }
    }
}

// Packs [Co][3][3][Ci] bf16 weights into the fragment order above: one lane
// per 16-byte piece of the packed array.
__global__ __launch_bounds__(kThreads) void gn_conv_pack_weights(const uint16_t *__restrict__ wt,
                                                                 uint16_t *__restrict__ packed,
                                                                 int Ci, int64_t pieces) {
    const int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (v >= pieces) return;
    // v = ((((cb * nsteps + step) * 2 + ks) * 2 + wn) * 2 + ni) * 64 + lane
    const int lane = static_cast<int>(v & 63);
    int64_t r = v >> 6;
    const int ni = static_cast<int>(r & 1);
    r >>= 1;
    const int wn = static_cast<int>(r & 1);
    r >>= 1;
    const int ks = static_cast<int>(r & 1);
    r >>= 1;
    const int nsteps = (Ci / BK) * 9;
    const int step = static_cast<int>(r % nsteps);
    const int64_t cb = r / nsteps;
    const int k = step / 9, t = step % 9;
    const int64_t co = cb * BN + wn * 64 + ni * 32 + (lane & 31);
    const int ci = k * BK + ks * 16 + 8 * (lane >> 5);
    *reinterpret_cast<u32x4 *>(packed + v * 8) =
        *reinterpret_cast<const u32x4 *>(wt + (co * 9 + t) * Ci + ci);
}

// Merge of the per-tile (count, mean, M2) of each (n, group) into fp32 mean
// and rstd, in fp64.  Merged, the group's sum of squared deviations is
// sum_t [M2_t + c_t (m_t - mean)^2]; written about a pivot p (tile 0's mean)
// with d_t = m_t - p, S0 = sum c_t, S1 = sum c_t d_t and
// S2 = sum (M2_t + c_t d_t^2), it is S2 - S1^2 / S0 and mean = p + S1 / S0.
// The pivot keeps that subtraction small when the group's mean is large
// against its spread (the tiles' means then lie close to p).  One pass over
// the records: thread j adds tiles j, j + 256, ... in increasing order, an xor
// butterfly sums each wave (every lane ends with the same bits) and thread 0
// adds the four wave sums in order -- a fixed order, so the statistics are
// reproducible bit for bit.
__global__ __launch_bounds__(kThreads) void gn_conv_stats_finalize(const float *part, int tiles,
                                                                   int G2, float eps, float *mean,
                                                                   float *rstd) {
    __shared__ double w0[kThreads / 64], w1[kThreads / 64], w2[kThreads / 64];
    const int ng = blockIdx.x;
    const int n = ng / G2, g = ng % G2;
    const int tid = threadIdx.x;
    const float *base = part + (static_cast<int64_t>(n) * tiles * G2 + g) * 4;
    const double p = base[1];
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
#pragma unroll 4
    for (int t = tid; t < tiles; t += kThreads) {
        const float4 r = *reinterpret_cast<const float4 *>(base + static_cast<int64_t>(t) * G2 * 4);
        const double c = r.x;
        const double d = static_cast<double>(r.y) - p;
        const double cd = c * d;
        s0 += c;
        s1 += cd;
        s2 += static_cast<double>(r.z) + cd * d;
    }
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
        s0 += __shfl_xor(s0, m, 64);
        s1 += __shfl_xor(s1, m, 64);
        s2 += __shfl_xor(s2, m, 64);
    }
    if ((tid & 63) == 0) {
        w0[tid >> 6] = s0;
        w1[tid >> 6] = s1;
        w2[tid >> 6] = s2;
    }
    __syncthreads();
    if (tid == 0) {
        double t0 = 0.0, t1 = 0.0, t2 = 0.0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) {
            t0 += w0[w];
            t1 += w1[w];
            t2 += w2[w];
        }
        const double dm = t1 / t0;  // t0 >= 1: every tile holds a pixel
        const double m2 = t2 - t1 * dm;
        const double var = m2 > 0.0 ? m2 / t0 : 0.0;
        mean[ng] = static_cast<float>(p + dm);
        rstd[ng] = static_cast<float>(1.0 / sqrt(var + static_cast<double>(eps)));
    }
}

}  // namespace gnconv
