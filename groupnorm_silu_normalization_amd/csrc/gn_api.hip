// gn_api.hip -- host side of libgnsilu.so: argument checks, the launch plan,
// the per-(device, stream) scratch buffer and the C-ABI entry points declared
// in include/gnsilu.h.
//
// The contract follows "FLUX.2 VAE decoder fast path behind quality=high",
// Modifications section 1 "Kernel": group_norm_silu_4d / group_norm_silu_rows
// return a result, or decline inputs outside the supported set so that the
// caller falls back; here "decline" is the status GN_UNSUPPORTED.  The
// pages' kernel declines C that is not a power of two and C > 2048; this
// library takes any C for which a tile layout exists (choose_layout below),
// which covers every C <= 2048 that is a multiple of 8 and 16-bit C up to
// 8192 that is a multiple of 32, and it also takes 5-D NDHWC activations
// through the rows form.  A layout that is not channels-last is still
// declined.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "gn_conv.hpp"
#include "gn_kernels.hpp"
#include "gnsilu.h"

// The scratch of gn_silu_rows_noalloc: one fixed buffer per device, part of
// the library's code object (allocated by the runtime when the code is loaded
// on a device, held until the process ends).  In host code this name is only
// a stand-in for the symbol; the device address of each device's copy comes
// from hipGetSymbolAddress (fixed_scratch below) and is the only form of it
// that host code passes on.
static __device__ __align__(256) char scratch[GN_NOALLOC_SCRATCH_BYTES];

namespace gnsilu {
namespace {

// Launch plan constants, measured on MI355X (256 CUs, 256 MB Infinity Cache)
// over the full three-step sequence at the decoder shapes.
constexpr int kUnrollStats = 8;             // 16-byte loads in flight per lane, step 1
constexpr int kUnrollApply = 4;             // 16-byte loads in flight per lane, step 3 ...
constexpr int kUnrollApplyDeep = 8;         // ... or twice that (Plan::apply_deep)
constexpr int64_t kStatsBlocks = 256;       // step-1 workgroups in total: one per CU ...
constexpr int64_t kStatsBlocksSmall = 128;  // ... or half that for x up to kStatsSmallBytes,
constexpr int64_t kStatsSmallBytes = int64_t{16} << 20;  // where latency, not bandwidth, rules
constexpr int64_t kSepFinalizeMaxBytes = int64_t{160} << 20;  // step 2 as its own kernel above
                                                              // kStatsSmallBytes up to this
constexpr int64_t kStatsMinTiles = 8;       // tiles per workgroup, at least
constexpr int64_t kStatsMaxTiles = 1024;    // caps each lane's sequential fp32 run
constexpr int64_t kApplyElemsPerBlock = 16 * 2048;  // step-3 workgroups: elements / 32768 ...
constexpr int64_t kApplyMinBlocks = 256;    // ... clamped to [256, 2048]
constexpr int64_t kApplyMaxBlocks = 2048;
// Step 1 reads the last cache's worth of x with ordinary loads (the rest with
// nontemporal ones), so that part of x is still in the 256 MB Infinity Cache
// when step 3 reads it again; step 3 writes y with nontemporal stores so y
// does not evict it.  A tensor larger than the cache cannot be served from it
// whole, and step 3 then streams x with nontemporal loads.
constexpr int64_t kCacheResidentBytes = int64_t{256} << 20;
// The single launch (gn_strip), measured on MI355X against the three-step
// path over N in {1..16}, L in {256..4096}, C in {128, 256, 512}: 10-30%
// faster with at most one workgroup per CU, at most kStripPieces pieces per
// lane and up to 4 MiB; slower beyond (a second round of workgroups: up to
// 4x; four pieces per lane: 2-20%; the (1,128,64,64) decoder shape is one of
// those, 2% slower).
constexpr int64_t kStripMaxBytes = int64_t{4} << 20;
constexpr int64_t kStripMaxBlocks = 256;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t gcd64(int64_t a, int64_t b) {
    while (b != 0) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The dtype argument: a gn_dtype for x and y in the low bits, or-ed with at
// most one GN_AFFINE_* value for gamma and beta (none: fp32).
inline int x_dtype(int dtype) { return dtype & ~GN_AFFINE_MASK; }
inline bool valid_dtype(int dtype) {
    const int xd = x_dtype(dtype), ad = dtype & GN_AFFINE_MASK;
    return (xd == GN_DTYPE_BF16 || xd == GN_DTYPE_F16 || xd == GN_DTYPE_F32) &&
           (ad == 0 || ad == GN_AFFINE_F32 || ad == GN_AFFINE_BF16 || ad == GN_AFFINE_F16);
}
inline int affine_type(int dtype) {
    switch (dtype & GN_AFFINE_MASK) {
        case GN_AFFINE_BF16: return Affine::kBf16;
        case GN_AFFINE_F16: return Affine::kF16;
        default: return Affine::kF32;
    }
}
inline int64_t elem_bytes(int dtype) { return x_dtype(dtype) == GN_DTYPE_F32 ? 4 : 2; }

// How a tile is laid over the lanes (see gn_kernels.hpp): R whole rows,
// T = R*C = A*W*NV elements; the first A lanes each make NV accesses of W
// consecutive elements.
struct Layout {
    int w;      // elements per access: a 16-byte access (8 of a 16-bit type, 4 fp32), or 1
    int nv;     // accesses per lane and tile: 1, 2 or 4
    int a;      // active lanes, <= kThreads
    int64_t t;  // elements per tile
};

// The tile layout for a sample of E = L*C elements.  16-byte accesses need
// every sample to start on a 16-byte boundary, i.e. E a multiple of W;
// otherwise W = 1.  A tile must be a whole number of rows, so C must divide
// A*W*NV: A is the largest multiple of m = C / gcd(C, W*NV) not above
// kThreads.  The smallest NV keeping at least half of the lanes busy is taken,
// else the NV with the most active lanes: measured on MI355X, fewer accesses
// per lane beat more active lanes (C = 1280: NV = 1 with 160 lanes runs the
// path 8% faster than NV = 2 with 240; C = 2560: NV = 2 with 160 lanes 22%
// faster than NV = 4 with 240), because each extra access costs 2*W*NV
// registers of scale/shift and sums per lane, and with them occupancy and
// loads in flight.  fp32 starts at NV = 2 so that a lane moves 32 bytes per
// tile, as a 16-bit lane moves 16.  No NV with m <= kThreads: no layout, and
// the shape is declined.
bool choose_layout(int64_t E, int64_t C, int dtype, Layout *out) {
    const int w16 = static_cast<int>(16 / elem_bytes(dtype));
    const int w = (E % w16 == 0) ? w16 : 1;
    const int nv_min = (w == 4) ? 2 : 1;
    bool found = false;
    for (int nv = nv_min; nv <= 4; nv *= 2) {
        const int64_t m = C / gcd64(C, static_cast<int64_t>(w) * nv);
        if (m > kThreads) continue;
        const int a = static_cast<int>((kThreads / m) * m);
        if (!found || a > out->a) {
            *out = Layout{w, nv, a, static_cast<int64_t>(a) * w * nv};
            found = true;
        }
        if (2 * out->a >= kThreads) break;
    }
    return found;
}

// Channel counts whose 256-lane layout leaves a quarter or more of the lanes
// idle or needs more than the minimal accesses per lane (C = 1280, 2560:
// 2560 = 5*512, so no 256-lane tile of whole rows keeps every lane busy) run
// in workgroups of kWideThreads = 320 lanes (five waves) when those are all
// busy with the minimal accesses: one row of 2560 or two of 1280 per tile.
constexpr int kWideThreads = 320;
bool choose_wide_layout(int64_t C, const Layout &lay, Layout *out) {
    const int nv_min = (lay.w == 4) ? 2 : 1;
    if (lay.w == 1) return false;                                     // 1-element accesses
    if (lay.nv == nv_min && 4 * lay.a >= 3 * kThreads) return false;  // >= 75% busy already
    const int64_t m = C / gcd64(C, static_cast<int64_t>(lay.w) * nv_min);
    if (kWideThreads % m != 0) return false;
    *out = Layout{lay.w, nv_min, kWideThreads,
                  static_cast<int64_t>(kWideThreads) * lay.w * nv_min};
    return true;
}

struct Plan {
    Layout lay;       // tile layout of all three steps
    int threads;      // lanes per workgroup of steps 1 and 3: kThreads or kWideThreads
    bool fused;       // step 2 runs in the tail of step 1 (G <= kThreads)
    bool late;        // ... or, for a small x, in the prologue of step 3 (LateStats)
    bool apply_ntl;   // step 3 reads x with nontemporal loads
    bool apply_deep;  // step 3 keeps kUnrollApplyDeep loads in flight, not kUnrollApply
    int dtype;        // gn_dtype of x and y
    int affine;       // element type of gamma and beta (Affine::kF32, ...)
    Geometry stats;   // chunking of steps 1 and 2
    Geometry apply;   // chunking of step 3
    int64_t N;
    double inv_m;     // 1 / (L*Cg)
    bool strip;       // steps 1-3 in one launch (gn_strip), no scratch
    int strip_sub;    // SUB of gn_strip: min(Cg, W)
    StripGeo sg;
};

// The single launch: one workgroup per strip of gpw whole, consecutive groups
// of a sample.  Needs 16-byte rows (C*esize % 16 == 0) and groups that split
// into 16-byte pieces or fill them exactly: Cg a multiple of W (gpw = 1,
// P = Cg/W pieces per row, a power of two <= 64) or a divisor of W (gpw =
// W/Cg groups per piece, P = 1).
bool choose_strip(int64_t N, int64_t L, int64_t C, int64_t G, int dtype, StripGeo *sg, int *sub) {
    const int64_t es = elem_bytes(dtype);
    const int64_t W = 16 / es;
    if ((C * es) % 16 != 0) return false;
    const int64_t Cg = C / G;
    int64_t gpw;
    if (Cg >= W) {
        if (Cg % W != 0) return false;
        gpw = 1;
        *sub = static_cast<int>(W);
    } else {
        if (W % Cg != 0) return false;
        gpw = W / Cg;
        if (G % gpw != 0) return false;
        *sub = static_cast<int>(Cg);
    }
    const int64_t P = gpw * Cg / W;
    if (P > 64 || (P & (P - 1)) != 0) return false;
    if (N * L * C * es > kStripMaxBytes) return false;
    if (N * (G / gpw) > kStripMaxBlocks) return false;
    if (ceil_div(L, kStripThreads / P) > kStripPieces) return false;
    sg->L = L;
    sg->E = L * C;
    sg->C = static_cast<int>(C);
    sg->G = static_cast<int>(G);
    sg->Cg = static_cast<int>(Cg);
    sg->gpw = static_cast<int>(gpw);
    sg->P = static_cast<int>(P);
    sg->S = static_cast<int>(G / gpw);
    sg->blocks = N * sg->S;
    sg->xcd = (sg->blocks % 8 == 0) ? 1 : 0;
    sg->inv_m = 1.0 / (static_cast<double>(L) * static_cast<double>(Cg));
    sg->eps = 0.0f;
    return true;
}

// The plan depends on the shape only, never on the device, so the order of
// every floating-point reduction is fixed by (N, L, C, G).
Plan make_plan(int64_t N, int64_t L, int64_t C, int64_t G, int dtype) {
    Plan p;
    p.N = N;
    p.dtype = x_dtype(dtype);
    p.affine = affine_type(dtype);
    const int64_t E = L * C;
    (void)choose_layout(E, C, dtype, &p.lay);  // check_shape has accepted the shape
    // Beyond the latency-bound sizes (where the late finalize, laid out for 256
    // threads, may run), both passes take the 320-lane layout where it keeps
    // every lane busy and the 256-lane one does not.
    p.threads = kThreads;
    if (N * E * elem_bytes(dtype) > kStatsSmallBytes) {
        Layout wide;
        if (choose_wide_layout(C, p.lay, &wide)) {
            p.lay = wide;
            p.threads = kWideThreads;
        }
    }
    // Step 2 runs in the tail of step 1 (the last workgroup of each sample)
    // when one workgroup's threads cover the groups, except from 16 to 160 MiB,
    // where the separate finalize kernel is faster: measured on MI355X, the
    // last workgroup's chain (write-through partials, arrival, coherent reads)
    // costs more there than a third launch (64 MiB: 40.2 -> 39.5 us, 32 MiB:
    // 25.8 -> 25.2 us, 80-160 MiB: 0.4-0.7 us less); from 256 MiB up the two
    // are within noise.
    const int64_t xbytes = N * E * elem_bytes(dtype);
    p.fused = G <= kThreads && !(xbytes > kStatsSmallBytes && xbytes <= kSepFinalizeMaxBytes);
    p.apply_ntl = N * E * elem_bytes(dtype) > kCacheResidentBytes;
    Geometry g;
    g.E = E;
    g.T = p.lay.t;
    g.tiles = ceil_div(E, g.T);
    g.full = E / g.T;
    g.C = static_cast<int>(C);
    g.G = static_cast<int>(G);
    g.Cg = static_cast<int>(C / G);
    g.A = p.lay.a;
    g.cg_shift = 0;
    while ((int64_t{1} << g.cg_shift) < C / G) ++g.cg_shift;
    if (p.lay.a != kThreads) g.cg_shift = 0;  // only the power-of-two kernels use it
    g.plain_tail = 0;
    g.rem = 0;
    const int64_t total = N * g.tiles;
    const int64_t bytes = N * E * elem_bytes(dtype);
    p.stats = g;
    // Step 1 on a small x is a chain of latencies (load batch, LDS reduction,
    // write-through partials, arrival atomic, finalize), and every extra
    // workgroup adds an arrival on the same counter line: measured on MI355X
    // (bf16, stats kernel alone), 0.5-16 MiB shapes take 9.1-12.0 us with at
    // least 8 tiles per workgroup and at most 128 workgroups, against
    // 9.9-13.3 us with 256 workgroups of fewer tiles; from 64 MiB up, 256
    // workgroups are 1-30% faster than 128.
    const int64_t blocks = bytes <= kStatsSmallBytes ? kStatsBlocksSmall : kStatsBlocks;
    p.stats.tpc = std::min(kStatsMaxTiles,
                           std::max(kStatsMinTiles, ceil_div(total, blocks)));
    p.stats.K = ceil_div(g.tiles, p.stats.tpc);
    // Step 1's plain-load tail: the fraction cache / tensor of every chunk (all
    // of it when the tensor fits), so about one cache's worth of x is read
    // last with allocating loads.  Measured on MI355X over the whole path:
    // 512 MiB bf16 -1.7%, 1 GiB -3.7%; a smaller plain fraction slows step 3
    // by more than it saves in step 1.
    p.stats.plain_tail =
        bytes <= kCacheResidentBytes
            ? p.stats.tpc
            : std::max<int64_t>(1, ceil_div(p.stats.tpc * kCacheResidentBytes, bytes));
    p.apply = g;
    // Step 3: about one workgroup per 32768 elements, between 256 and 2048,
    // rounded to whole rounds of 256 (one workgroup on every CU of an MI355X
    // per round) and the tiles split evenly (the first tiles % K chunks take
    // one more), so every CU ends its last round with the same work.
    // Measured on MI355X against the previous rule (whole-tile chunks of
    // ceil(total / blocks) tiles, e.g. 1821 workgroups at (1,960,256,256)):
    // y bitwise the same (the chunking of step 3 changes no arithmetic).
    int64_t apply_blocks = std::min(
        kApplyMaxBlocks, std::max(kApplyMinBlocks, total * g.T / kApplyElemsPerBlock));
    apply_blocks = (apply_blocks + kApplyMinBlocks / 2) / kApplyMinBlocks * kApplyMinBlocks;
    p.apply.K = std::max<int64_t>(1, std::min(g.tiles, ceil_div(apply_blocks, N)));
    p.apply.tpc = g.tiles / p.apply.K;
    p.apply.rem = g.tiles - p.apply.tpc * p.apply.K;
    // Step 3 keeps twice the loads in flight where every workgroup's tiles
    // make whole batches of the deeper unroll (at least two, no uneven
    // split) and x is at most kSepFinalizeMaxBytes.  Measured on MI355X
    // against four in flight (one process, best of four alternating rounds,
    // y bitwise the same): 16 MiB -4%, 32 MiB -2.2%, 64 MiB -1.3%,
    // (1,65536,1280) -3.4%, 128 MiB -0.6%; with a part-filled last batch it
    // loses (1-2% at 1-4 MiB, 9% at (1,16384,2560), 12-13 tiles per
    // workgroup), and from 256 MiB up it is within +-1% (the 512 MiB
    // headline +0.9%), so those keep four.
    static_assert(kSepFinalizeMaxBytes <= kCacheResidentBytes,
                  "the deeper step 3 never takes nontemporal loads");
    const int64_t deep = kUnrollApplyDeep;
    p.apply_deep = bytes <= kSepFinalizeMaxBytes && p.apply.rem == 0 &&
                   p.apply.tpc >= 2 * deep && p.apply.tpc % deep == 0;
    p.inv_m = 1.0 / (static_cast<double>(L) * static_cast<double>(C / G));
    // The late finalize: for a small x (latency-bound) whose sample's step-1
    // partials one finalize batch per thread covers, step 1 only writes its
    // partials and every step-3 workgroup reduces them itself: the arrival
    // count and the last workgroup's round trips leave the chain.  Bounded to
    // small x because every step-3 workgroup re-reads the sample's partials.
    p.late = p.fused && bytes <= kStatsSmallBytes &&
             p.stats.K <= kFinalizeBatch * (kThreads / G);
    p.strip = choose_strip(N, L, C, G, dtype, &p.sg, &p.strip_sub);
    return p;
}

size_t partial_floats(const Plan &p) {
    return static_cast<size_t>(p.N) * p.stats.K * p.stats.G;
}

// Scratch bytes of a call: the arrival counter words (arrival_stride(K1) per
// sample, at the front, 256-byte aligned), the partial sums, the partial squares, the finalize's
// over-read padding, and -- for the full path -- mean and rstd.  The padding
// sits right after the partial squares, so a finalize batch that reads past
// them never touches mean/rstd while another sample writes them.
int64_t arrival_words(const Plan &p) { return p.N * arrival_stride(p.stats.K); }
size_t arrivals_bytes(int64_t words) { return align_up(static_cast<size_t>(words) * 4, 256); }
size_t payload_bytes(const Plan &p, bool with_stats) {
    return sizeof(float) * (2 * partial_floats(p) + static_cast<size_t>(kFinalizeOverread) +
                            (with_stats ? 2 * static_cast<size_t>(p.N) * p.stats.G : 0));
}

// Checks with no HIP call.  INVALID before UNSUPPORTED.
gn_status check_shape(const void *x, const void *y, int64_t N, int64_t L, int64_t C, int64_t G,
                      float eps, int apply_silu, bool need_y, int dtype) {
    if (!valid_dtype(dtype)) return GN_INVALID_ARGUMENT;
    if (x == nullptr || (need_y && y == nullptr)) return GN_INVALID_ARGUMENT;
    if (N < 0 || L < 0 || C <= 0 || G <= 0 || C % G != 0) return GN_INVALID_ARGUMENT;
    if (!(eps >= 0.0f) || std::isinf(eps)) return GN_INVALID_ARGUMENT;
    if (apply_silu != 0 && apply_silu != 1) return GN_INVALID_ARGUMENT;
    if (L > 0 && N > INT64_MAX / L) return GN_INVALID_ARGUMENT;
    if (N * L > 0 && C > INT64_MAX / (N * L) / 4) return GN_INVALID_ARGUMENT;
    if (C > GN_MAX_CHANNELS) return GN_UNSUPPORTED;
    Layout lay;
    if (!choose_layout(L * C, C, dtype, &lay)) return GN_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(x) & 15u) != 0) return GN_UNSUPPORTED;
    if (need_y && (reinterpret_cast<uintptr_t>(y) & 15u) != 0) return GN_UNSUPPORTED;
    // Grid extents: a dispatch holds at most 2^32 work-items, i.e. 2^24
    // workgroups of 256.  Step 3 launches at most kApplyMaxBlocks + N
    // workgroups, step 1 at most total tiles / kStatsMaxTiles + N (+256), the
    // separate finalize N*G.
    if (N > (int64_t{1} << 24) - 2 * kApplyMaxBlocks || N * G >= (int64_t{1} << 24))
        return GN_UNSUPPORTED;
    if (L > 0 && N * ceil_div(L * C, lay.t) / kStatsMaxTiles > (int64_t{1} << 23))
        return GN_UNSUPPORTED;
    return GN_OK;
}

// Restores the caller's current device on scope exit.
struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    gn_status enter(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) return GN_DEVICE_ERROR;
        if (prev != dev) {
            if (hipSetDevice(dev) != hipSuccess) return GN_DEVICE_ERROR;
            changed = true;
        }
        return GN_OK;
    }
    ~DeviceGuard() {
        if (changed) (void)hipSetDevice(prev);
    }
};

gn_status stream_device(hipStream_t s, int *dev) {
    if (s == nullptr) return hipGetDevice(dev) == hipSuccess ? GN_OK : GN_DEVICE_ERROR;
    hipDevice_t d;
    if (hipStreamGetDevice(s, &d) != hipSuccess) {
        (void)hipGetLastError();
        return GN_INVALID_ARGUMENT;
    }
    *dev = static_cast<int>(d);
    return GN_OK;
}

// A pointer the kernels may dereference: device (or managed) memory on `dev`.
bool on_device(const void *ptr, int dev) {
    if (ptr == nullptr) return true;  // optional argument absent
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, ptr) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged) return false;
    return a.device == dev;
}

// ---- scratch buffer per (device, stream) ----------------------------------
// Layout: [arrival counters: `arrivals` uint32 words, zero between calls][payload].
// The counter region only grows, so a payload never overlaps a counter.
struct Scratch {
    char *ptr = nullptr;
    size_t bytes = 0;
    int64_t arrivals = 0;
};

std::mutex &scratch_mutex() {
    static std::mutex *m = new std::mutex;  // never destroyed: outlives atexit teardown
    return *m;
}
std::map<std::pair<int, uintptr_t>, Scratch> &scratch_map() {
    static auto *m = new std::map<std::pair<int, uintptr_t>, Scratch>;
    return *m;
}

gn_status zero_counters(unsigned *p, int64_t n, hipStream_t s) {
    if (n <= 0) return GN_OK;
    gn_zero_u32<<<static_cast<unsigned>(ceil_div(n, kThreads)), kThreads, 0, s>>>(p, n);
    return hipGetLastError() == hipSuccess ? GN_OK : GN_DEVICE_ERROR;
}

// Buffers a stream has outgrown.  They are never freed: work already
// enqueued, and HIP graphs captured with calls of this library, keep their
// addresses and may run (or be replayed) at any later time.  Growth doubles,
// so the retired buffers of a stream total less than its current one.
std::vector<void *> &retired_scratch() {
    static auto *v = new std::vector<void *>;
    return *v;
}

// Caller holds scratch_mutex().  Returns the arrival counter words (>= n of
// them, all zero in stream order) and the payload (>= payload bytes).  Grows the
// buffer when needed; the old one is retired, not freed.
gn_status scratch_for(int dev, hipStream_t s, int64_t n, size_t payload, unsigned **counters,
                      char **payload_ptr) {
    Scratch &sc = scratch_map()[{dev, reinterpret_cast<uintptr_t>(s)}];
    const int64_t want_arrivals = std::max(sc.arrivals, n);
    const size_t head = arrivals_bytes(want_arrivals);
    const size_t need = head + payload;
    bool clear = want_arrivals > sc.arrivals;  // the counter region grows
    if (sc.bytes < need) {
        size_t sz = size_t{1} << 16;
        while (sz < need) sz <<= 1;
        void *p = nullptr;
        if (hipMalloc(&p, sz) != hipSuccess) {
            (void)hipGetLastError();
            return GN_DEVICE_ERROR;
        }
        if (sc.ptr != nullptr) retired_scratch().push_back(sc.ptr);
        sc.ptr = static_cast<char *>(p);
        sc.bytes = sz;
        clear = true;  // fresh memory
    }
    if (clear) {
        // Counters beyond the old region may hold stale payload bytes: clear
        // the region, in stream order, before this call's kernels.
        const gn_status st =
            zero_counters(reinterpret_cast<unsigned *>(sc.ptr), want_arrivals, s);
        if (st != GN_OK) return st;
    }
    sc.arrivals = want_arrivals;
    *counters = reinterpret_cast<unsigned *>(sc.ptr);
    *payload_ptr = sc.ptr + head;
    return GN_OK;
}

// ---- launches ---------------------------------------------------------------
// Kernel slots, as reported by gn_profile_rows / gn_kernel_name.
enum { kSlotStats = 0, kSlotFinalize = 1, kSlotApply = 2, kSlotStrip = 3, kSlots = 4 };
const char *kKernelNames[kSlots] = {"gn_partial_stats", "gn_finalize_stats", "gn_apply",
                                    "gn_strip"};

struct Events {
    hipEvent_t ev[2 * kSlots];  // start/stop per slot
};

template <int V> using IC = std::integral_constant<int, V>;
template <class T> struct TypeTag {
    using type = T;
};

// Calls f(IC<W>, IC<NV>, IC<POW2>) with a layout as compile-time constants;
// POW2 = all 256 lanes of a 256-lane workgroup busy, which happens exactly
// when C is a power of two.
template <class D, class F>
void with_layout(const Layout &lay, F &&f) {
    constexpr int W16 = static_cast<int>(16 / sizeof(typename D::storage));
    auto by_pow2 = [&](auto wc, auto nvc) {
        if (lay.a == kThreads)
            f(wc, nvc, IC<1>{});
        else
            f(wc, nvc, IC<0>{});
    };
    if (lay.w == 1) {
        switch (lay.nv) {
            case 1: by_pow2(IC<1>{}, IC<1>{}); break;
            case 2: by_pow2(IC<1>{}, IC<2>{}); break;
            default: by_pow2(IC<1>{}, IC<4>{}); break;
        }
    } else {
        switch (lay.nv) {
            case 1:
                if constexpr (W16 != 4) by_pow2(IC<W16>{}, IC<1>{});  // fp32 starts at NV = 2
                break;
            case 2: by_pow2(IC<W16>{}, IC<2>{}); break;
            default: by_pow2(IC<W16>{}, IC<4>{}); break;
        }
    }
}

// Loads in flight per lane: kUnroll* tiles of up to two accesses, half as
// many tiles of four.
constexpr int unroll_for(int base, int nv) { return nv <= 2 ? base : base / 4; }
// Step 3's loads in flight for Plan::apply_deep: deeper only with one 16-byte
// access per lane and tile (two or more would spill or were not measured);
// otherwise the same kernel as without.
constexpr int deep_unroll_for(int nv) {
    return nv == 1 ? kUnrollApplyDeep : unroll_for(kUnrollApply, nv);
}

// late: the plan's late finalize runs in step 3, so step 1 only writes its
// partials (false for a caller that needs mean/rstd from steps 1-2 alone).
template <class D>
void launch_stats_t(const Plan &p, const void *xv, const StatsOut &o, bool late, hipStream_t s,
                    const Events *ev) {
    using T = typename D::storage;
    const T *x = static_cast<const T *>(xv);
    const dim3 block(kThreads);
    const dim3 grid1(static_cast<unsigned>(p.N * p.stats.K));
    if (ev) (void)hipEventRecord(ev->ev[2 * kSlotStats], s);
    if (p.threads == kWideThreads) {
        const dim3 wblock(kWideThreads);
        with_layout<D>(p.lay, [&](auto wc, auto nvc, auto pc) {
            constexpr int W = decltype(wc)::value;
            constexpr int NV = decltype(nvc)::value;
            constexpr bool P2 = decltype(pc)::value != 0;
            if constexpr (W > 1 && NV == (W == 4 ? 2 : 1) && !P2) {
                constexpr int U = unroll_for(kUnrollStats, NV);
                constexpr int NT = kWideThreads;
                if (p.fused && !late)
                    gn_partial_stats<D, W, NV, false, U, true, NT><<<grid1, wblock, 0, s>>>(
                        x, p.stats, o);
                else
                    gn_partial_stats<D, W, NV, false, U, false, NT><<<grid1, wblock, 0, s>>>(
                        x, p.stats, o);
            }
        });
    } else {
        with_layout<D>(p.lay, [&](auto wc, auto nvc, auto pc) {
            constexpr int W = decltype(wc)::value;
            constexpr int NV = decltype(nvc)::value;
            constexpr bool P2 = decltype(pc)::value != 0;
            constexpr int U = unroll_for(kUnrollStats, NV);
            if (p.fused && !late)
                gn_partial_stats<D, W, NV, P2, U, true><<<grid1, block, 0, s>>>(x, p.stats, o);
            else
                gn_partial_stats<D, W, NV, P2, U, false><<<grid1, block, 0, s>>>(x, p.stats,
                                                                                  o);
        });
    }
    if (ev) (void)hipEventRecord(ev->ev[2 * kSlotStats + 1], s);
    if (!p.fused) {  // (late implies fused)
        const dim3 grid2(static_cast<unsigned>(p.N * p.stats.G));
        if (ev) (void)hipEventRecord(ev->ev[2 * kSlotFinalize], s);
        gn_finalize_stats<D><<<grid2, block, 0, s>>>(x, p.stats, o);
        if (ev) (void)hipEventRecord(ev->ev[2 * kSlotFinalize + 1], s);
    }
}

// ls.part_s non-null: the late finalize (the plan's `late`).  Workgroups of
// p.threads lanes: kThreads, or kWideThreads for the wide layout (16-byte
// accesses, minimal NV, never the power-of-two or late kernels).
template <class D, bool SILU>
void launch_apply_s(const Plan &p, const void *xv, void *yv, const float *mean, const float *rstd,
                    const Affine &af, const LateStats &ls, hipStream_t s) {
    using T = typename D::storage;
    const T *x = static_cast<const T *>(xv);
    T *y = static_cast<T *>(yv);
    const dim3 grid(static_cast<unsigned>(p.N * p.apply.K));
    if (p.threads == kWideThreads) {
        const dim3 block(kWideThreads);
        with_layout<D>(p.lay, [&](auto wc, auto nvc, auto pc) {
            constexpr int W = decltype(wc)::value;
            constexpr int NV = decltype(nvc)::value;
            constexpr bool P2 = decltype(pc)::value != 0;
            if constexpr (W > 1 && NV == (W == 4 ? 2 : 1) && !P2) {
                constexpr int U = unroll_for(kUnrollApply, NV);
                constexpr int UD = deep_unroll_for(NV);
                constexpr int NT = kWideThreads;
                if (p.apply_deep)  // never with nontemporal loads (x <= 160 MiB)
                    gn_apply<D, W, NV, false, UD, SILU, false, true, 0, NT>
                        <<<grid, block, 0, s>>>(x, y, p.apply, mean, rstd, af, ls);
                else if (p.apply_ntl)
                    gn_apply<D, W, NV, false, U, SILU, true, true, 0, NT>
                        <<<grid, block, 0, s>>>(x, y, p.apply, mean, rstd, af, ls);
                else
                    gn_apply<D, W, NV, false, U, SILU, false, true, 0, NT>
                        <<<grid, block, 0, s>>>(x, y, p.apply, mean, rstd, af, ls);
            }
        });
        return;
    }
    const dim3 block(kThreads);
    with_layout<D>(p.lay, [&](auto wc, auto nvc, auto pc) {
        constexpr int W = decltype(wc)::value;
        constexpr int NV = decltype(nvc)::value;
        constexpr bool P2 = decltype(pc)::value != 0;
        constexpr int U = unroll_for(kUnrollApply, NV);
        constexpr int UD = deep_unroll_for(NV);
        // The late finalize's batch: the fewest slots (4, 8, 16) covering the
        // sample's chunks -- fewer load instructions, the same adds.
        // Measured on MI355X (per-workgroup timestamps): at (1,128,64,64) the
        // late finalize's partial loads took 3.3 us with 16 slots of which 4
        // were used, 0.55 us less with 4.
        const int tpg = kThreads / p.apply.G;
        const int lb = ls.K1 <= 4 * tpg ? 4 : (ls.K1 <= 8 * tpg ? 8 : 16);
        auto late = [&](auto u) {
            constexpr int UU = decltype(u)::value;
            if (lb == 4)
                gn_apply<D, W, NV, P2, UU, SILU, false, true, 4><<<grid, block, 0, s>>>(
                    x, y, p.apply, mean, rstd, af, ls);
            else if (lb == 8)
                gn_apply<D, W, NV, P2, UU, SILU, false, true, 8><<<grid, block, 0, s>>>(
                    x, y, p.apply, mean, rstd, af, ls);
            else
                gn_apply<D, W, NV, P2, UU, SILU, false, true, 16><<<grid, block, 0, s>>>(
                    x, y, p.apply, mean, rstd, af, ls);
        };
        if (p.apply_deep) {  // never with nontemporal loads (x <= 160 MiB)
            if (ls.part_s != nullptr)
                late(std::integral_constant<int, UD>{});
            else
                gn_apply<D, W, NV, P2, UD, SILU, false, true, 0><<<grid, block, 0, s>>>(
                    x, y, p.apply, mean, rstd, af, ls);
        } else if (p.apply_ntl)
            gn_apply<D, W, NV, P2, U, SILU, true, true, 0><<<grid, block, 0, s>>>(
                x, y, p.apply, mean, rstd, af, ls);
        else if (ls.part_s != nullptr)
            late(std::integral_constant<int, U>{});
        else
            gn_apply<D, W, NV, P2, U, SILU, false, true, 0><<<grid, block, 0, s>>>(
                x, y, p.apply, mean, rstd, af, ls);
    });
}

template <class D>
void launch_apply_t(const Plan &p, const void *x, void *y, const float *mean, const float *rstd,
                    const Affine &af, const LateStats &ls, int silu, hipStream_t s,
                    const Events *ev) {
    if (ev) (void)hipEventRecord(ev->ev[2 * kSlotApply], s);
    if (silu)
        launch_apply_s<D, true>(p, x, y, mean, rstd, af, ls, s);
    else
        launch_apply_s<D, false>(p, x, y, mean, rstd, af, ls, s);
    if (ev) (void)hipEventRecord(ev->ev[2 * kSlotApply + 1], s);
}

void launch_stats(const Plan &p, const void *x, const StatsOut &o, bool late, hipStream_t s,
                  const Events *ev) {
    switch (p.dtype) {
        case GN_DTYPE_F16: launch_stats_t<Fp16>(p, x, o, late, s, ev); break;
        case GN_DTYPE_F32: launch_stats_t<F32>(p, x, o, late, s, ev); break;
        default: launch_stats_t<Bf16>(p, x, o, late, s, ev); break;
    }
}

// late (non-null): step 3 runs the late finalize from these partials; else it
// reads mean/rstd.
// arrivals (non-null): step 1's arrival counters of this call, cleared by
// step 3 (LateStats::arrivals).
void launch_apply(const Plan &p, const void *x, void *y, const float *mean, const float *rstd,
                  const StatsOut *late, const void *gamma, const void *beta, int silu,
                  hipStream_t s, const Events *ev, unsigned *arrivals = nullptr) {
    Affine af;
    af.gamma = gamma;
    af.beta = beta;
    af.type = p.affine;
    LateStats ls{};
    if (late != nullptr) {
        ls.part_s = late->part_s;
        ls.part_q = late->part_q;
        ls.pivot = late->pivot;
        ls.K1 = p.stats.K;
        ls.inv_m = late->inv_m;
        ls.eps = late->eps;
    }
    if (arrivals != nullptr) {
        ls.arrivals = arrivals;
        ls.arrival_words = arrival_stride(p.stats.K);
    }
    switch (p.dtype) {
        case GN_DTYPE_F16: launch_apply_t<Fp16>(p, x, y, mean, rstd, af, ls, silu, s, ev); break;
        case GN_DTYPE_F32: launch_apply_t<F32>(p, x, y, mean, rstd, af, ls, silu, s, ev); break;
        default: launch_apply_t<Bf16>(p, x, y, mean, rstd, af, ls, silu, s, ev); break;
    }
}

// The single launch.  stats_only: steps 1-2 alone, mean/rstd to mo/ro.
template <class D, bool SILU>
void launch_strip_s(const Plan &p, const void *x, void *y, const Affine &af, float eps,
                    int stats_only, float *mo, float *ro, hipStream_t s) {
    using T = typename D::storage;
    constexpr int W = static_cast<int>(16 / sizeof(T));
    StripGeo sg = p.sg;
    sg.eps = eps;
    const dim3 grid(static_cast<unsigned>(sg.blocks)), block(kStripThreads);
    const T *xt = static_cast<const T *>(x);
    T *yt = static_cast<T *>(y);
    auto go = [&](auto subc) {
        constexpr int SUB = decltype(subc)::value;
        if constexpr (W % SUB == 0)
            gn_strip<D, SUB, SILU><<<grid, block, 0, s>>>(xt, yt, sg, af, stats_only, mo, ro);
    };
    switch (p.strip_sub) {
        case 1: go(IC<1>{}); break;
        case 2: go(IC<2>{}); break;
        case 4: go(IC<4>{}); break;
        default: go(IC<8>{}); break;
    }
}

void launch_strip(const Plan &p, const void *x, void *y, const void *gamma, const void *beta,
                  int silu, float eps, int stats_only, float *mo, float *ro, hipStream_t s,
                  const Events *ev) {
    Affine af;
    af.gamma = gamma;
    af.beta = beta;
    af.type = p.affine;
    if (ev) (void)hipEventRecord(ev->ev[2 * kSlotStrip], s);
    auto by_type = [&](auto dc) {
        using D = typename decltype(dc)::type;
        if (silu && !stats_only)
            launch_strip_s<D, true>(p, x, y, af, eps, stats_only, mo, ro, s);
        else
            launch_strip_s<D, false>(p, x, y, af, eps, stats_only, mo, ro, s);
    };
    switch (p.dtype) {
        case GN_DTYPE_F16: by_type(TypeTag<Fp16>{}); break;
        case GN_DTYPE_F32: by_type(TypeTag<F32>{}); break;
        default: by_type(TypeTag<Bf16>{}); break;
    }
    if (ev) (void)hipEventRecord(ev->ev[2 * kSlotStrip + 1], s);
}

// Everything a compute entry point needs after its argument checks.
struct Call {
    hipStream_t stream;
    int dev;
    DeviceGuard guard;
};

gn_status begin_call(void *stream, const std::vector<const void *> &ptrs, Call *c) {
    c->stream = static_cast<hipStream_t>(stream);
    gn_status st = stream_device(c->stream, &c->dev);
    if (st != GN_OK) return st;
    st = c->guard.enter(c->dev);
    if (st != GN_OK) return st;
    for (const void *q : ptrs)
        if (!on_device(q, c->dev)) return GN_UNSUPPORTED;
    return GN_OK;
}

// gamma and beta aligned to their element type.
gn_status check_affine(const void *gamma, const void *beta, int dtype) {
    const uintptr_t m = affine_type(dtype) == Affine::kF32 ? 3u : 1u;
    for (const void *q : {gamma, beta})
        if (q != nullptr && (reinterpret_cast<uintptr_t>(q) & m) != 0) return GN_UNSUPPORTED;
    return GN_OK;
}

gn_status finish_launch() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? GN_OK : GN_DEVICE_ERROR;
}

// Scratch bytes of the full path for a plan: the arrival counter words, then
// the payload (partials, padding, mean/rstd).  gn_plan_rows_dtype reports it.
size_t full_path_scratch_bytes(const Plan &p) {
    if (p.strip) return 0;  // the single launch keeps everything on chip
    return arrivals_bytes(arrival_words(p)) + payload_bytes(p, true);
}

// ---- the fixed scratch of gn_silu_rows_noalloc -------------------------------
// Device address of this device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
std::mutex &fixed_scratch_mutex() {
    static std::mutex *m = new std::mutex;
    return *m;
}
std::map<int, char *> &fixed_scratch_map() {
    static auto *m = new std::map<int, char *>;
    return *m;
}
gn_status fixed_scratch(int dev, char **out) {
    std::lock_guard<std::mutex> lock(fixed_scratch_mutex());
    auto it = fixed_scratch_map().find(dev);
    if (it != fixed_scratch_map().end()) {
        *out = it->second;
        return GN_OK;
    }
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        return GN_DEVICE_ERROR;
    }
    fixed_scratch_map()[dev] = static_cast<char *>(ptr);
    *out = static_cast<char *>(ptr);
    return GN_OK;
}

// Enqueues the full path with the given scratch: `counters` (arrival words,
// zero in stream order) and `payload`.  Events around each kernel when ev.
void enqueue_rows(const Plan &p, const void *x, const void *gamma, const void *beta, void *y,
                  int apply_silu, float eps, unsigned *counters, char *payload, hipStream_t s,
                  const Events *ev) {
    if (p.strip) {
        launch_strip(p, x, y, gamma, beta, apply_silu, eps, 0, nullptr, nullptr, s, ev);
        return;
    }
    const size_t nparts = partial_floats(p);
    const size_t nstats = static_cast<size_t>(p.N) * p.stats.G;
    StatsOut o;
    o.part_s = reinterpret_cast<float *>(payload);
    o.part_q = o.part_s + nparts;
    o.mean = o.part_q + nparts + kFinalizeOverread;
    o.rstd = o.mean + nstats;
    // The late finalize leaves mean/rstd unused: step 1 saves its pivots there.
    o.pivot = p.late ? o.mean : nullptr;
    o.arrivals = counters;
    o.inv_m = p.inv_m;
    o.eps = eps;
    launch_stats(p, x, o, p.late, s, ev);
    launch_apply(p, x, y, o.mean, o.rstd, p.late ? &o : nullptr, gamma, beta, apply_silu, s, ev,
                 p.fused && !p.late ? counters : nullptr);
}

// The full path, optionally with events around each kernel (iters > 0).
// fixed: the scratch is the fixed buffer (gn_silu_rows_noalloc), not the
// stream's allocated one.
gn_status run_rows(const void *x, const float *gamma, const float *beta, void *y, int64_t N,
                   int64_t L, int64_t C, int64_t G, float eps, int apply_silu, int dtype,
                   void *stream, int iters, float *kernel_ms, bool fixed = false) {
    gn_status st = check_shape(x, y, N, L, C, G, eps, apply_silu, true, dtype);
    if (st == GN_OK) st = check_affine(gamma, beta, dtype);
    if (st != GN_OK) return st;
    if (N * L == 0) {
        if (kernel_ms)
            for (int i = 0; i < kSlots; ++i) kernel_ms[i] = -1.0f;
        return GN_OK;
    }
    const Plan p = make_plan(N, L, C, G, dtype);
    if (fixed && full_path_scratch_bytes(p) > static_cast<size_t>(GN_NOALLOC_SCRATCH_BYTES))
        return GN_SCRATCH_TOO_SMALL;
    Call c;
    st = begin_call(stream, {x, y, gamma, beta}, &c);
    if (st != GN_OK) return st;

    if (p.strip) {  // one launch, no scratch
        if (iters <= 0) {
            enqueue_rows(p, x, gamma, beta, y, apply_silu, eps, nullptr, nullptr, c.stream,
                         nullptr);
            return finish_launch();
        }
    } else if (fixed) {
        // Same layout as the stream scratch: counters at the front, then the
        // payload.  The counters this call uses are cleared first (a fill
        // kernel), so whatever an earlier call left in the buffer -- possibly
        // payload of another layout where these counters sit -- is irrelevant.
        char *base = nullptr;
        st = fixed_scratch(c.dev, &base);
        if (st != GN_OK) return st;
        unsigned *counters = reinterpret_cast<unsigned *>(base);
        const int64_t words = arrival_words(p);
        if (p.fused && !p.late) {
            st = zero_counters(counters, words, c.stream);
            if (st != GN_OK) return st;
        }
        enqueue_rows(p, x, gamma, beta, y, apply_silu, eps, counters,
                     base + arrivals_bytes(words), c.stream, nullptr);
        return finish_launch();
    }

    std::unique_lock<std::mutex> lock(scratch_mutex(), std::defer_lock);
    unsigned *counters = nullptr;
    char *payload = nullptr;
    if (!p.strip) {
        lock.lock();
        st = scratch_for(c.dev, c.stream, arrival_words(p), payload_bytes(p, true), &counters,
                         &payload);
        if (st != GN_OK) return st;
    }

    if (iters <= 0) {
        enqueue_rows(p, x, gamma, beta, y, apply_silu, eps, counters, payload, c.stream, nullptr);
        return finish_launch();
    }

    // Measured form: events around every launch, in batches.
    constexpr int kBatch = 64;
    std::vector<Events> evs(kBatch);
    for (auto &e : evs)
        for (auto &h : e.ev)
            if (hipEventCreate(&h) != hipSuccess) return GN_DEVICE_ERROR;
    double sum_ms[kSlots] = {0.0, 0.0, 0.0, 0.0};
    auto launched = [&](int k) {
        if (p.strip) return k == kSlotStrip;
        return k != kSlotStrip && !(k == kSlotFinalize && p.fused);
    };
    st = GN_OK;
    for (int done = 0; done < iters && st == GN_OK;) {
        const int nb = std::min(kBatch, iters - done);
        for (int i = 0; i < nb; ++i)
            enqueue_rows(p, x, gamma, beta, y, apply_silu, eps, counters, payload, c.stream,
                         &evs[i]);
        st = finish_launch();
        if (st == GN_OK && hipStreamSynchronize(c.stream) != hipSuccess) st = GN_DEVICE_ERROR;
        for (int i = 0; i < nb && st == GN_OK; ++i)
            for (int k = 0; k < kSlots; ++k) {
                if (!launched(k)) continue;
                float ms = 0.0f;
                if (hipEventElapsedTime(&ms, evs[i].ev[2 * k], evs[i].ev[2 * k + 1]) != hipSuccess)
                    st = GN_DEVICE_ERROR;
                sum_ms[k] += ms;
            }
        done += nb;
    }
    for (auto &e : evs)
        for (auto &h : e.ev) (void)hipEventDestroy(h);
    if (st != GN_OK) return st;
    for (int k = 0; k < kSlots; ++k)
        kernel_ms[k] = launched(k) ? static_cast<float>(sum_ms[k] / iters) : -1.0f;
    return GN_OK;
}

// Dense channels-last check for the strides of logical (N, C, S1, ..., Sk)
// dimensions (k = 2: NHWC, k = 3: NDHWC): the dense strides are
// (S1*...*Sk*C, 1, S2*...*Sk*C, ..., C).  A dimension of extent 1 may carry
// any stride, as in torch's channels_last tests.
bool dense_channels_last(const int64_t *st, int64_t N, int64_t C, const int64_t *sp, int k) {
    int64_t inner = C;  // dense stride of the innermost spatial dimension
    for (int d = k - 1; d >= 0; --d) {
        if (sp[d] > 1 && st[2 + d] != inner) return false;
        inner *= sp[d];
    }
    if (N > 1 && st[0] != inner) return false;
    if (C > 1 && st[1] != 1) return false;
    return true;
}

// L = product of the k spatial extents, or -1 if one is negative or the
// product overflows int64.
int64_t spatial_rows(const int64_t *sp, int k) {
    int64_t L = 1;
    for (int d = 0; d < k; ++d) {
        if (sp[d] < 0) return -1;
        if (sp[d] > 0 && L > INT64_MAX / sp[d]) return -1;
        L *= sp[d];
    }
    return L;
}

// The strided 4-D and 5-D forms: argument errors first, then the layout.
gn_status run_strided(const void *x, const int64_t *x_strides, const float *gamma,
                      const float *beta, void *y, const int64_t *y_strides, int64_t N,
                      const int64_t *sp, int k, int64_t C, int64_t G, float eps, int apply_silu,
                      int dtype, void *stream) {
    if (x_strides == nullptr || y_strides == nullptr) return GN_INVALID_ARGUMENT;
    const int64_t L = spatial_rows(sp, k);
    if (L < 0) return GN_INVALID_ARGUMENT;
    const gn_status st = check_shape(x, y, N, L, C, G, eps, apply_silu, true, dtype);
    if (st == GN_INVALID_ARGUMENT) return st;
    if (!dense_channels_last(x_strides, N, C, sp, k) ||
        !dense_channels_last(y_strides, N, C, sp, k))
        return GN_UNSUPPORTED;
    return run_rows(x, gamma, beta, y, N, L, C, G, eps, apply_silu, dtype, stream, 0, nullptr);
}

}  // namespace
// ---- fused GroupNorm(+SiLU) -> 3x3 convolution (-> statistics) -------------

// Launch shape of gn_conv3x3 for a problem: real workgroups, grid size and
// whether the XCD-aware block order applies.
struct ConvPlan {
    int tiles_h, tiles_w, nb, xcd_map, wn;
    int64_t blocks, grid;
};

// Workgroups of 256 lanes.  wn = 4 (Co a multiple of 256): 256 output
// channels, 4 waves of 128 pixels x 64 channels; every weight fragment a
// wave pulls from L2 feeds twice the matrix-core work of wn = 2 (2 x 2 waves
// of 64 pixels over 128 channels), and each normalised halo serves twice the
// outputs.  Measured on MI355X at the decoder's ResnetBlock2D shapes: 5-16%
// faster than wn = 2, bitwise the same results (each output's sum runs in
// the same order either way).  (Workgroups of 512 lanes as 2 x 4 waves of 64
// pixels measured 7-10% slower than wn = 2.)
ConvPlan make_conv_plan(int64_t N, int64_t H, int64_t W, int64_t Co) {
    ConvPlan c;
    c.tiles_h = static_cast<int>(ceil_div(H, gnconv::TH));
    c.tiles_w = static_cast<int>(ceil_div(W, gnconv::TW));
    const int64_t tiles = N * c.tiles_h * c.tiles_w;
    c.wn = (Co % 256 == 0) ? 4 : 2;
    c.nb = static_cast<int>(Co / (64 * c.wn));
    c.blocks = tiles * c.nb;
    c.xcd_map = (8 % c.nb == 0) ? 1 : 0;
    // xcd_map: workgroup b runs output-channel block (b % 8) % nb on tile
    // (b / 8) * (8 / nb) + (b % 8) / nb; the grid covers every tile once per
    // block and is a multiple of 8 (the surplus exits at once).
    c.grid = c.xcd_map ? 8 * ceil_div(tiles, 8 / c.nb) : c.blocks;
    return c;
}

gn_status check_conv(const void *x, const float *nmean, const float *nrstd, int64_t G,
                     int apply_silu, const void *wt, const void *res, const void *z, int64_t N,
                     int64_t H, int64_t W, int64_t Ci, int64_t Co, int64_t G2, float eps2,
                     const float *mean2, const float *rstd2) {
    if (x == nullptr || wt == nullptr || z == nullptr) return GN_INVALID_ARGUMENT;
    if (N < 0 || H < 0 || W < 0 || Ci <= 0 || Co <= 0) return GN_INVALID_ARGUMENT;
    if ((nmean == nullptr) != (nrstd == nullptr)) return GN_INVALID_ARGUMENT;
    if (nmean != nullptr && (G <= 0 || Ci % G != 0)) return GN_INVALID_ARGUMENT;
    if (apply_silu != 0 && apply_silu != 1) return GN_INVALID_ARGUMENT;
    if ((mean2 == nullptr) != (rstd2 == nullptr)) return GN_INVALID_ARGUMENT;
    if (mean2 != nullptr) {
        if (G2 <= 0 || Co % G2 != 0) return GN_INVALID_ARGUMENT;
        if (!(eps2 >= 0.0f) || std::isinf(eps2)) return GN_INVALID_ARGUMENT;
    }
    if (W > 0 && H > INT64_MAX / W) return GN_INVALID_ARGUMENT;
    if (H * W > 0 && N > INT64_MAX / (H * W)) return GN_INVALID_ARGUMENT;
    const int64_t pix = N * H * W;
    const int64_t cmax = Ci > Co ? Ci : Co;
    if (pix > 0 && cmax > INT64_MAX / pix / 4) return GN_INVALID_ARGUMENT;
    // the kernel's tile shapes
    if (Ci % gnconv::BK != 0 || Ci > gnconv::kMaxCi || Co % gnconv::BN != 0) return GN_UNSUPPORTED;
    if (mean2 != nullptr && 64 % (Co / G2) != 0) return GN_UNSUPPORTED;  // groups within 64 ch
    for (const void *p : {x, wt, res, z})
        if (p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) != 0) return GN_UNSUPPORTED;
    // grid and 32-bit index limits of the kernel
    if (H > (1 << 20) || W > (1 << 20) || N > (1 << 20)) return GN_UNSUPPORTED;
    // per-sample element offsets of the halo loads are 32-bit
    if (H * W > 0 && (Ci > (INT32_MAX / (H * W)) || Co > (INT32_MAX / (H * W))))
        return GN_UNSUPPORTED;
    if (pix > 0) {
        const ConvPlan c = make_conv_plan(N, H, W, Co);
        if (c.grid >= (int64_t{1} << 31) || int64_t{c.tiles_h} * c.tiles_w >= (int64_t{1} << 31))
            return GN_UNSUPPORTED;
    }
    return GN_OK;
}

template <int WM, int WN, bool SILU, int WPE = 2>
void launch_conv_ws(const gnconv::ConvArgs &a, int64_t grid, bool stats, hipStream_t s) {
    const dim3 g(static_cast<unsigned>(grid)), b(64 * WM * WN);
    const bool res = a.res != nullptr;
    if (stats) {
        if (res)
            gnconv::gn_conv3x3<WM, WN, SILU, true, true, WPE><<<g, b, 0, s>>>(a);
        else
            gnconv::gn_conv3x3<WM, WN, SILU, true, false, WPE><<<g, b, 0, s>>>(a);
    } else {
        if (res)
            gnconv::gn_conv3x3<WM, WN, SILU, false, true, WPE><<<g, b, 0, s>>>(a);
        else
            gnconv::gn_conv3x3<WM, WN, SILU, false, false, WPE><<<g, b, 0, s>>>(a);
    }
}

// Grids of at most this many workgroups (one per CU of an MI355X) run the
// 128-pixel waves compiled for one wave per SIMD.  Only the speed depends on
// it: every variant computes each output in the same order.
constexpr int64_t kConvOneWaveMaxBlocks = 256;

// wn = 2: 2 x 2 waves of 64 pixels x 64 channels; wn = 4: 1 x 4 waves of
// 128 pixels x 64 channels.  256 lanes either way.
void launch_conv(const gnconv::ConvArgs &a, int64_t grid, int wn, bool silu, bool stats,
                 hipStream_t s) {
    if (wn == 4 && grid <= kConvOneWaveMaxBlocks) {
        if (silu)
            launch_conv_ws<1, 4, true, 1>(a, grid, stats, s);
        else
            launch_conv_ws<1, 4, false, 1>(a, grid, stats, s);
    } else if (wn == 4) {
        if (silu)
            launch_conv_ws<1, 4, true>(a, grid, stats, s);
        else
            launch_conv_ws<1, 4, false>(a, grid, stats, s);
    } else {
        if (silu)
            launch_conv_ws<2, 2, true>(a, grid, stats, s);
        else
            launch_conv_ws<2, 2, false>(a, grid, stats, s);
    }
}

}  // namespace gnsilu

using namespace gnsilu;

extern "C" {

gn_status gn_silu_rows_dtype(const void *x, const float *gamma, const float *beta, void *y,
                             int64_t N, int64_t L, int64_t C, int64_t G, float eps,
                             int apply_silu, int dtype, void *stream) {
    return run_rows(x, gamma, beta, y, N, L, C, G, eps, apply_silu, dtype, stream, 0, nullptr);
}

gn_status gn_silu_rows_noalloc(const void *x, const float *gamma, const float *beta, void *y,
                               int64_t N, int64_t L, int64_t C, int64_t G, float eps,
                               int apply_silu, int dtype, void *stream) {
    return run_rows(x, gamma, beta, y, N, L, C, G, eps, apply_silu, dtype, stream, 0, nullptr,
                    true);
}

gn_status gn_noalloc_scratch(int device, void **ptr_out, int64_t *bytes_out) {
    if (ptr_out == nullptr || bytes_out == nullptr || device < 0) return GN_INVALID_ARGUMENT;
    DeviceGuard guard;
    if (guard.enter(device) != GN_OK) return GN_DEVICE_ERROR;
    char *base = nullptr;
    const gn_status st = fixed_scratch(device, &base);
    if (st != GN_OK) return st;
    *ptr_out = base;
    *bytes_out = GN_NOALLOC_SCRATCH_BYTES;
    return GN_OK;
}

gn_status gn_silu_rows(const void *x, const float *gamma, const float *beta, void *y, int64_t N,
                       int64_t L, int64_t C, int64_t G, float eps, int apply_silu,
                       void *stream) {
    return gn_silu_rows_dtype(x, gamma, beta, y, N, L, C, G, eps, apply_silu, GN_DTYPE_BF16,
                              stream);
}

gn_status gn_silu_nhwc_dtype(const void *x, const float *gamma, const float *beta, void *y,
                             int64_t N, int64_t H, int64_t W, int64_t C, int64_t G, float eps,
                             int apply_silu, int dtype, void *stream) {
    if (H < 0 || W < 0) return GN_INVALID_ARGUMENT;
    if (W > 0 && H > INT64_MAX / W) return GN_INVALID_ARGUMENT;
    return gn_silu_rows_dtype(x, gamma, beta, y, N, H * W, C, G, eps, apply_silu, dtype, stream);
}

gn_status gn_silu_nhwc(const void *x, const float *gamma, const float *beta, void *y, int64_t N,
                       int64_t H, int64_t W, int64_t C, int64_t G, float eps, int apply_silu,
                       void *stream) {
    return gn_silu_nhwc_dtype(x, gamma, beta, y, N, H, W, C, G, eps, apply_silu, GN_DTYPE_BF16,
                              stream);
}

gn_status gn_silu_nhwc_strided_dtype(const void *x, const int64_t x_strides[4],
                                     const float *gamma, const float *beta, void *y,
                                     const int64_t y_strides[4], int64_t N, int64_t H, int64_t W,
                                     int64_t C, int64_t G, float eps, int apply_silu, int dtype,
                                     void *stream) {
    const int64_t sp[2] = {H, W};
    return run_strided(x, x_strides, gamma, beta, y, y_strides, N, sp, 2, C, G, eps, apply_silu,
                       dtype, stream);
}

gn_status gn_silu_ndhwc_dtype(const void *x, const float *gamma, const float *beta, void *y,
                              int64_t N, int64_t D, int64_t H, int64_t W, int64_t C, int64_t G,
                              float eps, int apply_silu, int dtype, void *stream) {
    const int64_t sp[3] = {D, H, W};
    const int64_t L = spatial_rows(sp, 3);
    if (L < 0) return GN_INVALID_ARGUMENT;
    return gn_silu_rows_dtype(x, gamma, beta, y, N, L, C, G, eps, apply_silu, dtype, stream);
}

gn_status gn_silu_ndhwc(const void *x, const float *gamma, const float *beta, void *y, int64_t N,
                        int64_t D, int64_t H, int64_t W, int64_t C, int64_t G, float eps,
                        int apply_silu, void *stream) {
    return gn_silu_ndhwc_dtype(x, gamma, beta, y, N, D, H, W, C, G, eps, apply_silu,
                               GN_DTYPE_BF16, stream);
}

gn_status gn_silu_ndhwc_strided_dtype(const void *x, const int64_t x_strides[5],
                                      const float *gamma, const float *beta, void *y,
                                      const int64_t y_strides[5], int64_t N, int64_t D,
                                      int64_t H, int64_t W, int64_t C, int64_t G, float eps,
                                      int apply_silu, int dtype, void *stream) {
    const int64_t sp[3] = {D, H, W};
    return run_strided(x, x_strides, gamma, beta, y, y_strides, N, sp, 3, C, G, eps, apply_silu,
                       dtype, stream);
}

gn_status gn_silu_nhwc_strided(const void *x, const int64_t x_strides[4], const float *gamma,
                               const float *beta, void *y, const int64_t y_strides[4],
                               int64_t N, int64_t H, int64_t W, int64_t C, int64_t G,
                               float eps, int apply_silu, void *stream) {
    return gn_silu_nhwc_strided_dtype(x, x_strides, gamma, beta, y, y_strides, N, H, W, C, G,
                                      eps, apply_silu, GN_DTYPE_BF16, stream);
}

gn_status gn_stats_rows_dtype(const void *x, int64_t N, int64_t L, int64_t C, int64_t G,
                              float eps, int dtype, float *mean_out, float *rstd_out,
                              void *stream) {
    if (mean_out == nullptr || rstd_out == nullptr) return GN_INVALID_ARGUMENT;
    gn_status st = check_shape(x, nullptr, N, L, C, G, eps, 0, false, dtype);
    if (st != GN_OK) return st;
    if (N * L == 0) return GN_OK;
    Call c;
    st = begin_call(stream, {x, mean_out, rstd_out}, &c);
    if (st != GN_OK) return st;
    const Plan p = make_plan(N, L, C, G, dtype);
    if (p.strip) {  // the single launch's own statistics, so that steps 1-2 then 3
                    // give the full path's y bit for bit
        launch_strip(p, x, const_cast<void *>(x), nullptr, nullptr, 0, eps, 1, mean_out, rstd_out,
                     c.stream, nullptr);
        return finish_launch();
    }
    const size_t nparts = partial_floats(p);
    std::lock_guard<std::mutex> lock(scratch_mutex());
    unsigned *counters = nullptr;
    char *payload = nullptr;
    st = scratch_for(c.dev, c.stream, arrival_words(p), payload_bytes(p, false), &counters,
                     &payload);
    if (st != GN_OK) return st;
    StatsOut o;
    o.part_s = reinterpret_cast<float *>(payload);
    o.part_q = o.part_s + nparts;
    o.arrivals = counters;
    o.mean = mean_out;
    o.rstd = rstd_out;
    o.pivot = nullptr;
    o.inv_m = p.inv_m;
    o.eps = eps;
    launch_stats(p, x, o, false, c.stream, nullptr);
    return finish_launch();
}

gn_status gn_stats_rows(const void *x, int64_t N, int64_t L, int64_t C, int64_t G, float eps,
                        float *mean_out, float *rstd_out, void *stream) {
    return gn_stats_rows_dtype(x, N, L, C, G, eps, GN_DTYPE_BF16, mean_out, rstd_out, stream);
}

gn_status gn_apply_rows_dtype(const void *x, const float *mean, const float *rstd,
                              const float *gamma, const float *beta, void *y, int64_t N,
                              int64_t L, int64_t C, int64_t G, int apply_silu, int dtype,
                              void *stream) {
    if (mean == nullptr || rstd == nullptr) return GN_INVALID_ARGUMENT;
    gn_status st = check_shape(x, y, N, L, C, G, 0.0f, apply_silu, true, dtype);
    if (st == GN_OK) st = check_affine(gamma, beta, dtype);
    if (st != GN_OK) return st;
    if (N * L == 0) return GN_OK;
    Call c;
    st = begin_call(stream, {x, y, mean, rstd, gamma, beta}, &c);
    if (st != GN_OK) return st;
    const Plan p = make_plan(N, L, C, G, dtype);
    launch_apply(p, x, y, mean, rstd, nullptr, gamma, beta, apply_silu, c.stream, nullptr);
    return finish_launch();
}

gn_status gn_apply_rows(const void *x, const float *mean, const float *rstd, const float *gamma,
                        const float *beta, void *y, int64_t N, int64_t L, int64_t C, int64_t G,
                        int apply_silu, void *stream) {
    return gn_apply_rows_dtype(x, mean, rstd, gamma, beta, y, N, L, C, G, apply_silu,
                               GN_DTYPE_BF16, stream);
}

gn_status gn_profile_rows_dtype(const void *x, const float *gamma, const float *beta, void *y,
                                int64_t N, int64_t L, int64_t C, int64_t G, float eps,
                                int apply_silu, int dtype, void *stream, int iters,
                                float *kernel_ms, int *n_kernels) {
    if (kernel_ms == nullptr || n_kernels == nullptr || iters < 1 || iters > 100000)
        return GN_INVALID_ARGUMENT;
    *n_kernels = kSlots;
    return run_rows(x, gamma, beta, y, N, L, C, G, eps, apply_silu, dtype, stream, iters,
                    kernel_ms);
}

gn_status gn_profile_rows(const void *x, const float *gamma, const float *beta, void *y,
                          int64_t N, int64_t L, int64_t C, int64_t G, float eps, int apply_silu,
                          void *stream, int iters, float *kernel_ms, int *n_kernels) {
    return gn_profile_rows_dtype(x, gamma, beta, y, N, L, C, G, eps, apply_silu, GN_DTYPE_BF16,
                                 stream, iters, kernel_ms, n_kernels);
}

gn_status gn_plan_rows_dtype(int64_t N, int64_t L, int64_t C, int64_t G, int dtype,
                             int64_t plan_out[15]) {
    if (plan_out == nullptr) return GN_INVALID_ARGUMENT;
    static const uint16_t aligned_probe[8] __attribute__((aligned(16))) = {};
    const gn_status st =
        check_shape(aligned_probe, aligned_probe, N, L, C, G, 0.0f, 0, true, dtype);
    if (st != GN_OK) return st;
    if (N * L == 0) {
        for (int i = 0; i < 15; ++i) plan_out[i] = 0;
        return GN_OK;
    }
    const Plan p = make_plan(N, L, C, G, dtype);
    plan_out[0] = static_cast<int64_t>(p.lay.w) * p.lay.nv;
    plan_out[1] = p.stats.tiles;
    plan_out[2] = p.stats.full;
    plan_out[3] = p.stats.tpc;
    plan_out[4] = p.stats.K;
    plan_out[5] = p.apply.tpc;
    plan_out[6] = p.apply.K;
    plan_out[7] = static_cast<int64_t>(full_path_scratch_bytes(p));
    plan_out[8] = p.apply_ntl ? 1 : 0;
    plan_out[9] = p.lay.w;
    plan_out[10] = p.lay.a;
    plan_out[11] = p.lay.t;
    plan_out[12] = p.stats.plain_tail;
    plan_out[13] = p.late ? 1 : 0;
    plan_out[14] = p.threads;
    return GN_OK;
}

gn_status gn_plan_single_launch(int64_t N, int64_t L, int64_t C, int64_t G, int dtype,
                                int64_t plan_out[6]) {
    if (plan_out == nullptr) return GN_INVALID_ARGUMENT;
    static const uint16_t aligned_probe[8] __attribute__((aligned(16))) = {};
    const gn_status st =
        check_shape(aligned_probe, aligned_probe, N, L, C, G, 0.0f, 0, true, dtype);
    if (st != GN_OK) return st;
    for (int i = 0; i < 6; ++i) plan_out[i] = 0;
    if (N * L == 0) return GN_OK;
    const Plan p = make_plan(N, L, C, G, dtype);
    if (!p.strip) return GN_OK;
    plan_out[0] = 1;
    plan_out[1] = p.sg.gpw;
    plan_out[2] = p.sg.P;
    plan_out[3] = p.sg.blocks;
    plan_out[4] = kStripThreads;
    plan_out[5] = ceil_div(L, kStripThreads / p.sg.P);
    return GN_OK;
}

gn_status gn_plan_rows(int64_t N, int64_t L, int64_t C, int64_t G, int64_t plan_out[8]) {
    if (plan_out == nullptr) return GN_INVALID_ARGUMENT;
    int64_t full[15] = {};
    const gn_status st = gn_plan_rows_dtype(N, L, C, G, GN_DTYPE_BF16, full);
    if (st == GN_OK)
        for (int i = 0; i < 8; ++i) plan_out[i] = full[i];
    return st;
}

gn_status gn_conv3x3_pack_weights(const void *wt, void *packed, int64_t Ci, int64_t Co,
                                  void *stream) {
    if (wt == nullptr || packed == nullptr || Ci <= 0 || Co <= 0) return GN_INVALID_ARGUMENT;
    if (Ci % gnconv::BK != 0 || Ci > gnconv::kMaxCi || Co % gnconv::BN != 0) return GN_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(wt) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(packed) & 15u) != 0)
        return GN_UNSUPPORTED;
    Call c;
    gn_status st = begin_call(stream, {wt, packed}, &c);
    if (st != GN_OK) return st;
    const int64_t pieces = Co * 9 * Ci / 8;
    gnconv::gn_conv_pack_weights<<<static_cast<unsigned>(ceil_div(pieces, gnconv::kThreads)),
                                   gnconv::kThreads, 0, c.stream>>>(
        static_cast<const uint16_t *>(wt), static_cast<uint16_t *>(packed), static_cast<int>(Ci),
        pieces);
    return finish_launch();
}

namespace gnsilu {
namespace {

// The convolution with weights either in the [Co][3][3][Ci] layout (packed
// into the stream's scratch first) or already packed.
gn_status run_conv(const void *x, const float *norm_mean, const float *norm_rstd,
                   const float *gamma, const float *beta, int64_t G, int apply_silu,
                   const void *wt, bool wt_packed, const float *bias, const void *res, void *z,
                   int64_t N, int64_t H, int64_t W, int64_t Ci, int64_t Co, int64_t G2, float eps2,
                   float *mean2_out, float *rstd2_out, void *stream) {
    gn_status st = check_conv(x, norm_mean, norm_rstd, G, apply_silu, wt, res, z, N, H, W, Ci,
                              Co, G2, eps2, mean2_out, rstd2_out);
    if (st != GN_OK) return st;
    if (N * H * W == 0) return GN_OK;
    Call c;
    st = begin_call(stream, {x, norm_mean, norm_rstd, gamma, beta, wt, bias, res, z, mean2_out,
                             rstd2_out},
                    &c);
    if (st != GN_OK) return st;
    const ConvPlan cp = make_conv_plan(N, H, W, Co);
    gnconv::ConvArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.mean = norm_mean;
    a.rstd = norm_rstd;
    a.gamma = gamma;
    a.beta = beta;
    a.wt = static_cast<const uint16_t *>(wt);
    a.bias = bias;
    a.res = static_cast<const uint16_t *>(res);
    a.z = static_cast<uint16_t *>(z);
    a.part = nullptr;
    a.N = static_cast<int>(N);
    a.H = static_cast<int>(H);
    a.W = static_cast<int>(W);
    a.Ci = static_cast<int>(Ci);
    a.Co = static_cast<int>(Co);
    a.G = norm_mean ? static_cast<int>(G) : 1;
    a.G2 = mean2_out ? static_cast<int>(G2) : 1;
    a.tiles_h = cp.tiles_h;
    a.tiles_w = cp.tiles_w;
    a.nb = cp.nb;
    a.xcd_map = cp.xcd_map;
    a.blocks = cp.blocks;
    const bool stats = mean2_out != nullptr;
    const int64_t tiles_per_sample = int64_t{cp.tiles_h} * cp.tiles_w;

    std::unique_lock<std::mutex> lock(scratch_mutex(), std::defer_lock);
    const size_t pack_bytes = wt_packed ? 0 : align_up(static_cast<size_t>(Co * 9 * Ci) * 2, 256);
    const size_t part_bytes =
        stats ? sizeof(float) * 4 * static_cast<size_t>(N * tiles_per_sample * G2) : 0;
    if (pack_bytes + part_bytes > 0) {
        lock.lock();
        unsigned *counters = nullptr;
        char *payload = nullptr;
        st = scratch_for(c.dev, c.stream, 0, pack_bytes + part_bytes, &counters, &payload);
        if (st != GN_OK) return st;
        if (!wt_packed) {
            const int64_t pieces = Co * 9 * Ci / 8;
            gnconv::gn_conv_pack_weights<<<static_cast<unsigned>(
                                               ceil_div(pieces, gnconv::kThreads)),
                                           gnconv::kThreads, 0, c.stream>>>(
                static_cast<const uint16_t *>(wt), reinterpret_cast<uint16_t *>(payload),
                static_cast<int>(Ci), pieces);
            a.wt = reinterpret_cast<const uint16_t *>(payload);
        }
        if (stats) a.part = reinterpret_cast<float *>(payload + pack_bytes);
    }
    launch_conv(a, cp.grid, cp.wn, apply_silu != 0, stats, c.stream);
    if (stats)
        gnconv::gn_conv_stats_finalize<<<static_cast<unsigned>(N * G2), gnconv::kThreads, 0,
                                         c.stream>>>(a.part, static_cast<int>(tiles_per_sample),
                                                     static_cast<int>(G2), eps2, mean2_out,
                                                     rstd2_out);
    return finish_launch();
}

}  // namespace
}  // namespace gnsilu

gn_status gn_conv3x3_nhwc(const void *x, const float *norm_mean, const float *norm_rstd,
                          const float *gamma, const float *beta, int64_t G, int apply_silu,
                          const void *wt, const float *bias, const void *res, void *z, int64_t N,
                          int64_t H, int64_t W, int64_t Ci, int64_t Co, int64_t G2, float eps2,
                          float *mean2_out, float *rstd2_out, void *stream) {
    return run_conv(x, norm_mean, norm_rstd, gamma, beta, G, apply_silu, wt, false, bias, res, z,
                    N, H, W, Ci, Co, G2, eps2, mean2_out, rstd2_out, stream);
}

gn_status gn_conv3x3_nhwc_packed(const void *x, const float *norm_mean, const float *norm_rstd,
                                 const float *gamma, const float *beta, int64_t G,
                                 int apply_silu, const void *packed_wt, const float *bias,
                                 const void *res, void *z, int64_t N, int64_t H, int64_t W,
                                 int64_t Ci, int64_t Co, int64_t G2, float eps2,
                                 float *mean2_out, float *rstd2_out, void *stream) {
    return run_conv(x, norm_mean, norm_rstd, gamma, beta, G, apply_silu, packed_wt, true, bias,
                    res, z, N, H, W, Ci, Co, G2, eps2, mean2_out, rstd2_out, stream);
}

gn_status gn_conv3x3_plan(int64_t N, int64_t H, int64_t W, int64_t Ci, int64_t Co, int64_t G2,
                          int64_t plan_out[7]) {
    if (plan_out == nullptr) return GN_INVALID_ARGUMENT;
    static const uint16_t probe[8] __attribute__((aligned(16))) = {};
    static float fprobe[4];
    const gn_status st = check_conv(probe, nullptr, nullptr, 0, 0, probe, nullptr, probe, N, H,
                                    W, Ci, Co, G2, 0.0f, G2 > 0 ? fprobe : nullptr,
                                    G2 > 0 ? fprobe : nullptr);
    if (st != GN_OK) return st;
    for (int i = 0; i < 7; ++i) plan_out[i] = 0;
    if (N * H * W == 0) return GN_OK;
    const ConvPlan c = make_conv_plan(N, H, W, Co);
    plan_out[0] = c.tiles_h;
    plan_out[1] = c.tiles_w;
    plan_out[2] = c.nb;
    plan_out[3] = c.xcd_map;
    plan_out[4] = c.blocks;
    plan_out[5] = c.grid;
    plan_out[6] = c.wn;
    return GN_OK;
}

const char *gn_kernel_name(int i) { return (i >= 0 && i < kSlots) ? kKernelNames[i] : nullptr; }

const char *gn_status_string(gn_status s) {
    switch (s) {
        case GN_OK: return "GN_OK";
        case GN_UNSUPPORTED: return "GN_UNSUPPORTED: input outside the supported set; fall back";
        case GN_INVALID_ARGUMENT: return "GN_INVALID_ARGUMENT: not a valid GroupNorm call";
        case GN_DEVICE_ERROR: return "GN_DEVICE_ERROR: a HIP call failed";
        case GN_SCRATCH_TOO_SMALL:
            return "GN_SCRATCH_TOO_SMALL: the call needs more scratch than the fixed "
                   "no-allocation buffer holds";
    }
    return "unknown gn_status";
}

int gn_version(void) { return 500; }

gn_status gn_device_info(int device, int64_t info_out[6]) {
    if (info_out == nullptr || device < 0) return GN_INVALID_ARGUMENT;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
        (void)hipGetLastError();
        return GN_DEVICE_ERROR;
    }
    info_out[0] = prop.multiProcessorCount;
    info_out[1] = prop.clockRate;
    info_out[2] = prop.memoryClockRate;
    info_out[3] = prop.memoryBusWidth;
    info_out[4] = static_cast<int64_t>(prop.totalGlobalMem);
    info_out[5] = prop.warpSize;
    return GN_OK;
}

}  // extern "C"
