"""Benchmark of the channels-last GroupNorm+SiLU path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one call of the whole path (statistics, finalize, apply+SiLU) on
one seeded synthetic bf16 tensor already resident in HBM.  The workload is the
largest decoder shape of the pages' kernel microbenchmark, logical
(N, C, H, W) = (1, 256, 1024, 1024) stored channels-last, G = 32, eps = 1e-6,
SiLU on.  Throughput counts algorithmic bytes: two reads and one write of the
bf16 tensor (3 * 2 * numel), per call.

Prints ONE JSON line.  Besides the contract fields it carries
  roofline     -- the dominant kernel (gn_apply): algorithmic bytes per
                  launch / its mean duration from HIP events recorded around
                  each launch on the stream it runs on (an effective rate: the
                  Infinity Cache serves part of its re-read of x), beside the
                  whole call's fraction, warm and cold;
  cpu_baseline -- the fp64 oracle (test infrastructure) timed on the host's
                  cores on the same tensor, and once on one core;
  kernels_ms   -- mean duration of each kernel from the same events;
  other_shapes -- us/call of the other four decoder shapes (context);
  other_dtypes -- the headline shape with fp16 and fp32 input/output;
  wide_shapes  -- shapes outside the pages' kernel's support set (C not a
                  power of two, C > 2048, 5-D NDHWC), measured the same way;
  extra_shapes -- (1,512,256,256), rows (1,16384,512) without SiLU, and one
                  GPU's share (1/8 of the rows) of the headline tensor;
  per_call     -- the headline call timed call by call: warm (back to back)
                  and cold (a 1 GiB buffer written, or read, before each call,
                  so the Infinity Cache holds none of x): mean / median / min;
  single_launch_shapes -- small rows shapes that take the single launch
                  (steps 1-3 in one kernel), us/call;
  resnet_block -- the decoder's ResnetBlock2D (GroupNorm -> SiLU -> conv3x3 ->
                  GroupNorm -> SiLU -> conv3x3 + shortcut) with the GroupNorms
                  fused into the convolutions, against the same block run as
                  separate GroupNorm and convolution calls (ours, and with the
                  convolutions from torch / MIOpen), plus the fused
                  convolution's matrix-core roofline.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0              # MI355X HBM3E, published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak, published
RESNET_SHAPES = ((1, 512, 128, 128), (1, 512, 256, 256), (1, 256, 512, 512))
# small rows shapes (N, L, C), G = 32, that take the single launch
SINGLE_LAUNCH_SHAPES = ((2, 1024, 256), (8, 1024, 128), (4, 2048, 256))
H200_US = {                        # the pages' new-kernel column (H200), context only
    "gn_silu_1x512x128x128": 76.0,
    "gn_silu_1x512x256x256": 121.0,
    "gn_silu_1x512x512x512": 311.1,
    "gn_silu_1x256x1024x1024": 913.8,
    "gn_silu_1x128x1024x1024": 307.9,
}
HEADLINE = 3                       # index into gn_inputs.WORKLOADS
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gn_silu_1x256x1024x1024.json")
KERNEL_SOURCES = [
    os.path.join(ROOT, "groupnorm_silu_normalization_amd", "csrc", "gn_kernels.hpp"),
    os.path.join(ROOT, "groupnorm_silu_normalization_amd", "csrc", "gn_api.hip"),
    os.path.join(ROOT, "groupnorm_silu_normalization_amd", "csrc", "gn_conv.hpp"),
]


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """Counter-measured HBM bytes per gn_apply launch, if taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("gn_apply_bytes_per_launch")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def device_tensor(torch, bits, dev):
    import numpy as np
    return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)


def time_calls(torch, fn, steps, warmup, stream):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall


def cpu_baseline(w, x_bits, gamma, beta, budget_s):
    import numpy as np

    import oracle
    threads = oracle.max_threads()
    runs, total = 0, 0.0
    while runs < 1 or (total < budget_s and runs < 5):
        t0 = time.perf_counter()
        y = oracle.gn_silu(x_bits, gamma, beta, w.N, w.L, w.C, w.G, w.eps, w.apply_silu,
                           out_dtype=np.float32)
        total += time.perf_counter() - t0
        runs += 1
        del y
    per_call = total / runs
    # the same call on one core, once (the oracle is the same code either way)
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        y = oracle.gn_silu(x_bits, gamma, beta, w.N, w.L, w.C, w.G, w.eps, w.apply_silu,
                           out_dtype=np.float32)
        one = time.perf_counter() - t0
        del y
    finally:
        oracle.set_threads(threads)
    return {
        "value": round(w.algorithmic_bytes / per_call / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "us_per_call": round(per_call * 1e6, 1),
        "sample": "the full %s tensor (%d elements), %d oracle call(s), fp64 two-pass, "
                  "%d OpenMP threads" % (w.label(), w.numel, runs, threads),
        "one_core": {"value": round(w.algorithmic_bytes / one / 1e9, 3), "unit": "GB/s",
                     "us_per_call": round(one * 1e6, 1), "cores": 1,
                     "sample": "the same tensor, one oracle call on one thread"},
    }


def time_events(torch, fn, steps, warmup, stream):
    """Mean ms of fn over `steps` calls between two events on `stream`."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def per_call_us(torch, fn, n, stream, before=None):
    """Sorted durations (us) of n calls of fn, each between its own pair of
    events on `stream`; `before`, if given, runs untimed ahead of every call
    on the same stream."""
    evs = []
    for _ in range(n):
        if before is not None:
            before()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)


def call_stats(us, nbytes):
    med = us[len(us) // 2]
    return {"calls": len(us), "mean_us": round(sum(us) / len(us), 2), "median_us": round(med, 2),
            "min_us": round(us[0], 2), "max_us": round(us[-1], 2),
            "GB_s_median": round(nbytes / (med * 1e-6) / 1e9, 1),
            "frac_of_peak_median": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def graph_of(torch, fn, stream):
    """fn captured into a HIP graph on `stream` (warmed up there first, so the
    library's per-stream scratch exists before capture and nothing is
    allocated while capturing)."""
    with torch.cuda.stream(stream):
        for _ in range(3):
            fn()
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    stream.synchronize()
    return g


def resnet_block(torch, gn, dev, shp, args):
    """ResnetBlock2D of the decoder at logical shape (N, C, H, W), C -> C, G=32.

    fused:    statistics of x; conv1 with GroupNorm1+SiLU in its prologue and
              the statistics for GroupNorm2 in its epilogue; conv2 with
              GroupNorm2+SiLU in its prologue and the shortcut x added in its
              epilogue.  Two full-tensor convolutions, one statistics pass.
    unfused:  GroupNorm1+SiLU; conv1; GroupNorm2+SiLU; conv2 + shortcut (our
              kernels, the same convolution kernel without the fusion).
    torch_conv: the unfused block with torch's conv2d (MIOpen) for the two
              convolutions and the shortcut added by torch.
    Seeded synthetic activations and weights (1/sqrt(9C)-scaled normal); the
    convolution FLOPs are 2*N*H*W*C*9*C per conv.  The weights are constants
    of the model, so both of our blocks use weights packed once, before the
    timed region (gn_conv3x3_pack_weights); conv_unpacked_us times the entry
    that packs on every call.  Our blocks are timed as HIP-graph replays (the
    kernel sequence without host launch overhead, as a decoder would run it)
    and eagerly; the torch block is timed eagerly (its convolution library
    is not captured).
    """
    N, C, H, W = shp
    G = 32
    g = torch.Generator(device="cpu").manual_seed(C * 7 + H)
    x = (torch.randn(N, C, H, W, generator=g) * 1.5 + 0.3).to(dev).bfloat16() \
        .contiguous(memory_format=torch.channels_last)
    ws = [(torch.randn(C, C, 3, 3, generator=g) / (9 * C) ** 0.5).to(dev).bfloat16()
          .contiguous(memory_format=torch.channels_last) for _ in range(2)]
    bs = [(torch.randn(C, generator=g) * 0.1).to(dev) for _ in range(2)]
    gam = [(1 + 0.1 * torch.randn(C, generator=g)).to(dev) for _ in range(2)]
    bet = [(0.1 * torch.randn(C, generator=g)).to(dev) for _ in range(2)]
    rows = x.permute(0, 2, 3, 1).reshape(N, H * W, C)
    stream = torch.cuda.current_stream(dev)
    with torch.no_grad():
        pw = [gn.pack_conv3x3_weight(w) for w in ws]

    def fused():
        m1, r1 = gn.group_stats_rows(rows, G, 1e-6)
        h, m2, r2 = gn.conv3x3(x, pw[0], bs[0], norm=(m1, r1, gam[0], bet[0]), apply_silu=True,
                               next_groups=G)
        return gn.conv3x3(h, pw[1], bs[1], norm=(m2, r2, gam[1], bet[1]), apply_silu=True,
                          residual=x)

    def unfused():
        y1 = gn.group_norm_silu_4d(x, G, gam[0], bet[0], 1e-6)
        h = gn.conv3x3(y1, pw[0], bs[0])
        y2 = gn.group_norm_silu_4d(h, G, gam[1], bet[1], 1e-6)
        return gn.conv3x3(y2, pw[1], bs[1], residual=x)

    bb = [b.bfloat16() for b in bs]

    def torch_conv():
        y1 = gn.group_norm_silu_4d(x, G, gam[0], bet[0], 1e-6)
        h = torch.nn.functional.conv2d(y1, ws[0], bb[0], padding=1)
        y2 = gn.group_norm_silu_4d(h, G, gam[1], bet[1], 1e-6)
        return torch.nn.functional.conv2d(y2, ws[1], bb[1], padding=1) + x

    m1, r1 = gn.group_stats_rows(rows, G, 1e-6)

    def conv1_fused():
        return gn.conv3x3(x, pw[0], bs[0], norm=(m1, r1, gam[0], bet[0]), apply_silu=True,
                          next_groups=G)

    def conv_plain():
        return gn.conv3x3(x, pw[0], bs[0])

    def conv_unpacked():
        return gn.conv3x3(x, ws[0], bs[0], norm=(m1, r1, gam[0], bet[0]), apply_silu=True,
                          next_groups=G)

    steps = max(5, min(args.steps, 30))
    gstream = torch.cuda.Stream(dev)

    def best(fn, s, rounds):
        return min(time_events(torch, fn, steps, 3, s) for _ in range(rounds))

    with torch.no_grad():
        for f in (fused, unfused, torch_conv):
            if f() is None:
                raise RuntimeError("resnet block declined")
        g_f = graph_of(torch, fused, gstream)
        g_u = graph_of(torch, unfused, gstream)
        # clocks up before anything is timed; then each variant twice, in
        # alternating order, best of the two (no order bias)
        with torch.cuda.stream(gstream):
            for _ in range(30):
                g_u.replay()
        gstream.synchronize()
        t_f = t_u = t_fe = t_ue = float("inf")
        for _ in range(2):
            with torch.cuda.stream(gstream):
                t_f = min(t_f, time_events(torch, g_f.replay, steps, 3, gstream))
                t_u = min(t_u, time_events(torch, g_u.replay, steps, 3, gstream))
            t_fe = min(t_fe, time_events(torch, fused, steps, 3, stream))
            t_ue = min(t_ue, time_events(torch, unfused, steps, 3, stream))
        t_t = best(torch_conv, stream, 2)
        t_c1 = best(conv1_fused, stream, 2)
        t_cp = best(conv_plain, stream, 2)
        t_cu = best(conv_unpacked, stream, 2)
        t_tc = best(lambda: torch.nn.functional.conv2d(x, ws[0], bb[0], padding=1), stream, 2)
        # the same contraction as a plain library GEMM (hipBLASLt through
        # torch.matmul, contiguous bf16 operands): M = pixels, K = 9*C, N = C
        ga_ = torch.randn(N * H * W, 9 * C, device=dev, dtype=torch.bfloat16)
        gb_ = torch.randn(9 * C, C, device=dev, dtype=torch.bfloat16)
        t_gemm = best(lambda: torch.matmul(ga_, gb_), stream, 2)
        del ga_, gb_
    flops = 2.0 * N * H * W * C * 9 * C
    tf = flops / (t_c1 * 1e-3) / 1e12
    tf_plain = flops / (t_cp * 1e-3) / 1e12
    tf_gemm = flops / (t_gemm * 1e-3) / 1e12
    return {
        "shape_nchw": [N, C, H, W],
        "fused_us": round(t_f * 1e3, 1),
        "unfused_us": round(t_u * 1e3, 1),
        "timing": "fused_us / unfused_us: HIP-graph replays; *_eager_us: eager calls; "
                  "each the best of two rounds in alternating order after a warm-up",
        "fused_eager_us": round(t_fe * 1e3, 1),
        "unfused_eager_us": round(t_ue * 1e3, 1),
        "torch_conv_us": round(t_t * 1e3, 1),
        "fused_speedup_vs_unfused": round(t_u / t_f, 3),
        "fused_speedup_vs_torch_conv": round(t_t / t_f, 3),
        "conv_fused_prologue_stats_us": round(t_c1 * 1e3, 1),
        "conv_plain_us": round(t_cp * 1e3, 1),
        "conv_unpacked_us": round(t_cu * 1e3, 1),
        "torch_conv2d_us": round(t_tc * 1e3, 1),
        "conv_roofline": {"kernel": "gn_conv3x3 (GroupNorm+SiLU prologue, statistics epilogue)",
                          "bound": "mfma", "achieved": round(tf, 1),
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                          "flops_per_launch": flops,
                          "plain_conv_frac": round(tf_plain / MFMA_BF16_PEAK_TFLOPS, 4)},
        "library_gemm_reference": {
            "what": "torch.matmul (hipBLASLt) on the same contraction as one plain GEMM: "
                    "[N*H*W, 9*C] x [9*C, C], contiguous bf16, no halo, no fusion",
            "us": round(t_gemm * 1e3, 1),
            "TFLOP_s": round(tf_gemm, 1),
            "frac": round(tf_gemm / MFMA_BF16_PEAK_TFLOPS, 4),
            "fused_conv_over_gemm_time": round(t_c1 / t_gemm, 3),
            "plain_conv_over_gemm_time": round(t_cp / t_gemm, 3),
        },
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--no-other-shapes", action="store_true")
    ap.add_argument("--no-other-dtypes", action="store_true")
    ap.add_argument("--no-wide-shapes", action="store_true")
    ap.add_argument("--no-extra-shapes", action="store_true")
    ap.add_argument("--no-resnet-block", action="store_true")
    ap.add_argument("--no-single-launch", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (for scaling PMC byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this library's path runs on a single GPU and "
              "no multi-GPU figure is produced (asked for --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")

    import numpy as np
    import torch

    import groupnorm_silu_normalization_amd as gn
    from gn_inputs import EXTRA_WORKLOADS, WIDE_WORKLOADS, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    stream = torch.cuda.current_stream(dev)

    w = WORKLOADS[HEADLINE]
    log("inputs %s %s" % (w.name, w.label()))
    x_bits, gamma, beta = make_inputs(w)
    x = device_tensor(torch, x_bits, dev).reshape(w.N, w.L, w.C)
    y = torch.empty_like(x)
    g = torch.from_numpy(gamma).to(dev)
    b = torch.from_numpy(beta).to(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    xp, yp = ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr())
    gp, bp = ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(b.data_ptr())

    def step():
        code = gn.gn_silu_nhwc(xp, gp, bp, yp, w.N, w.H, w.W, w.C, w.G, w.eps, 1, sh)
        if code != 0:
            raise RuntimeError(gn.status_text(code))

    log("timing %d steps after %d warmup" % (args.steps, args.warmup))
    ms, wall = time_calls(torch, step, args.steps, args.warmup, stream)
    value = w.algorithmic_bytes / (ms * 1e-3) / 1e9

    log("per-kernel events over %d steps" % args.steps)
    kms = gn.profile_rows(x, w.G, g, b, w.eps, True, y, args.steps)  # launched kernels only
    apply_ms = kms["gn_apply"]
    apply_bytes = 4 * w.numel  # one read and one write of the bf16 tensor
    achieved = apply_bytes / (apply_ms * 1e-3) / 1e9
    traffic = measured_traffic()

    # Each call timed alone: warm (back to back), then cold, with a 1 GiB buffer
    # touched (untimed, same stream) before every call so the 256 MB Infinity
    # Cache holds none of x.  Written, the buffer also leaves up to a cache's
    # worth of dirty lines whose write-back lands in the timed call; read, it
    # leaves clean lines only.
    log("per-call events, warm and cold")
    warm_us = per_call_us(torch, step, max(args.steps, 20), stream)
    scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cold_w_us = per_call_us(torch, step, 20, stream, before=lambda: scrub.fill_(1.0))
    cold_r_us = per_call_us(torch, step, 20, stream, before=lambda: scrub.sum())
    del scrub
    per_call = {"warm": call_stats(warm_us, w.algorithmic_bytes),
                "cold_after_write": call_stats(cold_w_us, w.algorithmic_bytes),
                "cold_after_read": call_stats(cold_r_us, w.algorithmic_bytes),
                "cold_note": "before each call a 1 GiB buffer is written (cold_after_write) "
                             "or read (cold_after_read), untimed, on the same stream"}

    other = {}
    if not args.no_other_shapes:
        for i, ow in enumerate(WORKLOADS):
            if i == HEADLINE:
                continue
            log("context shape %s" % ow.label())
            ob, og, obeta = make_inputs(ow)
            ox = device_tensor(torch, ob, dev)
            oy = torch.empty_like(ox)
            ogt, obt = torch.from_numpy(og).to(dev), torch.from_numpy(obeta).to(dev)
            oxp, oyp = ctypes.c_void_p(ox.data_ptr()), ctypes.c_void_p(oy.data_ptr())
            ogp, obp = ctypes.c_void_p(ogt.data_ptr()), ctypes.c_void_p(obt.data_ptr())

            def ostep(ow=ow, oxp=oxp, oyp=oyp, ogp=ogp, obp=obp):
                code = gn.gn_silu_nhwc(oxp, ogp, obp, oyp, ow.N, ow.H, ow.W, ow.C, ow.G,
                                       ow.eps, 1, sh)
                if code != 0:
                    raise RuntimeError(gn.status_text(code))

            oms, _ = time_calls(torch, ostep, args.steps, args.warmup, stream)
            ok = gn.profile_rows(ox.reshape(ow.N, ow.L, ow.C), ow.G, ogt, obt, ow.eps, True,
                                 oy.reshape(ow.N, ow.L, ow.C), args.steps)
            other[ow.name] = {
                "shape_nchw": [ow.N, ow.C, ow.H, ow.W],
                "us_per_call": round(oms * 1e3, 2),
                "GB_s": round(ow.algorithmic_bytes / (oms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(ow.algorithmic_bytes / (oms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "kernels_us": {k: round(v * 1e3, 2) for k, v in ok.items()},
                "h200_us_context": H200_US.get(ow.name),
            }
            del ox, oy

    dtypes = {}
    if not args.no_other_dtypes:
        for dname, tdt, esize in (("f16", torch.float16, 2), ("f32", torch.float32, 4)):
            log("headline shape in %s" % dname)
            dx_np, dg, dbeta = make_inputs(w, dtype=dname)
            dx = torch.from_numpy(dx_np).to(dev).reshape(w.N, w.L, w.C)
            assert dx.dtype == tdt
            dy = torch.empty_like(dx)
            dgt, dbt = torch.from_numpy(dg).to(dev), torch.from_numpy(dbeta).to(dev)
            code_dt = int(gn.dtype_code(tdt))
            dxp, dyp = ctypes.c_void_p(dx.data_ptr()), ctypes.c_void_p(dy.data_ptr())
            dgp, dbp = ctypes.c_void_p(dgt.data_ptr()), ctypes.c_void_p(dbt.data_ptr())

            def dstep(dxp=dxp, dyp=dyp, dgp=dgp, dbp=dbp, code_dt=code_dt):
                code = gn.gn_silu_nhwc_dtype(dxp, dgp, dbp, dyp, w.N, w.H, w.W, w.C, w.G, w.eps,
                                             1, code_dt, sh)
                if code != 0:
                    raise RuntimeError(gn.status_text(code))

            dms, _ = time_calls(torch, dstep, args.steps, args.warmup, stream)
            dk = gn.profile_rows(dx, w.G, dgt, dbt, w.eps, True, dy, args.steps)
            dbytes = 3 * esize * w.numel
            dtypes[dname] = {
                "us_per_call": round(dms * 1e3, 2),
                "bytes_per_call": dbytes,
                "GB_s": round(dbytes / (dms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "kernels_us": {k: round(v * 1e3, 2) for k, v in dk.items()},
            }
            del dx, dy, dx_np

    wide = {}
    if not args.no_wide_shapes:
        for ww in WIDE_WORKLOADS:
            log("wide shape %s" % ww.label())
            wb, wg, wbeta = make_inputs(ww)
            wx = device_tensor(torch, wb, dev).reshape(ww.N, ww.L, ww.C)
            wy = torch.empty_like(wx)
            wgt, wbt = torch.from_numpy(wg).to(dev), torch.from_numpy(wbeta).to(dev)
            wxp, wyp = ctypes.c_void_p(wx.data_ptr()), ctypes.c_void_p(wy.data_ptr())
            wgp, wbp = ctypes.c_void_p(wgt.data_ptr()), ctypes.c_void_p(wbt.data_ptr())

            def wstep(ww=ww, wxp=wxp, wyp=wyp, wgp=wgp, wbp=wbp):
                code = gn.gn_silu_rows(wxp, wgp, wbp, wyp, ww.N, ww.L, ww.C, ww.G, ww.eps, 1, sh)
                if code != 0:
                    raise RuntimeError(gn.status_text(code))

            wms, _ = time_calls(torch, wstep, args.steps, args.warmup, stream)
            wk = gn.profile_rows(wx, ww.G, wgt, wbt, ww.eps, True, wy, args.steps)
            plan = gn.plan_rows(ww.N, ww.L, ww.C, ww.G)
            wapply = 4 * ww.numel / (wk["gn_apply"] * 1e-3) / 1e9
            wide[ww.name] = {
                "shape": [ww.N, ww.C] + ([ww.D] if ww.D != 1 else []) + [ww.H, ww.W],
                "layout": "NDHWC" if ww.D != 1 else "NHWC",
                "us_per_call": round(wms * 1e3, 2),
                "GB_s": round(ww.algorithmic_bytes / (wms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(ww.algorithmic_bytes / (wms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "apply_frac_of_peak": round(wapply / HBM_PEAK_GBS, 4),
                "kernels_us": {k: round(v * 1e3, 2) for k, v in wk.items()},
                "tile": {"A": plan["A"], "W": plan["W"], "slots": plan["slots"], "T": plan["T"]},
                "threads": plan["threads"],
            }
            del wx, wy

    extra = {}
    if not args.no_extra_shapes:
        for ew in EXTRA_WORKLOADS:
            log("extra shape %s silu=%d" % (ew.label(), ew.apply_silu))
            eb, eg, ebeta = make_inputs(ew)
            ex = device_tensor(torch, eb, dev).reshape(ew.N, ew.L, ew.C)
            ey = torch.empty_like(ex)
            egt, ebt = torch.from_numpy(eg).to(dev), torch.from_numpy(ebeta).to(dev)
            exp_, eyp = ctypes.c_void_p(ex.data_ptr()), ctypes.c_void_p(ey.data_ptr())
            egp, ebp = ctypes.c_void_p(egt.data_ptr()), ctypes.c_void_p(ebt.data_ptr())

            def estep(ew=ew, exp_=exp_, eyp=eyp, egp=egp, ebp=ebp):
                code = gn.gn_silu_rows(exp_, egp, ebp, eyp, ew.N, ew.L, ew.C, ew.G, ew.eps,
                                       int(ew.apply_silu), sh)
                if code != 0:
                    raise RuntimeError(gn.status_text(code))

            ems, _ = time_calls(torch, estep, args.steps, args.warmup, stream)
            ek = gn.profile_rows(ex, ew.G, egt, ebt, ew.eps, ew.apply_silu, ey, args.steps)
            extra[ew.name] = {
                "shape": [ew.N, ew.C, ew.H, ew.W] if ew.W != 1 else [ew.N, ew.H, ew.C],
                "layout": "NHWC" if ew.W != 1 else "rows (N, L, C)",
                "apply_silu": ew.apply_silu,
                "note": ew.note,
                "us_per_call": round(ems * 1e3, 2),
                "GB_s": round(ew.algorithmic_bytes / (ems * 1e-3) / 1e9, 1),
                "frac_of_peak": round(ew.algorithmic_bytes / (ems * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "kernels_us": {k: round(v * 1e3, 2) for k, v in ek.items()},
                "h200_us_context": H200_US.get(ew.name),
            }
            del ex, ey

    single = {}
    if not args.no_single_launch:
        for (sN, sL, sC) in SINGLE_LAUNCH_SHAPES:
            sG = 32
            plan = gn.plan_single_launch(sN, sL, sC, sG)
            log("single-launch shape (%d,%d,%d) %s" % (sN, sL, sC, plan))
            gen = torch.Generator(device="cpu").manual_seed(sN * 1000 + sC)
            sx = (torch.randn(sN, sL, sC, generator=gen) * 1.5 + 0.2).bfloat16().to(dev)
            sy = torch.empty_like(sx)
            sgt = (1 + 0.1 * torch.randn(sC, generator=gen)).to(dev)
            sbt = (0.1 * torch.randn(sC, generator=gen)).to(dev)
            sxp, syp = ctypes.c_void_p(sx.data_ptr()), ctypes.c_void_p(sy.data_ptr())
            sgp, sbp = ctypes.c_void_p(sgt.data_ptr()), ctypes.c_void_p(sbt.data_ptr())

            def sstep(sN=sN, sL=sL, sC=sC, sG=sG, sxp=sxp, syp=syp, sgp=sgp, sbp=sbp):
                code = gn.gn_silu_rows(sxp, sgp, sbp, syp, sN, sL, sC, sG, 1e-6, 1, sh)
                if code != 0:
                    raise RuntimeError(gn.status_text(code))

            sms, _ = time_calls(torch, sstep, max(args.steps, 100), args.warmup, stream)
            sk = gn.profile_rows(sx, sG, sgt, sbt, 1e-6, True, sy, args.steps)
            sbytes = 6 * sN * sL * sC
            single["rows_%dx%dx%d" % (sN, sL, sC)] = {
                "shape_rows": [sN, sL, sC], "groups": sG,
                "plan": plan,
                "us_per_call": round(sms * 1e3, 2),
                "GB_s": round(sbytes / (sms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(sbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "kernels_us": {k: round(v * 1e3, 2) for k, v in sk.items()},
            }
            del sx, sy

    resnet = {}
    if not args.no_resnet_block:
        for shp in RESNET_SHAPES:
            log("resnet block %s" % (shp,))
            resnet["x".join(str(v) for v in shp)] = resnet_block(torch, gn, dev, shp, args)

    if args.copy_calibration:
        log("copy calibration: 512 MiB device-to-device copy x5")
        src = torch.empty(256 * 1024 * 1024, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on host cores")
        cpu = cpu_baseline(w, x_bits, gamma, beta, args.cpu_budget_s)

    result = {
        "metric": "GB/s (algorithmic: 2 reads + 1 write of the bf16 tensor) and us/call, "
                  "NHWC bf16 GroupNorm+SiLU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_call": round(ms * 1e3, 2),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(H200_US[w.name] / (ms * 1e3), 3),
        "vs_baseline_note": "value / the pages' H200 Triton kernel on the same shape "
                            "(913.8 us = 1762.6 GB/s): another machine, context only",
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "shape_nchw": [w.N, w.C, w.H, w.W],
            "layout": "NHWC (channels-last)",
            "groups": w.G,
            "eps": w.eps,
            "apply_silu": True,
            "inputs": w.note + "; gamma~N(1,0.1), beta~N(0,0.1); seed %d" % w.seed,
            "compute": "bf16 in/out, fp32 statistics and transform",
            "bytes_per_call": w.algorithmic_bytes,
        },
        "roofline": {
            "kernel": "gn_apply",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": apply_bytes,
            "mean_launch_ms": round(apply_ms, 5),
            "achieved_is": "algorithmic bytes (one read + one write of the tensor) / the "
                           "kernel's mean duration: an effective rate, not measured HBM "
                           "bandwidth -- part of step 3's read of x is served by the 256 MB "
                           "Infinity Cache, which step 1 fills with the last cache's worth of x",
            "traffic_is": "FETCH_SIZE + WRITE_SIZE per launch, scaled by a plain copy: requests "
                          "the L2 sends toward memory, whether the Infinity Cache or HBM serves "
                          "them (this part exposes no memory-side counter), so it shows no "
                          "wasted re-reads but cannot split HBM from Infinity-Cache bytes",
            "whole_call": {
                "what": "the whole call (both kernels), algorithmic bytes (two reads + one "
                        "write) / event-timed ms_per_step",
                "achieved": round(value, 1),
                "frac": round(value / HBM_PEAK_GBS, 4),
                "cold_after_write_frac": per_call["cold_after_write"]["frac_of_peak_median"],
                "cold_after_read_frac": per_call["cold_after_read"]["frac_of_peak_median"],
            },
        },
        "kernels_ms": {k: round(v, 5) for k, v in kms.items()},
        "per_call": per_call,
        "cpu_baseline": cpu,
        "gpu_over_cpu": None if cpu is None else {
            "all_cores": round(value / cpu["value"], 1),
            "one_core": round(value / cpu["one_core"]["value"], 1)},
        "other_shapes": other,
        "other_dtypes": dtypes,
        "wide_shapes": wide,
        "extra_shapes": extra,
        "single_launch_shapes": single,
        "resnet_block": resnet,
        "wall_s_timed_region": round(wall, 4),
        "device": dict({"name": props.name, "cus": props.multi_processor_count,
                        "arch": getattr(props, "gcnArchName", "")},
                       **gn.device_info(dev.index or 0)),
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
