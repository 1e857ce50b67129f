"""gn_silu_rows_noalloc (the entry point for callers that cannot allocate)
against gn_silu_rows_dtype, through the C ABI.

Both run the same kernels with the same launch plan; only the scratch
differs (a fixed buffer compiled into the library against the stream's
allocated one), so the outputs must agree bit for bit -- stricter than the
oracle tolerance, which one case also checks.  The calls come in a row on one
stream, each smaller than or laid out differently from the one before, so a
call that read what the previous one left in the shared buffer (arrival
counters where that call kept partial sums) would show.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-2, 1.6e-2

# (N, L, C, G, dtype, silu): consecutive calls of one sequence.  64 MiB with
# the two-level arrival count, then a smaller late-finalize shape, then a
# fused shape whose counters sit where the first call kept partials, then
# fp32, fp16 without SiLU, and the many-groups path (separate finalize).
SEQUENCE = [
    (1, 65536, 512, 32, "bf16", 1),
    (2, 4096, 320, 32, "bf16", 1),
    (3, 65536, 512, 32, "bf16", 1),
    (1, 16384, 256, 32, "f32", 1),
    (2, 8192, 128, 16, "f16", 0),
    (1, 4096, 1024, 512, "bf16", 1),
    (1, 4096, 128, 32, "bf16", 1),
]
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
CODE = {"bf16": 0, "f16": 1, "f32": 2}


@pytest.fixture(scope="module")
def gn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import groupnorm_silu_normalization_amd as g
    return g


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make(N, L, C, dt, seed, dev):
    g = torch.Generator(device="cpu").manual_seed(seed)
    mean = torch.randn(C, generator=g)
    std = 0.5 + 1.5 * torch.rand(C, generator=g)
    x = (mean + std * torch.randn(N, L, C, generator=g)).to(TORCH_DT[dt]).to(dev)
    gamma = (1.0 + 0.1 * torch.randn(C, generator=g)).to(dev)
    beta = (0.1 * torch.randn(C, generator=g)).to(dev)
    return x, gamma, beta


def test_noalloc_matches_the_allocating_entry_bitwise(gn):
    dev = torch.device("cuda:0")
    s = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    outs = []
    for i, (N, L, C, G, dt, silu) in enumerate(SEQUENCE):
        print("case noalloc %d: N=%d L=%d C=%d G=%d %s silu=%d" % (i, N, L, C, G, dt, silu),
              flush=True)
        x, gamma, beta = make(N, L, C, dt, 900 + i, dev)
        ref = torch.empty_like(x)
        code = gn.gn_silu_rows_dtype(vp(x), vp(gamma), vp(beta), vp(ref), N, L, C, G, 1e-6, silu,
                                     CODE[dt], s)
        assert code == gn.GnStatus.OK, gn.status_text(code)
        y = torch.empty_like(x)
        code = gn.gn_silu_rows_noalloc(vp(x), vp(gamma), vp(beta), vp(y), N, L, C, G, 1e-6,
                                       silu, CODE[dt], s)
        assert code == gn.GnStatus.OK, gn.status_text(code)
        outs.append((x, gamma, beta, ref, y))
    torch.cuda.synchronize()
    for i, (x, gamma, beta, ref, y) in enumerate(outs):
        assert torch.equal(y.view(-1).view(torch.uint8), ref.view(-1).view(torch.uint8)), \
            "call %d of the sequence differs from gn_silu_rows_dtype" % i


def test_two_calls_in_a_row_second_smaller_against_the_oracle(gn, oracle):
    """A large call then a smaller one, queued back to back on one stream with
    no synchronisation between them: each equals gn_silu_rows_dtype bit for
    bit and the oracle within the parity tolerance."""
    from gn_inputs import bf16_bits_to_f32
    dev = torch.device("cuda:0")
    s = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    calls = [(1, 65536, 512, 32), (1, 4096, 128, 32)]
    res = []
    for i, (N, L, C, G) in enumerate(calls):
        print("case noalloc pair %d: N=%d L=%d C=%d G=%d" % (i, N, L, C, G), flush=True)
        x, gamma, beta = make(N, L, C, "bf16", 950 + i, dev)
        y = torch.empty_like(x)
        code = gn.gn_silu_rows_noalloc(vp(x), vp(gamma), vp(beta), vp(y), N, L, C, G, 1e-6, 1,
                                       0, s)
        assert code == gn.GnStatus.OK, gn.status_text(code)
        res.append((N, L, C, G, x, gamma, beta, y))
    torch.cuda.synchronize()
    for N, L, C, G, x, gamma, beta, y in res:
        ref_t = torch.empty_like(x)
        code = gn.gn_silu_rows_dtype(vp(x), vp(gamma), vp(beta), vp(ref_t), N, L, C, G, 1e-6, 1,
                                     0, s)
        assert code == gn.GnStatus.OK
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref_t.view(torch.int16))
        xb = x.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
        ref = oracle.gn_silu(xb, gamma.cpu().numpy(), beta.cpu().numpy(), N, L, C, G, 1e-6, 1)
        got = bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1))
        err = np.abs(got.astype(np.float64) - ref.reshape(-1))
        bad = int(np.count_nonzero(~(err <= ATOL + RTOL * np.abs(ref.reshape(-1)))))
        print("noalloc (%d,%d,%d): max|y-ref| = %.3e, violations %d" % (N, L, C, err.max(), bad),
              flush=True)
        assert bad == 0


def test_too_large_for_the_fixed_buffer_is_refused(gn):
    """A shape whose scratch exceeds the fixed buffer returns
    GN_SCRATCH_TOO_SMALL before any GPU work, with real device tensors."""
    dev = torch.device("cuda:0")
    s = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    N, L, C, G = 1, 65536, 4096, 4096
    assert gn.plan_rows(N, L, C, G)["scratch_bytes"] > gn.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(N, L, C, device=dev, dtype=torch.bfloat16)
    y = torch.full_like(x, 3.0)
    code = gn.gn_silu_rows_noalloc(vp(x), None, None, vp(y), N, L, C, G, 1e-6, 1, 0, s)
    assert code == gn.GnStatus.SCRATCH_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
