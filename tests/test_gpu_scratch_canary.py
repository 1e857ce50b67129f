"""Canaries around the library's scratch, checked after GPU calls.

The no-allocation entry point keeps its scratch in a fixed per-device buffer
whose address gn_noalloc_scratch reports, so the whole buffer can be filled
with a canary byte before a call and read back after it.  The layout of a
call's scratch is the one gn_plan_rows_dtype's scratch_bytes counts:
arrival counters (N * (288 if K1 >= 64 else 1) words, rounded up to 256
bytes), partial sums and partial squares (N*K1*G floats each), 3840 floats of
padding that the fused finalize may read past the squares but never writes,
then mean and rstd (N*G floats each).  After each call nothing past
scratch_bytes and nothing in the padding may have changed, and the arrival
counters are either back to zero (a call that counts arrivals) or untouched.  The calls are the
same kernels as the allocating entry points, writing at the same offsets from
their scratch base.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

CANARY = 0xA5
PAD_FLOATS = 15 * 256


@pytest.fixture(scope="module")
def gn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import groupnorm_silu_normalization_amd as g
    return g


def hip_runtime():
    """The HIP runtime already mapped in this process (torch's)."""
    with open("/proc/self/maps") as f:
        paths = sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    assert len(paths) == 1, paths
    hip = ctypes.CDLL(paths[0])
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    return hip


# (N, L, C, G): the fused finalize (two-level count), a separate finalize
# kernel, the late finalize, more groups than threads, fp32
CASES = [(1, 196608, 512, 32, 0), (1, 65536, 512, 32, 0), (1, 4096, 128, 32, 0),
         (1, 4096, 1024, 512, 0), (2, 40000, 256, 32, 2), (3, 70001, 128, 32, 0)]


@pytest.mark.parametrize("N,L,C,G,dt", CASES)
def test_scratch_canaries(gn, N, L, C, G, dt):
    dev = torch.device("cuda:0")
    hip = hip_runtime()
    base = ctypes.c_void_p()
    size = ctypes.c_int64()
    assert gn.gn_noalloc_scratch(0, ctypes.byref(base), ctypes.byref(size)) == 0
    assert size.value == gn.NOALLOC_SCRATCH_BYTES and base.value
    p = gn.plan_rows(N, L, C, G, dt)
    need = p["scratch_bytes"]
    K1 = p["K1"]
    words = N * (288 if K1 >= 64 else 1)
    arr = -(-4 * words // 256) * 256
    nparts = N * K1 * G
    assert need == arr + 4 * (2 * nparts + PAD_FLOATS + 2 * N * G) <= size.value
    print("case canary N=%d L=%d C=%d G=%d dt=%d need=%d K1=%d late=%d" % (
        N, L, C, G, dt, need, K1, p["late_finalize"]), flush=True)
    tdt = {0: torch.bfloat16, 2: torch.float32}[dt]
    gen = torch.Generator(device="cpu").manual_seed(N + L + C)
    x = torch.randn(N, L, C, generator=gen).to(tdt).to(dev)
    y = torch.empty_like(x)
    fill = torch.full((size.value,), CANARY, dtype=torch.uint8, device=dev)
    dump = torch.empty_like(fill)
    torch.cuda.synchronize()
    assert hip.hipMemcpy(base, ctypes.c_void_p(fill.data_ptr()), size.value, 3) == 0
    s = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for _ in range(2):
        code = gn.gn_silu_rows_noalloc(ctypes.c_void_p(x.data_ptr()), None, None,
                                       ctypes.c_void_p(y.data_ptr()), N, L, C, G, 1e-6, 1, dt, s)
        assert code == 0, gn.status_text(code)
    torch.cuda.synchronize()
    assert hip.hipMemcpy(ctypes.c_void_p(dump.data_ptr()), base, size.value, 3) == 0
    torch.cuda.synchronize()
    d = dump.cpu().numpy()
    assert np.all(d[need:] == CANARY), "written past the call's scratch (first at %d)" % (
        need + int(np.flatnonzero(d[need:] != CANARY)[0]))
    pad0 = arr + 8 * nparts
    assert np.all(d[pad0:pad0 + 4 * PAD_FLOATS] == CANARY), "the over-read padding was written"
    assert np.all(d[4 * words:arr] == CANARY), "written between the counters and the partials"
    # arrival counters: zero again where the call counted arrivals (cleared
    # before, reset by the kernels after), untouched where it did not
    cnt = d[:4 * words]
    assert np.all(cnt == 0) or np.all(cnt == CANARY), "arrival counters left non-zero"
    # the partial sums were written (not all canary): the call used this scratch
    assert not np.all(d[arr:arr + 8 * nparts] == CANARY)
    ref = torch.empty_like(x)
    assert gn.gn_silu_rows_dtype(ctypes.c_void_p(x.data_ptr()), None, None,
                                 ctypes.c_void_p(ref.data_ptr()), N, L, C, G, 1e-6, 1, dt, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(y.view(-1).view(torch.uint8), ref.view(-1).view(torch.uint8))
