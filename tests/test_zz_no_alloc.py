"""The allocation-free variant of the global-scale call,
nvfp4_quantize_global_noalloc, called through the C ABI: its kernels keep
the tensor-max pass's partial maxima in the library's own fixed device
array instead of a caller's workspace.  Its outputs must equal those of
nvfp4_quantize_global (which takes a workspace) bit for bit, on two calls
in a row on the same device, the second with a smaller tensor -- the
array then still holds the first call's partials, which must not leak into
the second result."""
import ctypes

import numpy as np
import pytest
import torch

import fp4_block_quantization_amd as fq
import workloads
from gpuutil import Guards, assert_same, bits_of, host, to_dev

pytestmark = pytest.mark.gpu

vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = fq.lib()
    lib.nvfp4_quantize_global_noalloc.argtypes = [vp, i64, i64, ci, vp, vp, vp, vp, vp]
    lib.nvfp4_quantize_global_noalloc.restype = ci
    return lib


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc(L, x, fos, stream=None):
    rows, hidden = x.shape
    gu = Guards()
    out = gu.nvfp4(rows, hidden)
    ts = gu.empty((1,), torch.float32)
    stream = torch.cuda.current_stream() if stream is None else stream
    st = L.nvfp4_quantize_global_noalloc(ptr(x), rows, hidden, fos, ptr(out[0]), ptr(out[1]),
                                         ptr(ts), ptr(out[3]), ctypes.c_void_p(stream.cuda_stream))
    assert st == 0, L.fp4q_status_string(st)
    gu.check("noalloc %dx%d" % (rows, hidden))
    return out[0], out[1], ts, out[3]


@pytest.mark.parametrize("fos", [1, 0, 2])
def test_noalloc_equals_the_workspace_call_twice(L, fos):
    # first a large tensor whose maximum sits in its last rows, then a
    # smaller one with a smaller maximum: stale partials from the first call
    # would raise the second call's tensor scale
    big = workloads.rows("moe_act", 0, 2048).copy()
    big[-1, -1] = 0x4580  # BF16 4096.0
    small = workloads.rows("moe_act", 4096, 300)
    for x_bits, label in ((big, "first call 2048x7168"), (small, "second call 300x7168")):
        x = to_dev(x_bits)
        got = noalloc(L, x, fos)
        want = fq.nvfp4_quantize_global(x, fos)
        torch.cuda.synchronize()
        assert_same(host(got[0]), host(want[0]), label + " codes")
        assert_same(host(got[1]), host(want[1]), label + " scales")
        assert_same(host(got[2])[None, :], host(want[2])[None, :], label + " tensor scale")
        assert_same(bits_of(got[3]), bits_of(want[3]), label + " dequant")
    # the second tensor's scale is its own maximum's, not the first's
    amax = np.abs((small.astype(np.uint32) << 16).view(np.float32)).max()
    assert host(got[2])[0] == np.float32(amax) / np.float32(1536 if fos else 2688)


def test_noalloc_on_a_created_stream(L):
    # a stream other than the NULL stream: the library finds the array on
    # the stream's device (a created stream at the default priority)
    x = to_dev(workloads.rows("moe_act", 0, 256))
    want = fq.nvfp4_quantize_global(x, 1)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = noalloc(L, x, 1, side)
    side.synchronize()
    for g, w, what in zip(got, want, ("codes", "scales", "tensor scale", "dequant")):
        g, w = (bits_of(g), bits_of(w)) if what == "dequant" else (host(g), host(w))
        if what == "tensor scale":
            g, w = g[None, :], w[None, :]
        assert_same(g, w, "side stream " + what)


def test_noalloc_rejects_like_the_workspace_call(L):
    s = ctypes.c_void_p(0)
    a16 = ctypes.c_void_p(0x10000)
    assert L.nvfp4_quantize_global_noalloc(a16, 4, 24, 1, a16, a16, a16, a16, s) == 2
    assert L.nvfp4_quantize_global_noalloc(None, 4, 64, 1, a16, a16, a16, a16, s) == 1
    assert L.nvfp4_quantize_global_noalloc(a16, 4, 64, 3, a16, a16, a16, a16, s) == 5
    assert L.nvfp4_quantize_global_noalloc(None, 0, 64, 1, None, None, None, None, s) == 0
