"""K0, the HBM probes (include/fp4q_membench.h), against torch on the GPU:
every copy mode moves the bytes exactly, the read/write mix writes the XOR
folds it names, the write probe writes its index pattern, and nothing lands
outside the destination (256 guard bytes on both sides)."""
import ctypes

import numpy as np
import pytest
import torch

from fp4_block_quantization_amd import _build

pytestmark = pytest.mark.gpu

GUARD = 256


@pytest.fixture(scope="module")
def M():
    L = ctypes.CDLL(_build.MEMBENCH_PATH)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.fp4q_k0_copy.argtypes = [vp, vp, i64, ci, vp]
    L.fp4q_k0_copy_stream.argtypes = [vp, vp, i64, ci, ci, vp]
    L.fp4q_k0_read.argtypes = [vp, i64, ci, ci, vp, vp]
    L.fp4q_k0_write.argtypes = [vp, i64, ci, vp]
    L.fp4q_k0_mix.argtypes = [vp, vp, i64, ci, ci, vp]
    return L


def guarded(nbytes):
    buf = torch.full((nbytes + 2 * GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
    return buf, buf[GUARD:GUARD + nbytes]


def guards_intact(buf, nbytes):
    return bool((buf[:GUARD] == 0xA5).all()) and bool((buf[GUARD + nbytes:] == 0xA5).all())


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def source(nbytes, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)


# whole 4 KiB wavefront chunks, a ragged tail, and more than one workgroup
SIZES = [16, 4096, 4096 * 5 + 48, (1 << 20) + 4096 * 3 + 16 * 7]


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_copy_modes(M, nbytes, mode):
    src = source(nbytes, nbytes + mode)
    buf, dst = guarded(nbytes)
    assert M.fp4q_k0_copy(ptr(src), ptr(dst), nbytes, mode, stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert guards_intact(buf, nbytes)


@pytest.mark.parametrize("mode", [1, 2])
def test_copy_stream(M, mode):
    nbytes = (1 << 20) + 4096 * 3 + 16 * 7
    src = source(nbytes, 7)
    buf, dst = guarded(nbytes)
    assert M.fp4q_k0_copy_stream(ptr(src), ptr(dst), nbytes, mode, 3, stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert guards_intact(buf, nbytes)


@pytest.mark.parametrize("divisor", [1, 2, 4])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_mix_writes_the_xor_folds(M, divisor, mode):
    nbytes = 4096 * 37
    src = source(nbytes, divisor * 3 + mode)
    buf, dst = guarded(nbytes // divisor)
    assert M.fp4q_k0_mix(ptr(src), ptr(dst), nbytes, divisor, mode, stream()) == 0
    torch.cuda.synchronize()
    # each wavefront: 4 KiB = 4 instructions x 64 lanes x 16 bytes; output
    # unit (i, lane) of a chunk is the XOR of input units i*D .. i*D + D - 1
    # of that lane
    s = src.view(37, 4, 64, 16).cpu().numpy()
    want = np.bitwise_xor.reduce(s.reshape(37, 4 // divisor, divisor, 64, 16), axis=2)
    assert np.array_equal(dst.cpu().numpy(), want.reshape(-1))
    assert guards_intact(buf, nbytes // divisor)


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("mode", [1, 2])
def test_write_pattern(M, nbytes, mode):
    buf, dst = guarded(nbytes)
    assert M.fp4q_k0_write(ptr(dst), nbytes, mode, stream()) == 0
    torch.cuda.synchronize()
    u = np.arange(nbytes // 16, dtype=np.uint32)
    want = np.stack([u, u + 1, u + 2, u + 3], -1).view(np.uint8).reshape(-1)
    assert np.array_equal(dst.cpu().numpy(), want)
    assert guards_intact(buf, nbytes)


@pytest.mark.parametrize("width", [1, 2, 4, 8, 16])
def test_read_leaves_the_sink(M, width):
    nbytes = 4096 * 9 + 16 * 3
    src = source(nbytes, width)
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    for nt in (0, 1):
        assert M.fp4q_k0_read(ptr(src), nbytes, width, nt, ptr(sink), stream()) == 0
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]
