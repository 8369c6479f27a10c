"""Helpers shared by the GPU tests: BF16 bit arrays <-> device tensors, the
oracle run over row chunks in threads (the oracle itself is single-threaded;
ctypes releases the GIL), and first-mismatch reporting."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

WORKERS = min(16, os.cpu_count() or 1)


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    return None if t is None else t.cpu().numpy()


def _chunks(rows, n):
    step = max(1, (rows + n - 1) // n)
    return [(a, min(rows, a + step)) for a in range(0, rows, step)]


def oracle_nvfp4(x_bits, four_over_six=True, dequant=True):
    rows = x_bits.shape[0]
    parts = _chunks(rows, WORKERS * 4)
    with ThreadPoolExecutor(WORKERS) as ex:
        res = list(ex.map(lambda ab: oracle.nvfp4_quantize(x_bits[ab[0]:ab[1]], four_over_six,
                                                           dequant=dequant), parts))
    out = []
    for k in range(4):
        if res[0][k] is None:
            out.append(None)
        else:
            out.append(np.concatenate([r[k] for r in res], 0))
    return tuple(out)


def oracle_mx(x_bits):
    rows = x_bits.shape[0]
    parts = _chunks(rows, WORKERS * 4)
    with ThreadPoolExecutor(WORKERS) as ex:
        res = list(ex.map(lambda ab: oracle.mxfp4_resq_quantize(x_bits[ab[0]:ab[1]]), parts))
    return tuple(np.concatenate([r[k] for r in res], 0) for k in range(5))


def oracle_mx_dense(x_bits):
    rows = x_bits.shape[0]
    parts = _chunks(rows, WORKERS * 4)
    with ThreadPoolExecutor(WORKERS) as ex:
        res = list(ex.map(lambda ab: oracle.mxfp4_resq_dense_quantize(x_bits[ab[0]:ab[1]]),
                          parts))
    return tuple(np.concatenate([r[k] for r in res], 0) for k in range(4))


def assert_same(got, want, name):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.nonzero(got.reshape(got.shape[0], -1) != want.reshape(want.shape[0], -1))
    if bad[0].size:
        r, c = bad[0][0], bad[1][0]
        raise AssertionError("%s: %d mismatches; first at row %d col %d: got %s want %s"
                             % (name, bad[0].size, r, c, hex(int(got.reshape(got.shape[0], -1)[r, c])),
                                hex(int(want.reshape(want.shape[0], -1)[r, c]))))


GUARD = 256      # bytes before and after every output
GUARD_FILL = 0xA5


class Guards:
    """Output tensors placed inside 0xA5-filled uint8 allocations with GUARD
    bytes on both sides (plus an optional extra offset in front), so that a
    store past either end of an output is seen by check()."""

    def __init__(self):
        self._bufs = []

    def empty(self, shape, dtype, offset=0):
        shape = tuple(int(d) for d in shape)
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((n + 2 * GUARD + offset,), GUARD_FILL, dtype=torch.uint8, device="cuda")
        o = GUARD + offset
        self._bufs.append((buf, o, n))
        return buf[o:o + n].view(dtype).view(shape)

    def nvfp4(self, rows, hidden, dequant=True):
        """(codes, block_scales, token_scales, dequant or None)."""
        return (self.empty((rows, hidden // 2), torch.uint8),
                self.empty((rows, hidden // 16), torch.uint8),
                self.empty((rows,), torch.float32),
                self.empty((rows, hidden), torch.bfloat16) if dequant else None)

    def global_(self, rows, hidden, dequant=True):
        """(codes, block_scales, tensor_scale, dequant or None), workspace."""
        out = self.nvfp4(rows, hidden, dequant)
        return (out[0], out[1], self.empty((1,), torch.float32), out[3]), \
            self.empty((1024,), torch.uint8)

    def mx(self, rows, hidden):
        return tuple(self.empty((rows, hidden // k), torch.uint8) for k in (2, 32, 4, 8, 32))

    def mx_dense(self, rows, hidden):
        return tuple(self.empty((rows, hidden // k), torch.uint8) for k in (2, 32, 2, 32))

    def guided(self, rows, hidden, dequant=True):
        return (self.empty((rows, hidden // 2), torch.uint8),
                self.empty((rows, hidden), torch.bfloat16) if dequant else None)

    def check(self, label=""):
        torch.cuda.synchronize()
        for buf, o, n in self._bufs:
            lo_ok = bool((buf[:o] == GUARD_FILL).all())
            hi_ok = bool((buf[o + n:] == GUARD_FILL).all())
            assert lo_ok and hi_ok, "%s: a guard byte around a %d-byte output was written (%s)" % (
                label, n, "before" if not lo_ok else "after")
