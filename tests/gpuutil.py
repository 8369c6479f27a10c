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
