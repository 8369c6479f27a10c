"""The exact-decision build (libfp4q_exactdecision.so, the same sources
with -DFP4Q_NV_CERTIFY=0: every 4/6 block decided from both candidates'
errors computed by the definition) is a measurement variant: the bench
times it as the straightforward FP32 decision.  Its outputs must equal the
oracle's bit for bit, like the library's, so that it times the same
results: the edge suite at every kernel shape (split rows, the widest split
rows, the long-row kernel), moe_act rows and a ragged range, with guard
bytes around every output."""
import ctypes

import numpy as np
import pytest
import torch

import fp4_block_quantization_amd as fq
import workloads
from fp4_block_quantization_amd import _build
from gpuutil import Guards, assert_same, bits_of, host, oracle_nvfp4, to_dev
from test_gpu_parity import edge_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def E():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()
    return fq.declare(ctypes.CDLL(_build.EXACTDECISION_PATH))


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def run(E, x_bits, fos, offsets=None):
    x = to_dev(x_bits)
    R, H = x_bits.shape
    gu = Guards()
    out = gu.nvfp4(R, H)
    for t in out:  # rows outside a ragged range must stay as they were
        t.view(torch.uint8).fill_(0x5A)
    offs = None if offsets is None else torch.tensor(offsets, dtype=torch.int64, device="cuda")
    ng = 0 if offsets is None else len(offsets) - 1
    st = E.nvfp4_quantize(ptr(x), R, H, ptr(offs), ng, fos, *[ptr(t) for t in out],
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, E.fp4q_status_string(st)
    gu.check("exact-decision %dx%d" % (R, H))
    return out


def compare(out, x_bits, fos, label, lo=0, hi=None):
    hi = x_bits.shape[0] if hi is None else hi
    want = oracle_nvfp4(x_bits[lo:hi], fos)
    assert_same(host(out[0])[lo:hi], want[0], label + " codes")
    assert_same(host(out[1])[lo:hi], want[1], label + " block_scales")
    assert_same(host(out[2])[lo:hi, None], want[2][:, None], label + " token_scales")
    assert_same(bits_of(out[3])[lo:hi], want[3], label + " dequant")


@pytest.mark.parametrize("H", [16, 1040, 2048, 7168, 8208, 32768, 32784])
@pytest.mark.parametrize("fos", [1, 0])
def test_exact_decision_build_edge_suite(E, H, fos):
    x_bits = edge_rows(H, seed=H + 7)
    compare(run(E, x_bits, fos), x_bits, fos, "exact-decision edge H=%d fos=%d" % (H, fos))


def test_exact_decision_build_moe_act_rows(E):
    x_bits = workloads.rows("moe_act", 1000, 512)
    compare(run(E, x_bits, 1), x_bits, 1, "exact-decision moe_act rows")


def test_exact_decision_build_ragged_range(E):
    x_bits = workloads.rows("ragged_routed", 0, 300)
    out = run(E, x_bits, 1, offsets=[17, 40, 40, 233])
    compare(out, x_bits, 1, "exact-decision ragged", 17, 233)
    codes = host(out[0])
    assert (codes[:17] == 0x5A).all() and (codes[233:] == 0x5A).all()
