"""Calls larger than one launch: libfp4q built with a limit of 4096
work-items per launch (tests/gpu_probes/build.py) splits every call below
into many launches over consecutive rows or units; the results must still
equal the CPU oracle's bit for bit."""
import ctypes
import os

import numpy as np
import pytest
import torch

import fp4_block_quantization_amd as fq
import oracle
import workloads
from gpuutil import (assert_same, bits_of, host, oracle_mx, oracle_mx_dense, oracle_nvfp4,
                     to_dev)

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SPLIT_LIB = os.path.join(ROOT, "tests", "_build", "libfp4q_split4096.so")
vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(SPLIT_LIB):
        pytest.fail("split-launch library not built: run __graft_entry__.build()")
    return fq.declare(ctypes.CDLL(SPLIT_LIB))


def ptr(t):
    return None if t is None else t.data_ptr()


def stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("H", [32, 2048, 7168, 32768, 33024, 66048])
def test_nvfp4_split_launch(lib, H):
    # H = 32768: 16 waves a row, 4 rows a launch; H = 33024 takes the
    # one-wave-per-row kernel (more than 16 waves a row); H = 66048: one row
    # of the dequantizer is more work-items than this build's launch limit,
    # so every launch holds a single row
    rows = {32: 1000, 2048: 300, 7168: 67, 32768: 21, 33024: 150, 66048: 9}[H]
    rng = np.random.default_rng(H)
    x_bits = workloads.to_bf16_bits(rng.standard_t(3, (rows, H)).astype(np.float32) *
                                    np.exp(rng.standard_normal((rows, 1))).astype(np.float32))
    x = to_dev(x_bits)
    for fos in (True, False):
        codes = torch.empty((rows, H // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((rows, H // 16), dtype=torch.uint8, device="cuda")
        ts = torch.empty((rows,), dtype=torch.float32, device="cuda")
        dq = torch.empty_like(x)
        assert lib.nvfp4_quantize(ptr(x), rows, H, None, 0, int(fos), ptr(codes), ptr(scales),
                                  ptr(ts), ptr(dq), stream()) == 0
        back = torch.empty_like(x)
        assert lib.nvfp4_dequantize(ptr(codes), ptr(scales), ptr(ts), rows, H, ptr(back),
                                    stream()) == 0
        torch.cuda.synchronize()
        want = oracle_nvfp4(x_bits, fos)
        label = "split H=%d fos=%s" % (H, fos)
        assert_same(host(codes), want[0], label + " codes")
        assert_same(host(scales), want[1], label + " scales")
        assert_same(host(ts)[:, None], want[2][:, None], label + " token_scales")
        assert_same(bits_of(dq), want[3], label + " dequant")
        assert_same(bits_of(back), want[3], label + " standalone dequant")


def test_nvfp4_split_launch_ragged(lib):
    # a row range that starts and ends inside launches
    rows, H = 700, 2048
    x_bits = workloads.rows("ragged_routed", 0, rows)
    x = to_dev(x_bits)
    offs = torch.tensor([37, 100, 100, 650], dtype=torch.int64, device="cuda")
    codes = torch.full((rows, H // 2), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, H // 16), 0xCD, dtype=torch.uint8, device="cuda")
    ts = torch.full((rows,), -1.0, dtype=torch.float32, device="cuda")
    assert lib.nvfp4_quantize(ptr(x), rows, H, ptr(offs), 3, 1, ptr(codes), ptr(scales), ptr(ts),
                              None, stream()) == 0
    torch.cuda.synchronize()
    want = oracle_nvfp4(x_bits[37:650], True, dequant=False)
    c, s, t = host(codes), host(scales), host(ts)
    assert_same(c[37:650], want[0], "ragged codes")
    assert_same(s[37:650], want[1], "ragged scales")
    assert_same(t[37:650, None], want[2][:, None], "ragged token_scales")
    assert (c[:37] == 0xAB).all() and (c[650:] == 0xAB).all()
    assert (s[:37] == 0xCD).all() and (s[650:] == 0xCD).all()
    assert (t[:37] == -1.0).all() and (t[650:] == -1.0).all()


@pytest.mark.parametrize("H", [32, 7168])
def test_mx_split_launch(lib, H):
    rows = {32: 8192, 7168: 40}[H]
    x_bits = np.ascontiguousarray(workloads.rows("resq_act", 0, rows)[:, :H])
    x = to_dev(x_bits)
    kw = dict(dtype=torch.uint8, device="cuda")
    out = (torch.empty((rows, H // 2), **kw), torch.empty((rows, H // 32), **kw),
           torch.empty((rows, H // 4), **kw), torch.empty((rows, H // 8), **kw),
           torch.empty((rows, H // 32), **kw))
    assert lib.mxfp4_resq_quantize(ptr(x), rows, H, *[ptr(t) for t in out], stream()) == 0
    torch.cuda.synchronize()
    want = oracle_mx(x_bits)
    for g, w, n in zip(out, want, ("codes", "scales", "res_codes", "res_meta", "res_scales")):
        assert_same(host(g), w, "mx split H=%d %s" % (H, n))


def test_next_rows_split_launch(lib):
    """The guided, global-scale, dense-residual and reconstruction calls
    split into many launches too."""
    u8 = dict(dtype=torch.uint8, device="cuda")
    # TRACE guided rounding under a rollout's scales, 300 x 2048
    rows, H = 300, 2048
    x_bits = workloads.rows("moe_act", 0, rows)[:, :H].copy()
    roll = oracle_nvfp4(workloads.perturbed(x_bits, seed=5), True, dequant=False)
    x = to_dev(x_bits)
    g, bs, ts = (torch.from_numpy(a).cuda() for a in roll[:3])
    codes = torch.empty((rows, H // 2), **u8)
    dq = torch.empty_like(x)
    assert lib.nvfp4_quantize_guided(ptr(x), rows, H, ptr(g), ptr(bs), ptr(ts), ptr(codes),
                                     ptr(dq), stream()) == 0
    torch.cuda.synchronize()
    want = oracle.nvfp4_quantize_guided(x_bits, roll[0], roll[1], roll[2])
    assert_same(host(codes), want[0], "split guided codes")
    assert_same(bits_of(dq), want[1], "split guided dequant")
    # the same without a guide: round to nearest under the rollout's scales
    assert lib.nvfp4_quantize_guided(ptr(x), rows, H, None, ptr(bs), ptr(ts), ptr(codes),
                                     ptr(dq), stream()) == 0
    torch.cuda.synchronize()
    want = oracle.nvfp4_quantize_guided(x_bits, None, roll[1], roll[2])
    assert_same(host(codes), want[0], "split nearest codes")
    assert_same(bits_of(dq), want[1], "split nearest dequant")
    # one scale for the whole tensor, 67 x 7168
    rows, H = 67, 7168
    x_bits = workloads.rows("moe_act", 100, rows)
    x = to_dev(x_bits)
    codes = torch.empty((rows, H // 2), **u8)
    scales = torch.empty((rows, H // 16), **u8)
    tsc = torch.empty(1, dtype=torch.float32, device="cuda")
    dq = torch.empty_like(x)
    ws = torch.empty(fq.GLOBAL_WORKSPACE_BYTES, **u8)
    assert lib.nvfp4_quantize_global(ptr(x), rows, H, 1, ptr(codes), ptr(scales), ptr(tsc),
                                     ptr(dq), ptr(ws), stream()) == 0
    torch.cuda.synchronize()
    want = oracle.nvfp4_quantize_global(x_bits, True)
    assert_same(host(codes), want[0], "split global codes")
    assert_same(host(scales), want[1], "split global scales")
    assert_same(host(tsc)[None, :], want[2][None, :], "split global tensor scale")
    assert_same(bits_of(dq), want[3], "split global dequant")
    # Rollout-ResQ-Dense and the three reconstructions, 40 x 7168
    rows, H = 40, 7168
    x_bits = np.ascontiguousarray(workloads.rows("resq_act", 0, rows))
    x = to_dev(x_bits)
    dense = (torch.empty((rows, H // 2), **u8), torch.empty((rows, H // 32), **u8),
             torch.empty((rows, H // 2), **u8), torch.empty((rows, H // 32), **u8))
    assert lib.mxfp4_resq_dense_quantize(ptr(x), rows, H, *[ptr(t) for t in dense],
                                         stream()) == 0
    torch.cuda.synchronize()
    wd = oracle_mx_dense(x_bits)
    for gt, w, n in zip(dense, wd, ("codes", "scales", "res_codes", "res_scales")):
        assert_same(host(gt), w, "split dense " + n)
    ws = oracle_mx(x_bits)
    sparse = [torch.from_numpy(a).cuda() for a in ws]
    for mode, (rc, rm, rs) in ((0, (None, None, None)), (1, tuple(sparse[2:5])),
                               (2, (dense[2], None, dense[3]))):
        out = torch.empty((rows, H), dtype=torch.float32, device="cuda")
        assert lib.mxfp4_resq_reconstruct(ptr(sparse[0]), ptr(sparse[1]), ptr(rc), ptr(rm),
                                          ptr(rs), rows, H, mode, ptr(out), stream()) == 0
        torch.cuda.synchronize()
        wargs = {0: (None, None, None), 1: (ws[2], ws[3], ws[4]), 2: (wd[2], None, wd[3])}[mode]
        wh = oracle.mxfp4_resq_reconstruct(ws[0], ws[1], *wargs, residual=mode)
        assert_same(host(out), wh, "split reconstruct residual=%d" % mode)
