"""Exhaustive GPU parity of the number-format conversions the kernels use
(fp4q_device.h) -- the gfx950 conversion instructions on the fast path and
the portable helpers on the rare paths -- against the CPU oracle's pinned
primitives.

The probe kernels (tests/gpu_probes/probes.hip) evaluate a conversion on
every binary32 pattern of a range; the host compares each result with the
oracle."""
import ctypes
import os
import struct

import numpy as np
import pytest
import torch

import oracle
from conftest import fnptr

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBES = os.path.join(ROOT, "tests", "_build", "libprobes.so")
CHUNK = 1 << 26  # result pairs per launch

HW_FP4, SW_FP4, HW_BF16, SW_BF16, HW_FP8, SW_FP8, HW_FP4_FLOOR, RECIP = range(8)


def bits(f):
    return struct.unpack("<I", struct.pack("<f", f))[0]


@pytest.fixture(scope="module")
def probes():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(PROBES):
        pytest.fail("probe library not built: run __graft_entry__.build()")
    L = ctypes.CDLL(PROBES)
    L.probe_launch.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64,
                               ctypes.c_void_p, ctypes.c_void_p]
    L.probe_launch.restype = ctypes.c_int
    L.probe_decode_tables.argtypes = [ctypes.c_void_p] * 5
    L.probe_decode_tables.restype = ctypes.c_int
    L.probe_decode_scaled.argtypes = [ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    L.probe_decode_scaled.restype = ctypes.c_int
    L.probe_encode_scaled.argtypes = [ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_void_p]
    L.probe_encode_scaled.restype = ctypes.c_int
    L.probe_amax_over_c.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.probe_amax_over_c.restype = ctypes.c_int
    return L


def run(probes, which, lo, flip, n, dtype):
    out = torch.empty(n, dtype=dtype, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert probes.probe_launch(which, lo, flip, n, ctypes.c_void_p(out.data_ptr()),
                               ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy()


def sweep(probes, pins, olib, which, cmp, fn_name, lo, hi, flip, dtype):
    """Compare every pattern in [lo, hi] (hi - lo + 1 even)."""
    total_bad = 0
    start = lo
    while start <= hi:
        n = min(CHUNK, (hi - start + 1) // 2)
        got = np.ascontiguousarray(run(probes, which, start, flip, n, dtype))
        first = ctypes.c_uint64(0)
        if cmp == "fp4":
            bad = pins.cmp_fp4(fnptr(olib, fn_name), start, flip, n, got.ctypes.data, ctypes.byref(first))
        else:
            bad = getattr(pins, "cmp_" + cmp)(fnptr(olib, fn_name), start, n, got.ctypes.data,
                                              ctypes.byref(first))
        assert bad == 0, "%s: %d mismatches, first pair at pattern %#x" % (
            cmp, bad, (start + 2 * first.value) ^ flip)
        total_bad += bad
        start += 2 * n
    return total_bad


@pytest.mark.parametrize("flip", [0, 0x80000000])
def test_e2m1_hw_conversion_exhaustive(probes, pins, olib, flip):
    # every FP32 value in [-8, 8]: code with the sign bit kept (also for
    # zeros and values that round to zero)
    sweep(probes, pins, olib, HW_FP4, "fp4", "oracle_e2m1_code", 0, bits(8.0) + 1, flip, torch.uint8)


def test_e2m1_hw_conversion_saturation(probes, pins, olib):
    for flip in (0, 0x80000000):
        for lo in range(bits(8.0) + 2, 0x7F800000, 0x00800000):
            sweep(probes, pins, olib, HW_FP4, "fp4", "oracle_e2m1_code", lo, lo + (1 << 16) - 1,
                  flip, torch.uint8)
    # +-inf saturate (the kernels feed +-inf only through the portable path)
    got = run(probes, HW_FP4, 0x7F7FFFFF, 0, 1, torch.uint8)[0]
    assert got == 0x77


def floor_sweep(probes, pins, lo, hi):
    start = lo
    while start <= hi:
        n = min(CHUNK, (hi - start + 1) // 2)
        got = np.ascontiguousarray(run(probes, HW_FP4_FLOOR, start, 0, n, torch.uint8))
        first = ctypes.c_uint64(0)
        bad = pins.cmp_fp4_floor(start, n, got.ctypes.data, ctypes.byref(first))
        assert bad == 0, "floor: %d mismatches, first pair at pattern %#x" % (
            bad, start + 2 * first.value)
        start += 2 * n


def test_e2m1_lower_neighbour_exhaustive(probes, pins):
    # the zero-seed stochastic-rounding conversion is the E2M1 floor: every
    # FP32 value in [0, 8], then strided windows up to +inf (code 7)
    floor_sweep(probes, pins, 0, bits(8.0) + 1)
    for lo in range(bits(8.0) + 2, 0x7F800000, 0x00800000):
        floor_sweep(probes, pins, lo, lo + (1 << 16) - 1)
    floor_sweep(probes, pins, 0x7F7FFFFE, 0x7F7FFFFF)
    floor_sweep(probes, pins, 0x7F7FFFFF, 0x7F800000)  # the largest finite and +inf


def test_bf16_hw_conversion_exhaustive(probes, pins, olib):
    sweep(probes, pins, olib, HW_BF16, "bf16", "oracle_bf16_rne", 0, 0xFFFFFFFF, 0, torch.int32)


def test_e4m3_hw_conversion_0_to_448(probes, pins, olib):
    # the kernels clamp the target scale to 448 before converting
    sweep(probes, pins, olib, HW_FP8, "fp8", "oracle_e4m3_encode", 0, bits(448.0) + 1, 0,
          torch.int16)


@pytest.mark.parametrize("flip", [0, 0x80000000])
def test_e2m1_device_helper_exhaustive(probes, pins, olib, flip):
    # every FP32 magnitude in [0, 8] (and its negative), sign bit kept
    sweep(probes, pins, olib, SW_FP4, "fp4", "oracle_e2m1_code", 0, bits(8.0) + 1, flip, torch.uint8)


def test_e2m1_device_helper_saturation_and_nan(probes, pins, olib):
    # (8, +inf]: strided windows up to the infinity pattern
    for lo in range(bits(8.0) + 2, 0x7F800000, 0x00800000):
        sweep(probes, pins, olib, SW_FP4, "fp4", "oracle_e2m1_code", lo, lo + (1 << 16) - 1, 0,
              torch.uint8)
    sweep(probes, pins, olib, SW_FP4, "fp4", "oracle_e2m1_code", 0x7F7FFFFE, 0x7F800000 - 1, 0,
          torch.uint8)
    # +inf saturates; NaN (0 * inf) gives code 0 like the oracle
    got = run(probes, SW_FP4, 0x7F800000, 0, 1, torch.uint8)[0]
    assert got & 15 == 7 and got >> 4 == 0


def test_bf16_device_helper_exhaustive(probes, pins, olib):
    # all 2^32 patterns (NaN inputs skipped)
    sweep(probes, pins, olib, SW_BF16, "bf16", "oracle_bf16_rne", 0, 0xFFFFFFFF, 0, torch.int32)


def test_e4m3_device_helper_exhaustive(probes, pins, olib):
    sweep(probes, pins, olib, SW_FP8, "fp8", "oracle_e4m3_encode", 0, bits(1024.0) + 1, 0,
          torch.int16)
    for lo in range(bits(1024.0) + 2, 0x7F800000, 0x00400000):
        sweep(probes, pins, olib, SW_FP8, "fp8", "oracle_e4m3_encode", lo, lo + 4095, 0,
              torch.int16)


def test_decode_tables(probes):
    t = [torch.empty(n, dtype=torch.float32, device="cuda") for n in (512, 512, 256, 256)]
    st = torch.cuda.current_stream().cuda_stream
    assert probes.probe_decode_tables(*[ctypes.c_void_p(x.data_ptr()) for x in t],
                                      ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    fp4_hw, fp4_sw, fp8_hw, fp8_sw = (x.cpu().numpy() for x in t)
    for b in range(256):
        for h in range(2):
            nib = (b >> (4 * h)) & 15
            g = oracle.e2m1_value(nib & 7)
            want = -g if nib & 8 else g
            for tab in (fp4_hw, fp4_sw):
                assert tab[2 * b + h] == want and np.signbit(tab[2 * b + h]) == bool(nib & 8)
        want8 = oracle.e4m3_decode(b)
        for tab in (fp8_hw, fp8_sw):
            if want8 != want8:
                assert tab[b] != tab[b]
            else:
                assert tab[b] == want8


def test_e2m1_scaled_decode_every_scale(probes):
    # The MXFP4 dequant: the scaled decode of every code byte under every
    # E8M0 scale k + 127 a finite BF16 block can give (passed as the FP32
    # pattern (k + 127) << 23; k = -127 is the all-zero pattern; the block max
    # is below 2^128, so k = floor(log2 b) - 2 <= 125) is +-g 2^k exactly,
    # FP32 subnormals and -0 included.
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    b = np.arange(256)
    codes = np.stack([b & 15, b >> 4], 1).reshape(-1)  # out[2b]: low nibble
    out = torch.empty(512, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for k in range(-127, 126):
        assert probes.probe_decode_scaled((k + 127) << 23, ctypes.c_void_p(out.data_ptr()), st) == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint32)
        want = (np.where(codes & 8, -1.0, 1.0) * np.ldexp(grid[codes & 7], k)).astype(np.float32)
        bad = np.nonzero(got != want.view(np.uint32))[0]
        assert len(bad) == 0, "k=%d: byte %d nibble %d got %#x want %#x" % (
            k, bad[0] // 2, bad[0] % 2, got[bad[0]], want.view(np.uint32)[bad[0]])


def test_e2m1_scaled_encode_every_scale(probes, pins, olib):
    # The MXFP4 encode divides by the block's power of two inside the
    # conversion: under the scale operand (k + 127) << 23 it must give the
    # oracle's code of |a| * 2^-k for every k in -127..125 and every input a
    # block with that exponent can hold (|a| < 2^(k+3)).  The inputs are
    # every binary32 pattern with its low 13 bits zero: each BF16 element,
    # and each residual x - g 2^k (a multiple of 2^(k-9) below 2^(k+1), so
    # of at most 10 significant bits), subnormals and -0 included.
    n = 1 << 18
    out = torch.empty(n, dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f = fnptr(olib, "oracle_e2m1_code")
    for k in range(-127, 126):
        assert probes.probe_encode_scaled((k + 127) << 23, n, ctypes.c_void_p(out.data_ptr()),
                                          st) == 0
        torch.cuda.synchronize()
        got = np.ascontiguousarray(out.cpu().numpy())
        first = ctypes.c_uint64(0)
        bad = pins.cmp_fp4_scaled(f, k, n, got.ctypes.data, ctypes.byref(first))
        assert bad == 0, "k=%d: %d mismatches, first pair at pattern %#x" % (
            k, bad, (2 * first.value) << 13)


def test_reciprocal_every_normal_divisor(probes, pins):
    # The reciprocal table of the NVFP4 quantizer: the refined hardware
    # reciprocal equals the IEEE quotient 1/d for every binary32 d in
    # [2^-126, 2^126] (2.1e9 values), the range the kernels use it on.
    lo, hi = bits(2.0 ** -126), bits(2.0 ** 126)
    start = lo
    while start <= hi:
        n = min(CHUNK, hi - start + 1)
        got = np.ascontiguousarray(run(probes, RECIP, start, 0, n, torch.float32))
        first = ctypes.c_uint64(0)
        bad = pins.cmp_recip(start, n, got.ctypes.data, ctypes.byref(first))
        assert bad == 0, "%d mismatches, first at pattern %#x" % (bad, start + first.value)
        start += n


def test_token_scale_every_bf16_amax(probes):
    # The token scale s = fl(amax / C) by product and FMA correction equals
    # the IEEE quotient (numpy's float32 division) for every non-negative
    # finite BF16 amax, for C = 2688 (6 only) and C = 1536 (Four-Over-Six).
    n = 0x7F80
    out = torch.empty(2 * n, dtype=torch.float32, device="cuda")
    assert probes.probe_amax_over_c(ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    a = (np.arange(n, dtype=np.uint32) << 16).view(np.float32)
    for half, c in ((0, 2688.0), (1, 1536.0)):
        want = (a / np.float32(c)).astype(np.float32).view(np.uint32)
        bad = np.nonzero(got[half * n:(half + 1) * n] != want)[0]
        assert len(bad) == 0, "C=%g: amax pattern %#x" % (c, int(bad[0]) << 16)
