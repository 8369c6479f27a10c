"""Pins of the oracle's number-format primitives.

Each primitive is checked exhaustively (every binary32 pattern of the range
that matters) against an independent brute-force definition in
tests/pins/pins.c: nearest representable value computed exactly in double,
ties to the even code or mantissa.
"""
import ctypes
import math
import struct

import numpy as np
import torch

import oracle
from conftest import fnptr


def bits(f):
    return struct.unpack("<I", struct.pack("<f", f))[0]


def f32(u):
    return struct.unpack("<f", struct.pack("<I", u))[0]


def test_e2m1_exhaustive_0_to_8(pins, olib):
    # TRACE page, Jargon: E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 and
    # round-to-nearest; every FP32 value in [0, 8] (1.09e9 patterns).
    first = ctypes.c_uint32(0)
    bad = pins.pin_e2m1(fnptr(olib, "oracle_e2m1_code"), 0, bits(8.0),
                        ctypes.byref(first))
    assert bad == 0, "first mismatch at %#x" % first.value


def test_e2m1_saturation_and_specials():
    for v in [6.0, 6.5, 8.0, 1e3, 3.4e38, float("inf")]:
        assert oracle.e2m1_code(v) == 7
    assert oracle.e2m1_code(float("nan")) == 0
    # The TRACE worked example: 2.49 -> codeword 2, 2.51 -> codeword 3.
    assert oracle.e2m1_value(oracle.e2m1_code(2.49)) == 2.0
    assert oracle.e2m1_value(oracle.e2m1_code(2.51)) == 3.0
    assert [oracle.e2m1_value(q) for q in range(8)] == [0, .5, 1, 1.5, 2, 3, 4, 6]


def test_e4m3_exhaustive_0_to_1024(pins, olib):
    first = ctypes.c_uint32(0)
    bad = pins.pin_e4m3(fnptr(olib, "oracle_e4m3_encode"), 0, bits(1024.0),
                        ctypes.byref(first))
    assert bad == 0, "first mismatch at %#x" % first.value


def test_e4m3_saturation_above_1024(pins, olib):
    # Past 1024 every value saturates to 448 (0x7E); walk with a stride.
    for u in range(bits(1024.0), 0x7F800000, 4093):
        assert oracle.e4m3_encode(f32(u)) == 0x7E
    assert oracle.e4m3_encode(float("inf")) == 0x7E
    assert oracle.e4m3_encode(float("nan")) == 0
    assert oracle.e4m3_encode(-0.0) == 0


def test_e4m3_decode_roundtrip_and_torch():
    vals = [oracle.e4m3_decode(b) for b in range(127)]
    assert vals == sorted(vals) and len(set(vals)) == 127
    assert vals[0x7E] == 448.0 and vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6
    for b in range(127):
        assert oracle.e4m3_encode(vals[b]) == b
        assert oracle.e4m3_decode(b | 0x80) == -vals[b]
    assert math.isnan(oracle.e4m3_decode(0x7F))
    # torch's float8_e4m3fn is the same OCP format: compare the decode tables.
    tv = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    assert tv.tolist() == vals


def test_e4m3_matches_torch_cast_in_range():
    # torch's CPU cast to float8_e4m3fn rounds to nearest even (it does not
    # saturate, so only values <= 448 are compared).
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.uniform(0, 448, 200000), np.exp2(rng.uniform(-12, 8.8, 200000)),
    ]).astype(np.float32)
    x = x[x <= 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in x], np.uint8)
    assert (got == want).all()


def test_bf16_exhaustive_nonnegative(pins, olib):
    first = ctypes.c_uint32(0)
    bad = pins.pin_bf16(fnptr(olib, "oracle_bf16_rne"), 0, 0x7F7FFFFF,
                        ctypes.byref(first))
    assert bad == 0, "first mismatch at %#x" % first.value


def test_bf16_negative_range(pins, olib):
    first = ctypes.c_uint32(0)
    # negative normals around the largest finite, and all negative subnormals
    for lo, hi in [(0x80000000, 0x80FFFFFF), (0xFF000000, 0xFF7FFFFF),
                   (0xBF000000, 0xBFFFFFFF)]:
        bad = pins.pin_bf16(fnptr(olib, "oracle_bf16_rne"), lo, hi,
                            ctypes.byref(first))
        assert bad == 0, "first mismatch at %#x" % first.value


def test_bf16_matches_torch_sample():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2 ** 32, 300000, dtype=np.uint64).astype(np.uint32)
    u = u[(u & 0x7F800000) != 0x7F800000]
    x = u.view(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(v)) for v in x[:20000]], np.uint16)
    assert (got == want[:20000]).all()


def test_e8m0_subnormals_exhaustive_and_normals(pins, olib):
    first = ctypes.c_uint32(0)
    fn = fnptr(olib, "oracle_e8m0_exponent")
    assert pins.pin_e8m0(fn, 1, 0x007FFFFF, 1, ctypes.byref(first)) == 0, hex(first.value)
    assert pins.pin_e8m0(fn, 0x00800000, 0x7F7FFFFF, 509, ctypes.byref(first)) == 0, hex(first.value)
    # every BF16 magnitude exactly
    assert pins.pin_e8m0(fn, 0x00010000, 0x7F7F0000, 0x10000, ctypes.byref(first)) == 0, hex(first.value)
    assert oracle.e8m0_exponent(0.0) == -127
    assert oracle.e8m0_exponent(7.0) == 0 and oracle.e8m0_exponent(8.0) == 1
    assert oracle.e8m0_exponent(1.0) == -2


def test_product_table_exact_in_fp16_and_fp32():
    # NVFP4-RL blog section 4: an E2M1 x E4M3 product is exactly
    # representable in FP16 (<= 6 significant bits, 2^-10 .. 2688).
    for q in range(8):
        g = oracle.e2m1_value(q)
        for b in range(127):
            e = oracle.e4m3_decode(b)
            exact = g * e  # python float: exact for these few bits
            assert float(np.float32(g) * np.float32(e)) == exact
            assert float(np.float16(exact)) == exact
            if exact:
                m, _ = math.frexp(exact)
                assert (m * 64).is_integer()  # at most 6 significant bits


def test_scaled_encode_comparator_cpu(pins, olib):
    # The comparator behind the GPU pin of the scaled MX encode: it must
    # accept the codes of |a| * 2^-k computed here independently (nearest
    # grid value in float64, ties to the even code), skip inputs outside
    # |a| < 2^(k+3), and report a single planted wrong nibble at its index.
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    n = 1 << 18
    u = (np.arange(2 * n, dtype=np.uint64) << 13).astype(np.uint32)
    with np.errstate(invalid="ignore"):  # NaN patterns, skipped below
        a = u.view(np.float32).astype(np.float64)
    f = fnptr(olib, "oracle_e2m1_code")
    for k in (-127, -3, 0, 125):
        v = np.abs(a) * 2.0 ** -k
        inside = np.isfinite(a) & (np.abs(a) < 2.0 ** (k + 3))
        v = np.where(inside, v, 0.0)
        d = np.abs(v[:, None] - grid[None, :])
        q = np.argmin(d, axis=1)
        up = np.minimum(q + 1, 7)
        q = np.where((q % 2 == 1) & (d[np.arange(q.size), up] == d[np.arange(q.size), q]) & (q < 7),
                     up, q)
        nib = (q | ((u >> 31) << 3)).astype(np.uint8)
        got = np.ascontiguousarray(nib[0::2] | (nib[1::2] << 4))
        first = ctypes.c_uint64(0)
        assert pins.cmp_fp4_scaled(f, k, n, got.ctypes.data, ctypes.byref(first)) == 0, k
        i = int(np.nonzero(inside[0::2] & (q[0::2] > 0))[0][1000])
        got[i] ^= 1
        assert pins.cmp_fp4_scaled(f, k, n, got.ctypes.data, ctypes.byref(first)) == 1, k
        assert first.value == i


def test_reciprocal_comparator_cpu(pins):
    # The comparator behind the GPU pin of the refined reciprocal accepts
    # numpy's IEEE float32 quotients and reports one planted last-bit error
    # at its index.
    lo, n = bits(1.0) - 12345, 1 << 20
    d = (np.arange(n, dtype=np.uint64) + lo).astype(np.uint32).view(np.float32)
    got = np.ascontiguousarray((np.float32(1.0) / d).astype(np.float32))
    first = ctypes.c_uint64(0)
    assert pins.cmp_recip(lo, n, got.ctypes.data, ctypes.byref(first)) == 0
    got.view(np.uint32)[777] ^= 1
    assert pins.cmp_recip(lo, n, got.ctypes.data, ctypes.byref(first)) == 1
    assert first.value == 777
