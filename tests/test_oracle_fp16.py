"""Pins of the oracle's FP16 fast path for the 4/6 decision
(four_over_six = 2; NVFP4-RL blog, section 4, "The optimization": the
E2M1 x E4M3 products stay in FP16, where they are exact, and the target is
scaled down by the inverse token scale).

- The FP16 rounding matches an independent nearest-value search over every
  binary16 value, on every non-negative binary32 pattern below 2^16 and on
  strided windows above (tests/pins/pins.c).
- The blog's premise: every product g x e of an E2M1 value and a finite
  E4M3 value is exactly representable in FP16.
- Where every FP16 step is exact (power-of-two token scale, small integer
  multiples), the FP16 error equals the FP32 error divided by s^2 exactly.
- On the workloads, the FP16 choice agrees with the FP32 choice on all but
  about a thousandth of the blocks (the blog reports >99.97% on its own
  data); a mistake in the units, a sign or a dropped term disagrees on a
  large fraction.
- Codes and scales of each candidate are those of the exact path: where the
  two choices agree, the outputs are identical.
- A block with one nonzero element reduces to one term, (FP16(FP16(|x| *
  inv_s) - g e))^2, with numpy's IEEE binary16 conversion as the rounding.
"""
import ctypes
import math

import numpy as np
import pytest

import oracle
import workloads
from conftest import fnptr


def bits(f):
    return int(np.array([f], np.float32).view(np.uint32)[0])


def test_fp16_rounding_exhaustive_below_2_16(pins, olib):
    first = ctypes.c_uint32(0)
    bad = pins.pin_fp16(fnptr(olib, "oracle_fp16_rne"), 0, bits(65536.0), ctypes.byref(first))
    assert bad == 0, "first mismatch at pattern %#x" % first.value


def test_fp16_rounding_overflow_and_specials(pins, olib):
    first = ctypes.c_uint32(0)
    for lo in range(bits(65536.0), 0x7F800000, 0x00400000):
        bad = pins.pin_fp16(fnptr(olib, "oracle_fp16_rne"), lo, lo + 4095, ctypes.byref(first))
        assert bad == 0, "first mismatch at pattern %#x" % first.value
    assert oracle.fp16_rne(65519.99) == 65504.0
    assert math.isinf(oracle.fp16_rne(65520.0))  # the tie goes to the even pattern: infinity
    assert oracle.fp16_rne(-1.0009765625) == -1.0009765625
    assert oracle.fp16_rne(-3.0 * 2.0 ** -26) == -(2.0 ** -24)
    assert math.isnan(oracle.fp16_rne(float("nan")))
    assert math.isinf(oracle.fp16_rne(float("inf")))


def test_products_g_times_e_exact_in_fp16():
    for q in range(8):
        g = oracle.e2m1_value(q)
        for byte in range(0x7F):  # every finite non-negative E4M3 value
            p = g * oracle.e4m3_decode(byte)
            assert oracle.fp16_rne(p) == p, (q, byte)


def test_fp16_error_exact_case_matches_fp32_over_s_squared():
    # s = 2^-4 (inv_s = 16 exactly); x on a grid of 2^-5 with |x| <= 6.
    # y = 16 |x| and g e are exact in FP16 and so is every difference, so the
    # FP16 error is the FP32 error times 2^8, sum for sum.
    rng = np.random.default_rng(11)
    s = 2.0 ** -4
    for _ in range(200):
        x = (rng.integers(-192, 193, 16) / 32.0).astype(np.float32)
        x[rng.integers(16)] = 6.0
        b = oracle.nvfp4_block(x, s, 2)
        for k in range(2):
            assert b.err16[k] == np.float32(b.err[k] * 256.0), (x, k)
        want = 4 if b.err[1] < b.err[0] else 6
        assert b.choice == want


def test_fp16_error_in_units_of_s():
    # err16 is the error measured in units of s: err16 * s^2 tracks the FP32
    # error up to FP16 rounding of the target and the differences
    rng = np.random.default_rng(12)
    worst = 0.0
    for _ in range(400):
        s = float(np.float32(2.0 ** rng.uniform(-20, 10)))
        x = (rng.standard_normal(16) * s * rng.uniform(50, 1500)).astype(np.float32)
        x = np.clip(x, -1536 * s, 1536 * s).astype(np.float32)
        b = oracle.nvfp4_block(x, s, 2)
        for k in range(2):
            ref = b.err[k] / (s * s)
            if ref > 1e-3:
                worst = max(worst, abs(b.err16[k] - ref) / ref)
    assert worst < 0.02, worst


@pytest.mark.parametrize("name,nrows", [("tiny_ref", None), ("moe_act", 256),
                                        ("expert_weights", 256), ("ragged_routed", 1024)])
def test_fp16_choice_agreement_on_workloads(name, nrows):
    x = workloads.rows(name) if nrows is None else workloads.rows(name, 0, nrows)
    exact = oracle.nvfp4_quantize(x, 1, dequant=True)
    fast = oracle.nvfp4_quantize(x, 2, dequant=True)
    rows, hidden = x.shape
    # token scales are those of the exact path
    assert np.array_equal(exact[2].view(np.uint32), fast[2].view(np.uint32))
    same = (exact[1] == fast[1]) & (exact[0].reshape(rows, -1, 8) ==
                                    fast[0].reshape(rows, -1, 8)).all(-1)
    agree = same.mean()
    assert agree > 0.998, agree
    # a block that decides the same way is identical, dequant included
    dq_same = (exact[3].reshape(rows, -1, 16) == fast[3].reshape(rows, -1, 16)).all(-1)
    assert dq_same[same].all()
    # where the choices differ, each side is one of the two exact candidates:
    # the FP16 side's scale byte is the other candidate's byte
    rr, bb = np.nonzero(~same)
    for r, j in list(zip(rr, bb))[:20]:
        blk = oracle.nvfp4_block(
            (x[r, 16 * j:16 * j + 16].astype(np.uint32) << 16).view(np.float32), exact[2][r], 2)
        assert {int(exact[1][r, j]), int(fast[1][r, j])} == set(int(v) for v in blk.e_byte)


def test_single_element_blocks_reduce_to_one_fp16_term():
    rng = np.random.default_rng(13)
    checked = 0
    for _ in range(3000):
        s = np.float32(2.0 ** rng.uniform(-30, 20) * rng.uniform(1, 2))
        x = np.zeros(16, np.float32)
        mag = np.float32(s * rng.uniform(1, 1536))
        x[rng.integers(16)] = np.float32(-mag if rng.integers(2) else mag)
        x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)  # BF16 values
        b = oracle.nvfp4_block(x, float(s), 2)
        inv_s = np.float32(1) / np.float32(s)
        i = int(np.nonzero(x)[0][0])
        y = np.float16(np.abs(x[i]) * inv_s)
        for k in range(2):
            ge = np.float16(oracle.e2m1_value(b.code[k][i] & 7) * b.e[k])
            d = np.float16(y - ge)
            want = np.float32(np.float32(d) * np.float32(d))
            assert b.err16[k] == want, (x[i], s, k)
        checked += 1
    assert checked == 3000
