"""Host checks of a claim the NVFP4 kernel's certified 4/6 decision rests
on: halving the exponent of a non-negative FP32 A through its bit pattern,
((bits(A) + 0x3F800001) >> 1), never falls below sqrt(A) for A < 2^64,
and stays within a factor 1.07 of it for normal A.  Exhaustive over the
subnormals and over two adjacent binades (the value is invariant under
A -> 4A for normal A, so one even and one odd exponent cover every normal
A), plus random patterns across the whole range.  Without the added one
the truncating shift falls below sqrt(A) just under the powers of four
(checked too)."""
import numpy as np


def bound(bits):
    return ((bits + np.uint32(0x3F800001)) >> np.uint32(1)).view(np.float32).astype(np.float64)


def check(bits, normal):
    a = bits.view(np.float32).astype(np.float64)
    r = np.sqrt(a)
    y = bound(bits)
    assert (y >= r).all()
    if normal:
        assert (y <= 1.07 * r).all()


def test_sqrt_bound_subnormals_and_zero():
    check(np.arange(0, 0x00800000, dtype=np.uint32), normal=False)


def test_sqrt_bound_two_binades():
    check(np.arange(0x3F000000, 0x40000000, dtype=np.uint32), normal=True)  # [0.5, 2)


def test_sqrt_bound_random_patterns():
    rng = np.random.default_rng(3)
    bits = rng.integers(0x00800000, 0x5F800000, 2_000_000, dtype=np.uint32)  # normal, < 2^64
    check(bits, normal=True)


def test_truncating_halving_is_not_a_bound():
    bits = np.arange(0x3F000000, 0x40000000, dtype=np.uint32)
    y = ((bits + np.uint32(0x3F800000)) >> np.uint32(1)).view(np.float32).astype(np.float64)
    assert (y < np.sqrt(bits.view(np.float32).astype(np.float64))).any()
