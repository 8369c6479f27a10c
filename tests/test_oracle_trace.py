"""Pins of the oracle's TRACE rollout-guided rounding ("TRACE FP4 RL --
Rollout-guided FP4 rounding", learnaivisually.com):

- the page's worked example (tests/golden/trace_worked_example.txt);
- guided by its own round-to-nearest codes, the guided rounding is
  round-to-nearest (the nearest codeword is one of the two neighbours);
- the guided code is always one of the two grid neighbours of v;
- under the rollout's scale, the guided codeword is never farther from the
  rollout's codeword than round-to-nearest's (the page's by-construction
  guarantee for the local gap).
"""
import os
import struct

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "trace_worked_example.txt")
GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)


def bf16(v):
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    assert u & 0xFFFF == 0
    return u >> 16


def cases():
    out, cur = {}, None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("[case "):
            cur = out.setdefault(line[6:-1], {})
            continue
        k, v = [t.strip() for t in line.split(":", 1)]
        cur[k] = float(v) if k.endswith("_x") else int(v)
    return out


def one(xv, guide_nibble):
    x = np.zeros((1, 16), np.uint16)
    x[0, 0] = bf16(xv)
    g = np.zeros((1, 8), np.uint8)
    g[0, 0] = guide_nibble
    codes, _ = oracle.nvfp4_quantize_guided(x, g, np.full((1, 1), 0x38, np.uint8),
                                            np.ones(1, np.float32))
    return int(codes[0, 0] & 15)


@pytest.mark.parametrize("name", sorted(cases()))
def test_page_worked_example(name):
    c = cases()[name]
    # with s = e = 1 the rollout's own rounding is round-to-nearest; a guide
    # equal to that code reproduces it
    assert one(c["rollout_x"], c["rollout_code"]) == c["rollout_code"]
    assert one(c["training_x"], c["training_rne_code"]) == c["training_rne_code"]
    assert one(c["training_x"], c["rollout_code"]) == c["training_guided_code"]


def nibbles(packed):
    return np.stack([packed & 15, packed >> 4], -1).reshape(packed.shape[0], -1)


def signed_value(nib):
    return np.where(nib & 8, -1.0, 1.0) * GRID[nib & 7]


def rne_and_neighbours(x_bits, scales, ts):
    """v = |x| * fl(1/fl(e s)) in FP32; nearest codes by the pinned E2M1
    primitive and the two neighbours by search in the grid."""
    rows, hidden = x_bits.shape
    x = (x_bits.astype(np.uint32) << 16).view(np.float32)
    e = np.array([oracle.e4m3_decode(int(b)) for b in range(256)], np.float32)[scales]
    d = (np.repeat(e, 16, 1) * ts[:, None]).astype(np.float32)
    with np.errstate(divide="ignore"):
        r = np.where(d != 0, np.float32(1) / d, np.float32(0)).astype(np.float32)
    v = (np.abs(x) * r).astype(np.float32).astype(np.float64)
    lo = np.searchsorted(GRID, v, side="right") - 1
    hi = np.minimum(np.where(GRID[lo] < v, lo + 1, lo), 7)
    return x, v, lo, hi


def test_self_guided_is_round_to_nearest_and_neighbours():
    x = workloads.rows("moe_act", 0, 32)
    codes, scales, ts, _ = oracle.nvfp4_quantize(x, 1, dequant=False)
    guided, _ = oracle.nvfp4_quantize_guided(x, codes, scales, ts, dequant=False)
    assert np.array_equal(guided, codes)
    # a guide of all +0 always picks the lower neighbour, all 6 the upper
    _, v, lo, hi = rne_and_neighbours(x, scales, ts)
    for fill, want in ((0x00, lo), (0x77, hi)):
        g, _ = oracle.nvfp4_quantize_guided(x, np.full_like(codes, fill), scales, ts,
                                            dequant=False)
        n = nibbles(g)
        sign = (x.astype(np.uint32) >> 15) & 1
        if fill == 0x77:  # a positive guide: negative values move toward it = lower
            want = np.where(sign == 1, lo, hi)
        assert np.array_equal(n & 7, want)
        assert np.array_equal(n >> 3, sign)


def test_guided_gap_never_larger_than_nearest():
    rng = np.random.default_rng(21)
    x = workloads.rows("moe_act", 0, 64)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    rc, scales, ts, _ = oracle.nvfp4_quantize(x, 1, dequant=False)   # the rollout
    # training side: the same values perturbed by about one BF16 step
    xt = workloads.to_bf16_bits(xf * (1 + rng.standard_normal(xf.shape).astype(np.float32)
                                      * np.float32(2.0 ** -8)))
    guided, _ = oracle.nvfp4_quantize_guided(xt, rc, scales, ts, dequant=False)
    xtf, v, lo, hi = rne_and_neighbours(xt, scales, ts)
    rne = np.array([[oracle.e2m1_code(float(a)) for a in row] for row in v.astype(np.float32)])
    sign = np.where(np.signbit(xtf), -1.0, 1.0)
    g = nibbles(guided)
    assert ((g & 7) == lo).__or__((g & 7) == hi).all()
    G = signed_value(nibbles(rc))
    gap_guided = np.abs(signed_value(g) - G)
    gap_rne = np.abs(sign * GRID[rne] - G)
    assert (gap_guided <= gap_rne).all()
    # and it closes most of the rounding flips
    assert (gap_guided > 0).sum() < (gap_rne > 0).sum()


# ----------------------------------------------- no guide: round to nearest --
# With no guide the call rounds each value to its nearest codeword under the
# given (rollout-side) scales: the training side's plain rounding that the
# TRACE page sets guided rounding against.

def one_nearest(xv):
    x = np.zeros((1, 16), np.uint16)
    x[0, 0] = bf16(xv)
    codes, _ = oracle.nvfp4_quantize_guided(x, None, np.full((1, 1), 0x38, np.uint8),
                                            np.ones(1, np.float32))
    return int(codes[0, 0] & 15)


@pytest.mark.parametrize("name", sorted(cases()))
def test_page_worked_example_round_to_nearest(name):
    # the page's round-to-nearest outcomes: 2.49 -> 2 for training, 2.51 -> 3
    # for the rollout (with s = e = 1, so v = |x|)
    c = cases()[name]
    assert one_nearest(c["training_x"]) == c["training_rne_code"]
    assert one_nearest(c["rollout_x"]) == c["rollout_code"]


@pytest.mark.parametrize("name,fos", [("moe_act", 1), ("tiny_ref", 1), ("tiny_ref", 0)])
def test_nearest_under_own_scales_reproduces_the_quantizer(name, fos):
    # the quantizer's codes are the round-to-nearest codes of the chosen
    # candidate's scale, so rounding a tensor under its own stored scales
    # gives back its codes and its dequant bit for bit
    x = workloads.rows(name, 0, 48)
    codes, scales, ts, dq = oracle.nvfp4_quantize(x, fos)
    got, gdq = oracle.nvfp4_quantize_guided(x, None, scales, ts)
    assert np.array_equal(got, codes)
    assert np.array_equal(gdq, dq)


def test_nearest_is_the_e2m1_rounding_of_v():
    # under the rollout's scales, perturbed training values: each code is the
    # pinned E2M1 rounding of v = |x| * fl(1/fl(e s)), with x's sign
    rng = np.random.default_rng(5)
    x = workloads.rows("moe_act", 0, 16)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    _, scales, ts, _ = oracle.nvfp4_quantize(x, 1, dequant=False)
    xt = workloads.to_bf16_bits(xf * (1 + rng.standard_normal(xf.shape).astype(np.float32)
                                      * np.float32(2.0 ** -8)))
    got, _ = oracle.nvfp4_quantize_guided(xt, None, scales, ts, dequant=False)
    xtf, v, lo, hi = rne_and_neighbours(xt, scales, ts)
    rne = np.array([[oracle.e2m1_code(float(a)) for a in row] for row in v.astype(np.float32)])
    n = nibbles(got)
    assert np.array_equal(n & 7, rne)
    assert np.array_equal(n >> 3, np.signbit(xtf).astype(n.dtype))
    # and the nearest code is one of the two neighbours, the nearer one
    assert (((n & 7) == lo) | ((n & 7) == hi)).all()
    dist = np.abs(GRID[n & 7] - v)
    assert (dist <= np.minimum(np.abs(GRID[lo] - v), np.abs(GRID[hi] - v)) + 0.0).all()
