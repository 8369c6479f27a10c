"""Quality reports of the oracle's Four-Over-Six choice, on the CPU.  The
asserts are the properties the pages state; the figures (printed with -s)
are quoted in the design notes.

1. SSE(4/6) against the best block scale.  For every 16-element block, the
   squared error of the 4/6 choice, of always mapping to 6, and of the best
   of all 126 positive finite E4M3 block scales under the same token scale
   (each with round-to-nearest codes), all in double.  The humans& article
   (section 3) and the NVFP4-RL blog (section 4) present 4/6 as a cheap way
   to pick a better block scale than always-6; the ratio SSE(4/6) /
   SSE(best) says how much of the room between always-6 and the best scale
   it takes.

2. Where the FP16 fast path's choice differs from the FP32 one (NVFP4-RL
   blog, section 4, "The optimization": > 99.97% agreement on its data).
   Every differing block is checked against a bound derived from FP16's
   11-bit rounding of the targets and differences (how far it can move each
   candidate's error), and for FP16-subnormal targets (|x| / s below
   2^-14, where FP16 keeps fewer bits).
"""
import numpy as np
import pytest

import oracle
import workloads

GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)


def f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def nearest_code(a):
    """Round-to-nearest E2M1 magnitude code of a >= 0 (ties to the even
    code, saturating): the number of grid midpoints below a, strict where
    the lower neighbour's code is even."""
    return ((a > 0.25).astype(np.int8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5)
            + (a >= 3.5) + (a > 5.0))


def e4m3_positive_values():
    return np.array([oracle.e4m3_decode(b) for b in range(1, 0x7F)], np.float64)


def sse_report(x_bits, fos=True):
    """Per-block SSE (double) of the oracle's choice, of always-6 under the
    same token scale, and of the best E4M3 block scale, summed."""
    rows, hidden = x_bits.shape
    codes, scales, ts, _ = oracle.nvfp4_quantize(x_bits, fos, dequant=False)
    x = f32(x_bits).astype(np.float64).reshape(rows, hidden // 16, 16)
    s = ts.astype(np.float64)[:, None, None]
    a = np.abs(x)
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(rows, hidden // 16, 16)
    e = np.array([oracle.e4m3_decode(int(b)) for b in range(256)], np.float64)[scales][..., None]
    chosen = np.where(nib & 8, -1.0, 1.0) * GRID[nib & 7] * e * s
    sse_choice = ((x - chosen) ** 2).sum(-1)
    best = np.full(sse_choice.shape, np.inf)
    for ev in e4m3_positive_values():
        d = ev * s
        with np.errstate(divide="ignore", invalid="ignore"):
            q = nearest_code(np.where(d > 0, a / d, 0.0))
        sse = ((a - GRID[q] * d) ** 2).sum(-1)
        best = np.minimum(best, sse)
    # always 6 under the same token scale (the oracle's own 6 candidate)
    sse6 = np.zeros(sse_choice.shape)
    for r in range(rows):
        for j in range(hidden // 16):
            blk = oracle.nvfp4_block(x[r, j].astype(np.float32), float(ts[r]), 1)
            c6 = np.array(blk.cand[0][:], np.float64)
            sse6[r, j] = ((x[r, j] - c6) ** 2).sum()
    zero = (a.max(-1) == 0)
    best = np.where(zero, 0.0, best)
    return {"blocks": int(sse_choice.size), "sse_4over6": float(sse_choice.sum()),
            "sse_always6": float(sse6.sum()), "sse_best_e4m3": float(best.sum()),
            "4over6_picks_best_frac": float(np.mean(sse_choice <= best * (1 + 1e-12)))}


@pytest.mark.parametrize("name,row0,nrows", [("tiny_ref", 0, 96), ("moe_act", 0, 24),
                                              ("expert_weights", 0, 24)])
def test_four_over_six_against_the_best_block_scale(name, row0, nrows):
    rep = sse_report(workloads.rows(name, row0, nrows))
    ratio = rep["sse_4over6"] / rep["sse_best_e4m3"]
    ratio6 = rep["sse_always6"] / rep["sse_best_e4m3"]
    print("\n[4/6 quality] %s rows %d-%d: %d blocks; SSE(4/6)/SSE(best) = %.4f, "
          "SSE(always 6)/SSE(best) = %.4f, 4/6 at the best scale in %.1f%% of blocks" % (
              name, row0, row0 + nrows, rep["blocks"], ratio, ratio6,
              100 * rep["4over6_picks_best_frac"]))
    # the best scale bounds both from below; 4/6 never does worse than 6
    # (it keeps 6 unless 4 is strictly better) and strictly better in total
    assert rep["sse_best_e4m3"] <= rep["sse_4over6"] * (1 + 1e-9)
    assert rep["sse_4over6"] < rep["sse_always6"]


def fp16_reach(x, c, s):
    """How far the FP16 path's error of one candidate (in x units, err16 s^2)
    can lie from the FP32 one: the target |x|/s and the difference y - g e
    are each rounded to FP16's 11 significant bits (relative 2^-11 each), so
    every difference moves by at most delta = 2^-11 (|x| + |x - c|)
    (1 + 2^-10) plus the FP32 roundings of 1/s and |x|/s (2^-22 |x|), and its
    square by 2 |x - c| delta + delta^2; the FP32 sums add 16 ulps."""
    d = np.abs(x - c)
    delta = 2.0 ** -11 * (np.abs(x) + d) * (1 + 2.0 ** -10) + 2.0 ** -22 * np.abs(x)
    err = (d * d).sum()
    return (2 * d * delta + delta * delta).sum() + 16 * 2.0 ** -24 * err


def decision_breakdown(x_bits):
    """Blocks whose FP16-path choice differs from the FP32 one, by cause."""
    rows, hidden = x_bits.shape
    c1, s1, ts, _ = oracle.nvfp4_quantize(x_bits, 1, dequant=False)
    c2, s2, _, _ = oracle.nvfp4_quantize(x_bits, 2, dequant=False)
    nb = hidden // 16
    same = (s1 == s2) & (c1.reshape(rows, nb, 8) == c2.reshape(rows, nb, 8)).all(-1)
    diff = np.argwhere(~same)
    x = f32(x_bits).reshape(rows, nb, 16)
    out = {"blocks": int(same.size), "differ": int(diff.shape[0]), "subnormal_targets": 0,
           "within_fp16_reach": 0, "rel_gaps": [], "gap_over_reach": []}
    for r, j in diff:
        blk = oracle.nvfp4_block(x[r, j], float(ts[r]), 2)
        e6, e4 = float(blk.err[0]), float(blk.err[1])
        xd = x[r, j].astype(np.float64)
        reach = sum(fp16_reach(xd, np.array(blk.cand[k][:], np.float64), float(ts[r]))
                    for k in (0, 1))
        out["rel_gaps"].append(abs(e4 - e6) / max(e4, e6))
        out["gap_over_reach"].append(abs(e4 - e6) / reach)
        y = np.abs(xd) / float(ts[r])
        if ((y > 0) & (y < 2.0 ** -14)).any():
            out["subnormal_targets"] += 1
        if abs(e4 - e6) <= reach:
            out["within_fp16_reach"] += 1
    return out


@pytest.mark.parametrize("name,nrows", [("tiny_ref", 256), ("moe_act", 512),
                                        ("expert_weights", 512)])
def test_fp16_decision_disagreements_are_within_fp16_reach(name, nrows):
    b = decision_breakdown(workloads.rows(name, 0, nrows))
    g = np.array(b["rel_gaps"]) if b["rel_gaps"] else np.zeros(1)
    q = np.array(b["gap_over_reach"]) if b["gap_over_reach"] else np.zeros(1)
    print("\n[fp16 decision] %s %d rows: %d of %d blocks differ (agreement %.4f%%); "
          "FP16-subnormal targets in %d; within the FP16 rounding's reach %d; relative gap "
          "of the two FP32 errors median %.2e max %.2e; gap / reach median %.3f max %.3f" % (
              name, nrows, b["differ"], b["blocks"], 100 * (1 - b["differ"] / b["blocks"]),
              b["subnormal_targets"], b["within_fp16_reach"], np.median(g), g.max(),
              np.median(q), q.max()))
    # every flipped decision is one that FP16's rounding of the targets and
    # differences can flip: the two FP32 errors are closer than it can move
    # them
    assert b["within_fp16_reach"] == b["differ"]
    assert b["subnormal_targets"] == 0
