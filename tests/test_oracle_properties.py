"""Pins of the oracle's NVFP4 and MXFP4 pipelines by brute force, exact
arithmetic and invariants.

Nothing here retypes the oracle's FP32 formulas.  Each check derives the
expected answer another way -- exact double arithmetic, nearest-of-grid
search, torch's own format tables -- and allows disagreement only where the
pinned FP32 operation order legitimately decides (a value within a few ulps
of a rounding midpoint).  The MXFP4 path involves only exact power-of-two
scaling, so it is re-derived completely in double and compared bit-exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# E4M3FN values from torch's float8 type (independent of the oracle's decode)
E4M3 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E4M3_MID = (E4M3[1:] + E4M3[:-1]) / 2
GRID_MID = (GRID[1:] + GRID[:-1]) / 2


def as_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits_of_f32(a32):
    return torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def nearest_e4m3(t):
    """Index of the nearest E4M3 value, ties to the even byte, saturating."""
    t = np.minimum(t, 448.0)
    j = np.clip(np.searchsorted(E4M3, t, side="right") - 1, 0, 126)
    jn = np.minimum(j + 1, 126)
    dl, dh = t - E4M3[j], E4M3[jn] - t
    pick = np.where(dl < dh, j, np.where(dh < dl, jn, np.where(j % 2 == 0, j, jn)))
    return pick


def nearest_grid(v):
    """Nearest E2M1 code, ties to the even code, saturating at 6."""
    d = np.abs(v[..., None] - GRID)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among equals prefer an even code (ties sit between two codes)
    even = cand & (np.arange(8) % 2 == 0)
    return np.where(even.any(-1), np.argmax(even, -1), np.argmax(cand, -1))


def near(values, mids, rel):
    """True where a value lies within rel (relative) of any midpoint."""
    m = np.asarray(mids)
    return (np.abs(values[..., None] - m) <= rel * np.maximum(np.abs(m), 1e-300)).any(-1)


def property_rows(seed=7):
    """A mix of seeded rows: normal, heavy-tailed, outliers, scaled over a
    wide exponent range, and values placed on grid midpoints."""
    parts = [
        workloads.random_rows(seed, 300, 64),
        workloads.random_rows(seed + 1, 300, 128, dist=1, row_gain_sigma=2.0),
        workloads.random_rows(seed + 2, 300, 64, elem_p=0.02, elem_mult=60.0),
        workloads.random_rows(seed + 3, 200, 32, scale=2.0 ** -100),
        workloads.random_rows(seed + 4, 200, 32, scale=2.0 ** 100),
        workloads.random_rows(seed + 5, 100, 48, scale=2.0 ** -128),
    ]
    H = 64
    out = [p for p in parts if p.shape[1] == H]
    for p in parts:
        if p.shape[1] != H:  # re-tile to 64 columns
            flat = p.reshape(-1)
            n = flat.size // H
            out.append(flat[: n * H].reshape(n, H))
    # midpoint-heavy rows: row max 6 * 2^m, other values on grid midpoints
    rng = np.random.default_rng(seed)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 1.0, 3.0, 4.0])
    m = rng.choice(mids, size=(200, H)) * rng.choice([1, -1], size=(200, H))
    m[:, 0] = 6.0
    m *= 2.0 ** rng.integers(-20, 20, size=(200, 1))
    out.append(bf16_bits_of_f32(m.astype(np.float32)))
    return np.concatenate(out, 0)


ROWS = property_rows()


@pytest.mark.parametrize("fos", [True, False])
def test_nvfp4_brute_force_and_bounds(fos):
    x = ROWS
    xf = as_f64(x)
    codes, scales, ts, dq = oracle.nvfp4_quantize(x, four_over_six=fos)
    C = 1536.0 if fos else 2688.0
    amax = np.abs(xf).max(1)
    # token scale: the correctly rounded FP32 of amax / C
    np.testing.assert_array_equal(ts, (amax / C).astype(np.float32))

    R, H = x.shape
    nb = H // 16
    exceptions = {"code": 0, "scale": 0}
    checked_decisions = 0
    for r in range(R):
        s = float(ts[r])
        for j in range(nb):
            xb = xf[r, j * 16:(j + 1) * 16]
            blk = oracle.nvfp4_block(xb.astype(np.float32), s, fos)
            b = np.abs(xb).max()
            k_list = [6.0, 4.0] if fos else [6.0]
            exact_err = []
            tol = []
            for ki, K in enumerate(k_list):
                e = float(blk.e[ki])
                # (1) the block scale is the E4M3 nearest to b / (K s),
                #     except within 2^-20 of an E4M3 midpoint
                if b > 0 and s > 0:
                    T = b / (K * s)
                    want = nearest_e4m3(np.array([T]))[0]
                    if blk.e_byte[ki] != want:
                        assert near(np.array([T]), E4M3_MID, 2.0 ** -20)[0], (r, j, K, T)
                        exceptions["scale"] += 1
                else:
                    assert blk.e_byte[ki] == 0
                # the decode step is the FP32 product e*s (it rounds only
                # when the token scale is subnormal)
                d = float(np.float32(e * s))
                q = np.array(blk.code[ki][:]) & 7
                sign = np.array(blk.code[ki][:]) >> 3
                np.testing.assert_array_equal(sign, np.signbit(xb).astype(int))
                # (2) each magnitude code is the nearest grid point to |x|/d,
                #     except within 2^-20 of a grid midpoint
                if d >= 2.0 ** -128:
                    v = np.abs(xb) / d
                    wq = nearest_grid(v)
                    bad = wq != q
                    if bad.any():
                        assert near(v[bad], GRID_MID, 2.0 ** -20).all(), (r, j, K)
                        exceptions["code"] += int(bad.sum())
                elif d > 0:
                    # 1/d overflows FP32 to +inf: nonzero values saturate,
                    # zeros give 0 * inf = NaN, which rounds to code 0
                    np.testing.assert_array_equal(q, np.where(xb != 0, 7, 0))
                else:
                    assert (q == 0).all()
                # (3) FP32 candidate = exactly rounded signed g*e*s
                cand_exact = np.where(sign == 1, -1.0, 1.0) * GRID[q] * e * s
                np.testing.assert_array_equal(
                    np.array(blk.cand[ki][:], np.float32), cand_exact.astype(np.float32))
                # (4) error: the exact sum of squares within FP32 rounding
                delta = xb - cand_exact
                ee = float(np.sum(delta * delta))
                # relative FP32 rounding, plus up to 2^-150 absolute per
                # square and per sum when they fall in the subnormal range
                bound = (2.0 ** -19 * ee + 2.0 ** -23 * np.sum(np.abs(delta * cand_exact))
                         + 2.0 ** -46 * np.sum(cand_exact ** 2) + 40 * 2.0 ** -149)
                if not np.isfinite(blk.err[ki]):
                    # FP32 overflow of the squared error (|x| beyond ~2^63):
                    # the reading keeps FP32 arithmetic, so err is +inf
                    assert blk.err[ki] == np.inf and ee > 2.0 ** 127 * (1 - 2.0 ** -20), (r, j, K)
                    ee, bound = np.inf, 0.0
                else:
                    assert abs(float(blk.err[ki]) - ee) <= bound, (r, j, K)
                exact_err.append(ee)
                tol.append(bound)
                # (5) worst-case error bounds (humans& article section 3;
                #     NVFP4-RL blog section 4): 1/6 of the block max when
                #     mapping to 6, 1/8 when mapping to 4, widened by 17/16
                #     for E4M3's rounding of the scale (normal scales only)
                if e >= 2.0 ** -6 and d >= 2.0 ** -126 and e * s == d:
                    lim = (17.0 / 16.0) * b / (6.0 if K == 6.0 else 8.0)
                    assert np.abs(delta).max() <= lim * (1 + 2.0 ** -20), (r, j, K)
            # (6) the decision follows the exact errors outside the FP32 band
            if fos:
                if not np.isfinite(exact_err[0]) and not np.isfinite(exact_err[1]):
                    assert blk.choice == 6
                elif exact_err[1] + tol[1] < exact_err[0] - tol[0]:
                    assert blk.choice == 4
                    checked_decisions += 1
                elif exact_err[0] + tol[0] < exact_err[1] - tol[1]:
                    assert blk.choice == 6
                    checked_decisions += 1
                elif exact_err[0] == exact_err[1] and blk.err[0] == blk.err[1]:
                    assert blk.choice == 6  # ties, including both +inf, keep 6
            else:
                assert blk.choice == 6
            # (7) the row outputs carry the chosen candidate
            k = 1 if blk.choice == 4 else 0
            assert scales[r, j] == blk.e_byte[k]
            packed = np.array(blk.code[k][0::2]) | (np.array(blk.code[k][1::2]) << 4)
            np.testing.assert_array_equal(codes[r, j * 8:(j + 1) * 8], packed)
            np.testing.assert_array_equal(
                dq[r, j * 16:(j + 1) * 16],
                bf16_bits_of_f32(np.array(blk.cand[k][:], np.float32)))
    assert checked_decisions > 1000 or not fos
    # near-midpoint exceptions are allowed but must stay rare
    assert exceptions["code"] < 0.01 * R * H and exceptions["scale"] < 0.01 * R * nb


@pytest.mark.parametrize("fos", [True, False])
def test_dequant_fused_equals_standalone(fos):
    codes, scales, ts, dq = oracle.nvfp4_quantize(ROWS, four_over_six=fos)
    np.testing.assert_array_equal(oracle.nvfp4_dequantize(codes, scales, ts), dq)


def test_dequant_idempotence():
    """DQ(Q(DQ(Q(x)))) == DQ(Q(x)) bit for bit; codes are idempotent in
    6-only mode; with Four-Over-Six a re-quantized block may switch from 4
    to 6 only when both reproduce the same dequantized values (the tie
    keeps 6, as in worked block F)."""
    for fos in (True, False):
        c1, s1, t1, d1 = oracle.nvfp4_quantize(ROWS, four_over_six=fos)
        c2, s2, t2, d2 = oracle.nvfp4_quantize(d1, four_over_six=fos)
        np.testing.assert_array_equal(d2, d1)
        np.testing.assert_array_equal(t2, t1)
        if not fos:
            np.testing.assert_array_equal(c2, c1)
            np.testing.assert_array_equal(s2, s1)
        else:
            R, H = ROWS.shape
            blk_changed = (c1.reshape(R, H // 16, 8) != c2.reshape(R, H // 16, 8)).any(-1) | (s1 != s2)
            for r, j in zip(*np.nonzero(blk_changed)):
                b1 = oracle.nvfp4_block(as_f64(d1[r, j * 16:(j + 1) * 16]).astype(np.float32), t1[r], True)
                assert b1.choice == 6 and b1.err[0] == b1.err[1] == 0.0


def test_batch_invariance_and_permutation():
    """Per-token scaling (humans& article section 1; NVFP4-RL blog
    section 2): a row's outputs do not depend on the other rows."""
    x = ROWS[:400]
    full = oracle.nvfp4_quantize(x)
    perm = np.random.default_rng(3).permutation(x.shape[0])
    pf = oracle.nvfp4_quantize(x[perm])
    for a, b in zip(full, pf):
        np.testing.assert_array_equal(a[perm], b)
    for r in (0, 17, 399):
        alone = oracle.nvfp4_quantize(x[r:r + 1])
        for a, b in zip(full, alone):
            np.testing.assert_array_equal(a[r:r + 1], b)
    # scaling another row by a huge factor changes nothing in this one
    y = x.copy()
    y[1] = bf16_bits_of_f32((as_f64(x[1]) * 2.0 ** 60).astype(np.float32))
    other = oracle.nvfp4_quantize(y)
    for a, b in zip(full, other):
        np.testing.assert_array_equal(np.delete(a, 1, 0), np.delete(b, 1, 0))


def test_ragged_groups_equal_dense_and_leave_other_rows():
    x = ROWS[:300]
    offsets = np.array([5, 5, 40, 41, 200, 260], np.int64)
    dense = oracle.nvfp4_quantize(x)
    R, H = x.shape
    outs = (np.full((R, H // 2), 0xAB, np.uint8), np.full((R, H // 16), 0xCD, np.uint8),
            np.full((R,), -7.0, np.float32), np.full((R, H), 0x1234, np.uint16))
    oracle.nvfp4_quantize(x, offsets=offsets, outputs=outs)
    lo, hi = offsets[0], offsets[-1]
    for a, b, fill in zip(dense, outs, (0xAB, 0xCD, -7.0, 0x1234)):
        np.testing.assert_array_equal(b[lo:hi], a[lo:hi])
        assert (b[:lo] == fill).all() and (b[hi:] == fill).all()


def test_rejects_bad_arguments():
    x = ROWS[:4]
    with pytest.raises(ValueError):
        oracle.nvfp4_quantize(x[:, :24])  # hidden not a multiple of 16
    with pytest.raises(ValueError):
        oracle.nvfp4_quantize(x, offsets=np.array([0, 3, 2], np.int64))
    with pytest.raises(ValueError):
        oracle.nvfp4_quantize(x, offsets=np.array([0, 5], np.int64))
    with pytest.raises(ValueError):
        oracle.mxfp4_resq_quantize(x[:, :48])


# ---------------------------------------------------------------- MXFP4 ----

def mx_reference(xf):
    """MXFP4 + residual + 2:4 re-derived in exact double arithmetic."""
    R, H = xf.shape
    xb = xf.reshape(R, H // 32, 32)

    def quant(blocks):
        b = np.abs(blocks).max(-1)
        with np.errstate(divide="ignore"):
            k = np.where(b > 0, np.floor(np.log2(np.where(b > 0, b, 1.0))) - 2, -127)
        k = np.clip(k, -127, 127)
        v = np.abs(blocks) / np.exp2(k)[..., None]
        q = nearest_grid(v)
        sign = np.signbit(blocks).astype(np.int64)
        deq = np.where(sign == 1, -1.0, 1.0) * GRID[q] * np.exp2(k)[..., None]
        return k.astype(np.int64), q, sign, deq

    k, q, sg, deq = quant(xb)
    delta = xb - deq  # exact in double
    kr, qr, sr, _ = quant(delta)
    nib = (sg << 3) | q
    rnib = ((sr << 3) | qr).reshape(R, H // 4, 4)
    mag = rnib & 7
    # keep the two largest magnitudes of each group of 4, ties to lower index
    order = np.argsort(-mag, axis=-1, kind="stable")
    keep = np.sort(order[..., :2], axis=-1)
    i0, i1 = keep[..., 0], keep[..., 1]
    kept0 = np.take_along_axis(rnib, i0[..., None], -1)[..., 0]
    kept1 = np.take_along_axis(rnib, i1[..., None], -1)[..., 0]
    res_codes = (kept0 | (kept1 << 4)).astype(np.uint8)
    meta = (i0 | (i1 << 2)).reshape(R, H // 8, 2)
    res_meta = (meta[..., 0] | (meta[..., 1] << 4)).astype(np.uint8)
    nibf = nib.reshape(R, H)
    codes = (nibf[:, 0::2] | (nibf[:, 1::2] << 4)).astype(np.uint8)
    return (codes, (k + 127).astype(np.uint8), res_codes, res_meta,
            (kr + 127).astype(np.uint8), deq.reshape(R, H), delta.reshape(R, H))


def mx_rows():
    w = workloads.WORKLOADS["resq_act"]
    cm = workloads.channel_multipliers("resq_act")[:256]
    parts = [
        workloads.to_bf16_bits(workloads.fill_fp32(w["seed"], 0, 64, 256, col_mult=cm)),
        workloads.random_rows(21, 64, 256, dist=1, row_gain_sigma=3.0),
        workloads.random_rows(22, 64, 256, scale=2.0 ** -130),
        workloads.random_rows(23, 64, 256, scale=2.0 ** 120),
        workloads.random_rows(24, 64, 256, elem_p=0.05, elem_mult=1000.0),
    ]
    return np.concatenate(parts, 0)


def test_mxfp4_resq_matches_exact_rederivation():
    x = mx_rows()
    got = oracle.mxfp4_resq_quantize(x)
    want = mx_reference(as_f64(x))
    for name, g, w in zip(["codes", "scales", "res_codes", "res_meta", "res_scales"], got, want[:5]):
        np.testing.assert_array_equal(g, w, err_msg=name)


def test_mxfp4_resq_invariants():
    x = mx_rows()
    xf = as_f64(x)
    codes, scales, rc, rm, rs = oracle.mxfp4_resq_quantize(x)
    R, H = x.shape
    # decode primary
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(R, H)
    k = scales.astype(np.int64) - 127
    kf = np.repeat(k, 32, axis=1)
    deq = np.where(nib >> 3, -1.0, 1.0) * GRID[nib & 7] * np.exp2(kf)
    delta = xf - deq
    # the residual is exactly representable in FP32 (so FP32 subtraction is exact)
    assert (delta.astype(np.float32).astype(np.float64) == delta).all()
    # |delta| <= half the local grid step * 2^k for unclipped elements
    v = np.abs(xf) / np.exp2(kf)
    unclipped = v <= 6.0
    step = np.where(v < 2.0, 0.5, np.where(v < 4.0, 1.0, 2.0))
    assert (np.abs(delta)[unclipped] <= (step / 2 * np.exp2(kf))[unclipped]).all()
    # 2:4 structure: two distinct ascending indices per group
    meta = np.stack([rm & 15, rm >> 4], -1).reshape(R, H // 4)
    i0, i1 = meta & 3, meta >> 2
    assert (i0 < i1).all()
    # reconstruction error never exceeds the primary error
    kr = np.repeat(rs.astype(np.int64) - 127, 8, axis=1)  # per group
    lo, hi = rc & 15, rc >> 4
    recon = deq.copy().reshape(R, H // 4, 4)
    g = np.arange(H // 4)
    for idx, n in ((i0, lo), (i1, hi)):
        val = np.where(n >> 3, -1.0, 1.0) * GRID[n & 7] * np.exp2(kr)
        np.put_along_axis(recon, idx[..., None], np.take_along_axis(recon, idx[..., None], -1) + val[..., None], -1)
    recon = recon.reshape(R, H)
    assert (np.abs(xf - recon) <= np.abs(xf - deq)).all()
    # and improves it on the outlier-heavy rows overall
    assert np.sum((xf - recon) ** 2) < 0.6 * np.sum((xf - deq) ** 2)
