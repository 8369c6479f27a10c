"""Pins of the oracle's Rollout-ResQ-Dense quantization and the
reconstruction X_hat = Q(X) (+ S(Q(dX)) or + Q(dX)) (HiFloat4 page,
Rollout-ResQ section), from what the mathematics fixes:

- dense and sparse calls share the primary codes, both scales, and the
  sparse call's kept residual codes are the dense codes at the kept
  positions;
- values on the MX grid reconstruct exactly with a zero residual;
- per element, dense residual error <= sparse residual error <= primary
  error (0 is a grid point, so rounding to the nearest grid point never
  moves away; S only zeroes), up to the one FP32 rounding of the sum;
- the dense error is at most 2 residual steps 2^kr: the residual block max
  scales into [4, 8), where the grid's worst case is saturation from just
  below 8 to 6;
- S keeps at most two residual values per group of four.
"""
import numpy as np

import oracle
import workloads


def as_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def nibbles(packed):
    return np.stack([packed & 15, packed >> 4], -1).reshape(packed.shape[0], -1)


def test_dense_and_sparse_share_everything_but_s():
    x = workloads.rows("resq_act", 0, 64)
    c, s, rc, rm, rs = oracle.mxfp4_resq_quantize(x)
    cd, sd, rcd, rsd = oracle.mxfp4_resq_dense_quantize(x)
    assert np.array_equal(c, cd) and np.array_equal(s, sd) and np.array_equal(rs, rsd)
    dense = nibbles(rcd).reshape(64, -1, 4)          # [rows, groups, 4]
    kept = nibbles(rc).reshape(64, -1, 2)            # [rows, groups, 2]
    meta = nibbles(rm).reshape(64, -1)               # [rows, groups]
    i0, i1 = meta & 3, meta >> 2
    assert (i0 < i1).all()
    g = np.arange(dense.shape[1])[None, :]
    r = np.arange(64)[:, None]
    assert np.array_equal(kept[..., 0], dense[r, g, i0])
    assert np.array_equal(kept[..., 1], dense[r, g, i1])
    # the kept two are the largest magnitudes, the earlier of equals first
    mag = dense & 7
    for a in range(4):
        dropped = (a != i0) & (a != i1)
        assert ((mag[r, g, a] <= np.minimum(mag[r, g, i0], mag[r, g, i1])) | ~dropped).all()


def test_grid_values_reconstruct_exactly():
    rng = np.random.default_rng(5)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    rows = []
    for k in (-126, -10, 0, 7, 100):
        v = rng.choice(grid, 64) * rng.choice([-1, 1], 64) * 2.0 ** k
        v[0], v[32] = 6 * 2.0 ** k, 4 * 2.0 ** k  # block maxima in [4, 8) * 2^k
        rows.append(v)
    xb = workloads.to_bf16_bits(np.array(rows, np.float32))
    x = as_f64(xb)
    c, s, rc, rm, rs = oracle.mxfp4_resq_quantize(xb)
    cd, sd, rcd, rsd = oracle.mxfp4_resq_dense_quantize(xb)
    assert (nibbles(rcd) & 7 == 0).all()
    for mode, args in ((0, (None, None, None)), (1, (rc, rm, rs)), (2, (rcd, None, rsd))):
        assert np.array_equal(oracle.mxfp4_resq_reconstruct(c, s, *args, residual=mode), x)


def test_error_ordering_and_dense_bound():
    for name, n in (("resq_act", 96), ("moe_act", 32), ("expert_weights", 32)):
        xb = workloads.rows(name, 0, n)
        x = as_f64(xb)
        c, s, rc, rm, rs = oracle.mxfp4_resq_quantize(xb)
        cd, sd, rcd, rsd = oracle.mxfp4_resq_dense_quantize(xb)
        hp = oracle.mxfp4_resq_reconstruct(c, s, residual=0).astype(np.float64)
        hs = oracle.mxfp4_resq_reconstruct(c, s, rc, rm, rs, residual=1).astype(np.float64)
        hd = oracle.mxfp4_resq_reconstruct(cd, sd, rcd, None, rsd, residual=2).astype(np.float64)
        ep, es, ed = np.abs(x - hp), np.abs(x - hs), np.abs(x - hd)
        ulp = np.spacing(np.abs(hs).astype(np.float32)).astype(np.float64)
        assert (ed <= es + ulp).all() and (es <= ep + ulp).all(), name
        step = np.repeat(2.0 ** (rsd.astype(np.float64) - 127), 32, axis=1)
        assert (ed <= 2 * step + ulp).all(), name
        assert np.mean(ed ** 2) <= np.mean(es ** 2) <= np.mean(ep ** 2)
        # S contributes at most two residual values per group of four
        contrib = (hs != hp).reshape(n, -1, 4).sum(-1)
        assert contrib.max() <= 2


def test_residual_recovers_underflowed_activations():
    # outlier channels force large block scales; most small values of those
    # blocks round to 0 in Q(X) and come back through the residual
    xb = workloads.rows("resq_act", 0, 64)
    x = as_f64(xb)
    c, s, rc, rm, rs = oracle.mxfp4_resq_quantize(xb)
    hp = oracle.mxfp4_resq_reconstruct(c, s, residual=0)
    hs = oracle.mxfp4_resq_reconstruct(c, s, rc, rm, rs, residual=1)
    mse_p, mse_s = np.mean((x - hp) ** 2), np.mean((x - hs) ** 2)
    assert mse_s < 0.1 * mse_p, (mse_p, mse_s)
