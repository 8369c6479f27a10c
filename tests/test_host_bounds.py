"""Host check of the claim the NVFP4 kernel's certified 4/6 decision rests
on: from A = sum over the block of (v - g)^2 (accumulated in FP32 with
fused multiply-adds) and the decode step D = fl(e s), the enclosure

    lo = D^2 (A (1 - 330u) - 260u)
    hi = D^2 (A (1 + 330u) + 260u),     u = 2^-24,

holds the candidate's FP32 squared error as the definition computes it,
for every row scale s in [2^-50, 2^40] (the rows the kernel certifies).
The error comes from the oracle (its per-block internals), A and the bounds
from the same FP32 operations the kernel performs, so an enclosure that
missed the definition's error on any block here would let the kernel take
a 4/6 decision the oracle does not.  Blocks: rows of three workloads, and
adversarial blocks (values near the E2M1 rounding midpoints, near the
saturation at 6, the largest and smallest scales of the range, one large
value among tiny ones).  The enclosure is also checked to be tight enough
to decide nearly every block of the workloads."""
import numpy as np

import oracle
import workloads

U = 2.0 ** -24
F = np.float32
E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)


def fma32(a, b, c):
    """FP32 fused multiply-add: a*b is exact in binary64 for FP32 operands;
    the one-ulp chance of a double rounding is far inside the bound's
    factor-of-two slack."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def enclosure(A, D):
    D2 = (D * D).astype(np.float32)
    hi = fma32(A, np.full_like(A, F(1 + 330 * U)), np.full_like(A, F(260 * U)))
    lo = fma32(A, np.full_like(A, F(1 - 330 * U)), np.full_like(A, F(-260 * U)))
    return (D2 * lo).astype(np.float32), (D2 * hi).astype(np.float32)


def blocks_with_internals(x, s):
    """x: FP32 [n, 16] (BF16 values), s: FP32 [n] row scales of each block.
    Returns e [n, 2], err [n, 2] and magnitude codes [n, 2, 16] from the
    oracle (candidate 0 maps to 6, 1 to 4)."""
    n = x.shape[0]
    e = np.zeros((n, 2), np.float32)
    err = np.zeros((n, 2), np.float32)
    q = np.zeros((n, 2, 16), np.int64)
    for i in range(n):
        b = oracle.nvfp4_block(x[i], s[i], 1)
        e[i] = b.e[:]
        err[i] = b.err[:]
        q[i] = np.array([list(b.code[0]), list(b.code[1])]) & 7
    return e, err, q


def check(x, s):
    e, err, q = blocks_with_internals(x, s)
    for k in range(2):
        ok = e[:, k] != 0
        D = (e[ok, k] * s[ok]).astype(np.float32)
        r = (F(1) / D).astype(np.float32)
        v = (np.abs(x[ok]) * r[:, None]).astype(np.float32)
        g = E2M1[q[ok, k]]
        a = (v - g).astype(np.float32)  # exact (Sterbenz, or g = 0)
        A = np.zeros(ok.sum(), np.float32)
        for i in range(16):
            A = fma32(a[:, i], a[:, i], A)
        lo, hi = enclosure(A, D)
        ek = err[ok, k]
        bad = ~((lo <= ek) & (ek <= hi))
        assert not bad.any(), (k, np.nonzero(bad)[0][:5], lo[bad][:3], ek[bad][:3], hi[bad][:3])


def rows_blocks(bits):
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    amax = np.abs(x).max(1)
    s = (amax / F(1536)).astype(np.float32)
    R, H = x.shape
    return x.reshape(R * H // 16, 16), np.repeat(s, H // 16)


def test_enclosure_holds_on_workload_rows():
    for name, rows in (("moe_act", 8), ("ragged_routed", 24), ("expert_weights", 8)):
        x, s = rows_blocks(workloads.rows(name, 0, rows))
        keep = (s >= 2.0 ** -50) & (s <= 2.0 ** 40)
        check(x[keep], s[keep])


def test_enclosure_holds_on_adversarial_blocks():
    rng = np.random.default_rng(11)
    mids = np.array([.25, .75, 1.25, 1.75, 2.5, 3.5, 5], np.float64)
    parts = []
    n = 1500
    for scale in (2.0 ** -50 * 1536 * 1.25, 1.0, 2.0 ** 40 * 1536 / 448 * 0.9):
        # near the rounding midpoints of the 6-candidate grid (b maps to 6)
        v = rng.choice(mids, (n, 16)) * (1 + rng.uniform(-2e-3, 2e-3, (n, 16)))
        v[:, 0] = 6.0
        parts.append(v * rng.choice([-1, 1], (n, 16)) * scale / 6)
        # uniform magnitudes up to the block max, mantissas random
        w = rng.uniform(0, 1, (n, 16))
        w[:, 1] = 1.0
        parts.append(w * scale)
        # one large value among tiny ones, and near-saturation values
        t = rng.uniform(0, 1e-3, (n, 16))
        t[:, 2] = 1.0
        parts.append(t * scale)
        parts.append(rng.uniform(0.9, 1.0, (n, 16)) * scale)
    x64 = np.concatenate(parts, 0)
    bits = workloads.to_bf16_bits(x64.astype(np.float32))
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    # row scale from a row amax somewhat above the block max (and equal to it)
    amax = np.abs(x).max(1) * rng.choice([1.0, 1.0, 3.0, 50.0], x.shape[0]).astype(np.float32)
    s = (amax.astype(np.float32) / F(1536)).astype(np.float32)
    keep = (s >= 2.0 ** -50) & (s <= 2.0 ** 40)
    assert keep.mean() > 0.95
    check(x[keep], s[keep])


def test_enclosure_decides_nearly_every_workload_block():
    # the two candidates' enclosures overlap (and the kernel falls back to
    # the exact errors) only for near-ties: at most 1e-3 of the blocks here
    x, s = rows_blocks(workloads.rows("moe_act", 0, 64))
    e, err, q = blocks_with_internals(x, s)
    los, his = [], []
    for k in range(2):
        D = (e[:, k] * s).astype(np.float32)
        r = np.where(D > 0, F(1) / np.where(D > 0, D, F(1)), F(0)).astype(np.float32)
        v = (np.abs(x) * r[:, None]).astype(np.float32)
        a = (v - E2M1[q[:, k]]).astype(np.float32)
        A = np.zeros(x.shape[0], np.float32)
        for i in range(16):
            A = fma32(a[:, i], a[:, i], A)
        lo, hi = enclosure(A, D)
        los.append(lo)
        his.append(hi)
    decided = (his[1] < los[0]) | (los[1] >= his[0])
    assert 1.0 - decided.mean() <= 1e-3
    # where decided, the enclosures agree with the definition's comparison
    four = err[:, 1] < err[:, 0]
    assert np.array_equal((his[1] < los[0])[decided], four[decided])
