"""GPU parity on a seeded sweep of random shapes and options: row lengths
from one block to past the one-wave-per-row limit, row counts that leave
partial workgroups, ragged group ranges, every 4/6 mode, with and without
the dequant, and row scales from 2^-140 to 2^100.  Every output is compared
with the CPU oracle bit for bit; rows outside a ragged range must keep their
sentinel bytes, and the 256 guard bytes around every output must stay
untouched."""
import numpy as np
import pytest
import torch

import fp4_block_quantization_amd as fq
import oracle
from gpuutil import (Guards, assert_same, bits_of, host, oracle_mx, oracle_mx_dense,
                     oracle_nvfp4, to_dev)

pytestmark = pytest.mark.gpu

MAX_ELEMENTS = 1 << 21


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()


def random_rows(rng, rows, hidden):
    """Rows of mixed distributions, each under its own power-of-two gain."""
    kind = rng.integers(0, 4, rows)
    x = np.empty((rows, hidden), np.float32)
    for r in range(rows):
        if kind[r] == 0:
            v = rng.standard_normal(hidden)
        elif kind[r] == 1:
            v = rng.standard_t(3, hidden)
        elif kind[r] == 2:
            v = rng.standard_normal(hidden)
            v[rng.integers(0, hidden, max(1, hidden // 64))] *= 100.0
        else:
            v = rng.choice(np.array([0.0, 0.25, 0.5, 0.75, 1.25, 2.5, 5.0, 6.0]), hidden)
            v *= rng.choice([-1.0, 1.0], hidden)
        x[r] = v * np.float32(2.0 ** rng.integers(-140, 100))
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def shape(rng, unit):
    # with 16-element blocks: 1280, 1665 and 2048 blocks are rows of 10, 14
    # and 16 waves, 2100 a long row
    hidden = unit * int(rng.choice([1, 2, 3, 7, 64, 100, 127, 128, 129, 448, 449, 1024, 1280,
                                    1665, 2048, 2100]))
    rows = int(rng.integers(1, max(2, min(300, MAX_ELEMENTS // hidden))))
    return rows, hidden


@pytest.mark.parametrize("case", range(24))
def test_nvfp4_random_shapes(case):
    rng = np.random.default_rng(1000 + case)
    rows, hidden = shape(rng, 16)
    fos = int(rng.integers(0, 3))
    dequant = bool(rng.integers(0, 2))
    x_bits = random_rows(rng, rows, hidden)
    x = to_dev(x_bits)
    lo, hi = 0, rows
    offsets = None
    if rows > 2 and rng.integers(0, 2):  # a ragged range of several groups
        cuts = np.sort(rng.integers(0, rows + 1, int(rng.integers(2, 6))))
        lo, hi = int(cuts[0]), int(cuts[-1])
        offsets = torch.from_numpy(cuts.astype(np.int64)).cuda()
    gu = Guards()
    out = gu.nvfp4(rows, hidden, dequant)
    for t, f in zip(out, (0xAB, 0xCD, -7.0, 1.5)):
        if t is not None:
            t.fill_(f)
    fq.nvfp4_quantize(x, fos, offsets=offsets, dequant=dequant, out=out)
    label = "case %d: %d x %d fos=%d dequant=%s rows [%d, %d)" % (
        case, rows, hidden, fos, dequant, lo, hi)
    gu.check(label)
    if hi > lo:
        want = oracle_nvfp4(x_bits[lo:hi], fos, dequant=dequant)
        assert_same(host(out[0])[lo:hi], want[0], label + " codes")
        assert_same(host(out[1])[lo:hi], want[1], label + " scales")
        assert_same(host(out[2])[lo:hi, None], want[2][:, None], label + " token scales")
        if dequant:
            assert_same(bits_of(out[3])[lo:hi], want[3], label + " dequant")
    for t, fill in zip(out[:3], (0xAB, 0xCD, -7.0)):
        h = host(t)
        assert (h[:lo] == fill).all() and (h[hi:] == fill).all(), label + " outside the range"
    if dequant:
        d = bits_of(out[3])
        assert (d[:lo] == 0x3FC0).all() and (d[hi:] == 0x3FC0).all(), label + " dequant outside"


@pytest.mark.parametrize("case", range(12))
def test_mx_random_shapes(case):
    rng = np.random.default_rng(2000 + case)
    rows, hidden = shape(rng, 32)
    x_bits = random_rows(rng, rows, hidden)
    x = to_dev(x_bits)
    label = "mx case %d: %d x %d" % (case, rows, hidden)
    gu = Guards()
    got = fq.mxfp4_resq_quantize(x, out=gu.mx(rows, hidden))
    dense = fq.mxfp4_resq_dense_quantize(x, out=gu.mx_dense(rows, hidden))
    gu.check(label)
    want = oracle_mx(x_bits)
    for g, w, n in zip(got, want, ("codes", "scales", "res_codes", "res_meta", "res_scales")):
        assert_same(host(g), w, label + " " + n)
    wd = oracle_mx_dense(x_bits)
    for g, w, n in zip(dense, wd, ("codes", "scales", "res_codes", "res_scales")):
        assert_same(host(g), w, label + " dense " + n)
    xh = fq.mxfp4_resq_reconstruct(*got, residual=1, out=gu.empty((rows, hidden), torch.float32))
    gu.check(label + " reconstruct")
    assert_same(host(xh), oracle.mxfp4_resq_reconstruct(*want, residual=1),
                label + " reconstruct")


@pytest.mark.parametrize("case", range(8))
def test_guided_random_shapes(case):
    rng = np.random.default_rng(3000 + case)
    rows, hidden = shape(rng, 16)
    x_bits = random_rows(rng, rows, hidden)
    guide = rng.integers(0, 256, (rows, hidden // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (rows, hidden // 16), dtype=np.uint8)
    ts = (np.abs(rng.standard_normal(rows)) *
          2.0 ** rng.integers(-140, 60, rows)).astype(np.float32)
    for gd in (guide, None):  # guided, and round to nearest under the scales
        gu = Guards()
        got = fq.nvfp4_quantize_guided(to_dev(x_bits),
                                       None if gd is None else torch.from_numpy(gd).cuda(),
                                       torch.from_numpy(scales).cuda(),
                                       torch.from_numpy(ts).cuda(), out=gu.guided(rows, hidden))
        label = "%s case %d: %d x %d" % ("guided" if gd is not None else "nearest", case, rows,
                                         hidden)
        gu.check(label)
        want = oracle.nvfp4_quantize_guided(x_bits, gd, scales, ts)
        assert_same(host(got[0]), want[0], label + " codes")
        assert_same(bits_of(got[1]), want[1], label + " dequant")


@pytest.mark.parametrize("case", range(8))
def test_nvfp4_full_size_random_tensors(case):
    """Full-size 8192 x 7168 tensors of four distributions (normal,
    Student-t(3), per-row log-normal gains, uniform on [-6, 6]) under a
    random power-of-two gain: about 3.7 million blocks each, of which a few
    thousand are near-ties between the two candidates."""
    rng = np.random.default_rng(50000 + case)
    R, H = 8192, 7168
    kind = case % 4
    if kind == 0:
        x = rng.standard_normal((R, H)).astype(np.float32)
    elif kind == 1:
        x = rng.standard_t(3, (R, H)).astype(np.float32)
    elif kind == 2:
        x = (rng.standard_normal((R, H)) * np.exp(rng.standard_normal((R, 1)) * 2)).astype(
            np.float32)
    else:
        x = rng.uniform(-6, 6, (R, H)).astype(np.float32)
    x *= np.float32(2.0 ** rng.integers(-30, 30))
    x_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    gu = Guards()
    label = "full-size case %d" % case
    got = fq.nvfp4_quantize(to_dev(x_bits), True, out=gu.nvfp4(R, H))
    gu.check(label)
    want = oracle_nvfp4(x_bits, True)
    assert_same(host(got[0]), want[0], label + " codes")
    assert_same(host(got[1]), want[1], label + " scales")
    assert_same(host(got[2])[:, None], want[2][:, None], label + " token scales")
    assert_same(bits_of(got[3]), want[3], label + " dequant")
