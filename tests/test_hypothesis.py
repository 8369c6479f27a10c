"""Property tests over generated inputs (hypothesis, derandomized so every
run draws the same examples).  Tensors are small (1-4 rows of 1-6 blocks)
of finite BF16 values drawn from: any finite bit pattern, special values
(signed zeros, subnormals, the largest finite, E2M1 grid points and
midpoints), and moderate floats, under a per-tensor power-of-two gain.

CPU, on the oracle -- properties that hold exactly by the definitions:
  - rows are independent (per-token scaling): a tensor's outputs equal
    those of its rows quantized one at a time, in any order;
  - the fused dequant equals the standalone dequant of the outputs;
  - guided rounding toward the tensor's own codes under its own scales
    reproduces them;
  - a one-row tensor quantized with a global scale equals the per-token
    result;
  - Rollout-ResQ keeps exactly two codes of each group of four, at
    increasing positions, with magnitudes no smaller than the dropped
    ones', and the dense residual holds the kept codes at those positions.
GPU: every call bit-exact against the oracle on the same examples."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = dict(derandomize=True, deadline=None, database=None,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])

SPECIAL = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F,
           0x3E80, 0x3F00, 0x3F40, 0x3F80, 0x3FA0, 0x3FC0, 0x3FE0, 0x4000, 0x4020,
           0x4040, 0x4060, 0x4080, 0x40A0, 0x40C0, 0xC0C0, 0xBF80]


def _bf16(a):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


finite_pattern = st.integers(0, 0xFFFF).filter(lambda b: (b & 0x7F80) != 0x7F80)
moderate = st.floats(-100.0, 100.0, width=32).map(lambda f: int(_bf16(np.float32([f]))[0]))
element = st.one_of(finite_pattern, st.sampled_from(SPECIAL), moderate, moderate)


@st.composite
def tensors(draw, block=16, max_blocks=6):
    rows = draw(st.integers(1, 4))
    hidden = block * draw(st.integers(1, max_blocks))
    bits = np.array(draw(st.lists(element, min_size=rows * hidden, max_size=rows * hidden)),
                    np.uint16).reshape(rows, hidden)
    k = draw(st.integers(-40, 40))
    if k:
        x = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64) * 2.0 ** k
        big = 3.3895313892515355e38
        bits = _bf16(np.clip(x, -big, big).astype(np.float32))
    return bits


def _same(a, b):
    return all(np.array_equal(np.asarray(p).view(np.uint8), np.asarray(q).view(np.uint8))
               for p, q in zip(a, b) if p is not None)


# ------------------------------------------------------------- oracle (CPU) --

@settings(max_examples=150, **SETTINGS)
@given(tensors(), st.sampled_from([0, 1, 2]), st.randoms(use_true_random=False))
def test_rows_independent_and_dequant_consistent(x, fos, rnd):
    whole = oracle.nvfp4_quantize(x, fos)
    perm = list(range(x.shape[0]))
    rnd.shuffle(perm)
    for i in perm:
        one = oracle.nvfp4_quantize(x[i:i + 1], fos)
        assert _same([w[i:i + 1] for w in whole], one)
    back = oracle.nvfp4_dequantize(whole[0], whole[1], whole[2])
    assert np.array_equal(back, whole[3])


@settings(max_examples=100, **SETTINGS)
@given(tensors(), st.sampled_from([0, 1]))
def test_guided_by_own_codes_and_global_one_row(x, fos):
    codes, scales, ts, dq = oracle.nvfp4_quantize(x, fos)
    g = oracle.nvfp4_quantize_guided(x, codes, scales, ts)
    assert np.array_equal(g[0], codes) and np.array_equal(g[1], dq)
    row = x[:1]
    per = oracle.nvfp4_quantize(row, fos)
    glob = oracle.nvfp4_quantize_global(row, fos)
    assert glob[2].view(np.uint32)[0] == per[2].view(np.uint32)[0]
    assert _same([glob[0], glob[1], glob[3]], [per[0], per[1], per[3]])


@settings(max_examples=100, **SETTINGS)
@given(tensors(block=32, max_blocks=3))
def test_resq_two_of_four(x):
    c, s, rc, rm, rs = oracle.mxfp4_resq_quantize(x)
    dc, ds, drc, drs = oracle.mxfp4_resq_dense_quantize(x)
    assert np.array_equal(c, dc) and np.array_equal(s, ds) and np.array_equal(rs, drs)
    R, H = x.shape
    dense = np.stack([drc & 15, drc >> 4], -1).reshape(R, H // 4, 4)     # residual nibbles
    kept = np.stack([rc & 15, rc >> 4], -1).reshape(R, H // 4, 2)
    meta = np.stack([rm & 15, rm >> 4], -1).reshape(R, H // 4)
    i0, i1 = meta & 3, meta >> 2
    assert (i0 < i1).all()
    take = lambda idx: np.take_along_axis(dense, idx[..., None], -1)[..., 0]
    assert np.array_equal(kept[..., 0], take(i0)) and np.array_equal(kept[..., 1], take(i1))
    mag = dense & 7
    kept_min = np.minimum(take(i0) & 7, take(i1) & 7)
    dropped = np.where((np.arange(4) != i0[..., None]) & (np.arange(4) != i1[..., None]), mag, 0)
    assert (dropped.max(-1) <= kept_min).all()


# ----------------------------------------------------------- GPU vs oracle --

def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_block_quantization_amd as fq
    fq.lib()
    return fq


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _host(t):
    if t is None:
        return None
    t = t.cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).numpy()


@pytest.mark.gpu
@settings(max_examples=150, **SETTINGS)
@given(tensors(), st.sampled_from([0, 1, 2]), st.booleans())
def test_gpu_nvfp4_calls_match_oracle(x, fos, dequant):
    from gpuutil import Guards
    fq = _gpu()
    xd = _dev(x)
    R, H = x.shape
    gu = Guards()
    got = fq.nvfp4_quantize(xd, fos, dequant=dequant, out=gu.nvfp4(R, H, dequant))
    gu.check("nvfp4")
    want = oracle.nvfp4_quantize(x, fos, dequant=dequant)
    assert _same([_host(g) for g in got], want)
    back = fq.nvfp4_dequantize(*got[:3], out=gu.empty((R, H), torch.bfloat16))
    gd = fq.nvfp4_quantize_guided(xd, *got[:3], out=gu.guided(R, H))
    gout, ws = gu.global_(R, H)
    glob = fq.nvfp4_quantize_global(xd, fos, out=gout, workspace=ws)
    gu.check("dequant, guided, global")
    assert np.array_equal(_host(back).view(np.uint16), oracle.nvfp4_dequantize(*want[:3]))
    wg = oracle.nvfp4_quantize_guided(x, *want[:3])
    assert _same([_host(g) for g in gd], wg)
    assert _same([_host(g) for g in glob], oracle.nvfp4_quantize_global(x, fos))


@pytest.mark.gpu
@settings(max_examples=100, **SETTINGS)
@given(tensors(block=32, max_blocks=3))
def test_gpu_resq_calls_match_oracle(x):
    from gpuutil import Guards
    fq = _gpu()
    xd = _dev(x)
    R, H = x.shape
    gu = Guards()
    sp = fq.mxfp4_resq_quantize(xd, out=gu.mx(R, H))
    de = fq.mxfp4_resq_dense_quantize(xd, out=gu.mx_dense(R, H))
    gu.check("resq")
    wsp, wde = oracle.mxfp4_resq_quantize(x), oracle.mxfp4_resq_dense_quantize(x)
    assert _same([_host(g) for g in sp], wsp) and _same([_host(g) for g in de], wde)
    for mode, a, w in ((0, sp[:2] + (None, None, None), wsp[:2] + (None, None, None)),
                       (1, sp, wsp), (2, (de[0], de[1], de[2], None, de[3]),
                                      (wde[0], wde[1], wde[2], None, wde[3]))):
        xh = fq.mxfp4_resq_reconstruct(*a, residual=mode, out=gu.empty((R, H), torch.float32))
        gu.check("reconstruct %d" % mode)
        assert np.array_equal(_host(xh).view(np.uint32),
                              oracle.mxfp4_resq_reconstruct(*w, residual=mode).view(np.uint32))
