"""GPU parity at the largest size class: a 300000 x 7168 BF16 tensor
(2,150,400,000 elements, 4.3 GB), past 2^31 elements and 2^32 input and
dequant bytes, so the element, byte and row indexing of every kernel runs
beyond 32 bits.

Rows are independent, so the oracle checks sampled rows bit for bit: the
first and last, the rows around the 2^31-element boundary, the rows where
the seeded pool below wraps, and seeded random rows -- for NVFP4 (4/6 and
dequant), MXFP4-ResQ sparse and dense, the three reconstructions, and the
global-scale call (whose oracle also gets the row holding the tensor max,
found on the host from the pool, so that both use the same tensor scale).  Properties that hold
at any size cover every element: the fused dequant equals the standalone
dequantizer, and guided rounding toward the tensor's own codes under its
own scales reproduces those codes (it is round-to-nearest then).

The tensor is built on the device from a seeded pool of 4099 heavy-tailed
rows (Student-t(3) times a per-row LogNormal(0, 0.5) gain): row r is pool
row r mod 4099 times 2^((7 r mod 17) - 8), an exact BF16 scaling, so a
kernel that read a neighbouring row would see different values.  The
oracle's inputs are the sampled rows read back from device memory."""
import numpy as np
import pytest
import torch

import fp4_block_quantization_amd as fq
import oracle
import workloads
from gpuutil import Guards, assert_same, bits_of, host, oracle_mx, oracle_mx_dense, oracle_nvfp4

pytestmark = pytest.mark.gpu

ROWS, HIDDEN, POOL = 300000, 7168, 4099


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()
    assert ROWS * HIDDEN > 2 ** 31 and 2 * ROWS * HIDDEN > 2 ** 32
    print("max-size: building %dx%d BF16 on the device" % (ROWS, HIDDEN), flush=True)
    pool_bits = workloads.to_bf16_bits(workloads.fill_fp32(11, 0, POOL, HIDDEN, dist=1,
                                                           scale=1.0, row_gain_sigma=0.5))
    pool = torch.from_numpy(pool_bits.view(np.int16)).view(torch.bfloat16).cuda()
    x = torch.empty((ROWS, HIDDEN), dtype=torch.bfloat16, device="cuda")
    step = 16384
    for r0 in range(0, ROWS, step):
        r = torch.arange(r0, min(ROWS, r0 + step), device="cuda", dtype=torch.int64)
        gain = torch.pow(2.0, ((7 * r) % 17 - 8).to(torch.float32)).to(torch.bfloat16)
        x[r0:r0 + r.numel()] = pool[r % POOL] * gain[:, None]
    del pool
    torch.cuda.synchronize()
    yield x, pool_bits
    del x
    torch.cuda.empty_cache()


def sample_rows():
    b = 2 ** 31 // HIDDEN  # the row holding element 2^31 (and input byte 2^32)
    fixed = [0, 1, POOL - 1, POOL, b - 1, b, b + 1, ROWS - 2, ROWS - 1]
    rng = np.random.default_rng(2026)
    return np.unique(np.concatenate([fixed, rng.integers(0, ROWS, 23)])).astype(np.int64)


def host_rows(t, idx):
    return t[torch.from_numpy(idx).cuda()]


def test_nvfp4_max_size_sampled_rows_and_dequant(big):
    x = big[0]
    idx = sample_rows()
    print("max-size nvfp4_quantize 4/6 + dequant, rows", idx.tolist(), flush=True)
    gu = Guards()
    codes, scales, ts, dq = fq.nvfp4_quantize(x, four_over_six=True, dequant=True,
                                              out=gu.nvfp4(ROWS, HIDDEN))
    gu.check("max-size nvfp4")
    x_bits = bits_of(host_rows(x, idx))
    want = oracle_nvfp4(x_bits, True, dequant=True)
    assert_same(host(host_rows(codes, idx)), want[0], "max-size codes")
    assert_same(host(host_rows(scales, idx)), want[1], "max-size block_scales")
    assert_same(host(host_rows(ts, idx))[:, None], want[2][:, None], "max-size token_scales")
    assert_same(bits_of(host_rows(dq, idx)), want[3], "max-size dequant")

    print("max-size nvfp4_dequantize over every element", flush=True)
    back = fq.nvfp4_dequantize(codes, scales, ts, out=gu.empty((ROWS, HIDDEN), torch.bfloat16))
    gu.check("max-size dequant")
    assert torch.equal(back.view(torch.int16), dq.view(torch.int16))
    del back, dq

    print("max-size nvfp4_quantize_guided toward its own codes", flush=True)
    gcodes, _ = fq.nvfp4_quantize_guided(x, codes, scales, ts, dequant=False,
                                         out=gu.guided(ROWS, HIDDEN, dequant=False))
    gu.check("max-size guided")
    assert torch.equal(gcodes, codes)


def test_mx_max_size_sampled_rows(big):
    x = big[0]
    idx = sample_rows()
    print("max-size mxfp4_resq_quantize, rows", idx.tolist(), flush=True)
    gu = Guards()
    got = fq.mxfp4_resq_quantize(x, out=gu.mx(ROWS, HIDDEN))
    gu.check("max-size mx")
    want = oracle_mx(bits_of(host_rows(x, idx)))
    for g, w, n in zip(got, want, ("codes", "scales", "res_codes", "res_meta", "res_scales")):
        assert_same(host(host_rows(g, idx)), w, "max-size mx " + n)


def test_dense_reconstruct_and_global_max_size(big):
    x, pool_bits = big
    idx = sample_rows()
    xs = bits_of(host_rows(x, idx))
    print("max-size mxfp4_resq_dense_quantize and mxfp4_resq_reconstruct", flush=True)
    gu = Guards()
    sp = fq.mxfp4_resq_quantize(x)
    de = fq.mxfp4_resq_dense_quantize(x, out=gu.mx_dense(ROWS, HIDDEN))
    gu.check("max-size dense")
    w_sp, w_de = oracle_mx(xs), oracle_mx_dense(xs)
    for g, w, n in zip(de, w_de, ("codes", "scales", "res_codes", "res_scales")):
        assert_same(host(host_rows(g, idx)), w, "max-size dense " + n)
    out = gu.empty((ROWS, HIDDEN), torch.float32)
    for mode, a, wa in ((0, (None, None, None), (None, None, None)),
                        (1, sp[2:], w_sp[2:]),
                        (2, (de[2], None, de[3]), (w_de[2], None, w_de[3]))):
        src = sp if mode != 2 else de
        fq.mxfp4_resq_reconstruct(src[0], src[1], *a, residual=mode, out=out)
        gu.check("max-size reconstruct %d" % mode)
        ws = w_sp if mode != 2 else w_de
        want = oracle.mxfp4_resq_reconstruct(ws[0], ws[1], *wa, residual=mode)
        assert_same(host(host_rows(out, idx)), want, "max-size reconstruct %d" % mode)
    del out, sp, de, g
    torch.cuda.empty_cache()

    # the tensor max, from the pool and the row gains on the host: the
    # oracle sees the sampled rows plus the row holding it, so its tensor
    # scale is the whole tensor's
    pool_amax = np.abs((pool_bits.astype(np.uint32) << 16).view(np.float32)).max(1)
    r = np.arange(ROWS)
    row_amax = pool_amax[r % POOL].astype(np.float64) * np.exp2((7 * r) % 17 - 8)
    top = int(np.argmax(row_amax))
    print("max-size nvfp4_quantize_global; tensor max in row %d" % top, flush=True)
    gu = Guards()
    out, ws = gu.global_(ROWS, HIDDEN)
    got = fq.nvfp4_quantize_global(x, True, dequant=True, out=out, workspace=ws)
    gu.check("max-size global")
    idx2 = np.unique(np.concatenate([idx, [top]]))
    want = oracle.nvfp4_quantize_global(bits_of(host_rows(x, idx2)), True)
    assert host(got[2]).view(np.uint32)[0] == want[2].view(np.uint32)[0], "tensor scale"
    assert_same(host(host_rows(got[0], idx2)), want[0], "max-size global codes")
    assert_same(host(host_rows(got[1], idx2)), want[1], "max-size global scales")
    assert_same(bits_of(host_rows(got[3], idx2)), want[3], "max-size global dequant")
