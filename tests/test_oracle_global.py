"""Pins of the oracle's global-scale NVFP4 (one FP32 scale per tensor, the
naive baseline the pages contrast with per-token scaling: humans& article,
section 1; NVFP4-RL blog, section 2):

- the scale is the tensor amax over 1536 (4/6 on) or 2688 (off);
- a one-row tensor, or rows that share the same amax, give exactly the
  per-token outputs;
- the pages' batch dependency: a row quantized next to a row with a larger
  amax changes, while per-token scaling leaves it untouched.
"""
import numpy as np
import pytest

import oracle
import workloads


def f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("fos", [1, 0, 2])
def test_scale_is_tensor_amax_over_constant(fos):
    x = workloads.rows("moe_act", 0, 16)
    amax = np.abs(f32(x)).max()
    _, _, ts, _ = oracle.nvfp4_quantize_global(x, fos)
    assert ts[0] == np.float32(amax) / np.float32(2688.0 if fos == 0 else 1536.0)


@pytest.mark.parametrize("fos", [1, 0, 2])
def test_single_row_and_equal_amax_match_per_token(fos):
    x = workloads.rows("moe_act", 0, 8)
    for sub in (x[:1], None):
        if sub is None:  # give every row the same amax
            sub = x.copy()
            sub[:, 0] = np.uint16(0x4300)  # 128.0, above every other value
        g = oracle.nvfp4_quantize_global(sub, fos)
        p = oracle.nvfp4_quantize(sub, fos)
        for k in (0, 1, 3):
            assert np.array_equal(g[k], p[k])
        assert (p[2] == g[2][0]).all()


def test_batch_dependency():
    x = workloads.rows("moe_act", 0, 2)
    amax = np.abs(f32(x)).max(1)
    small = int(np.argmin(amax))
    alone = oracle.nvfp4_quantize_global(x[small:small + 1])
    both = oracle.nvfp4_quantize_global(x)
    # the smaller-amax row changes when the other row joins the tensor ...
    assert not np.array_equal(alone[0][0], both[0][small])
    # ... while its per-token quantization does not
    p_alone = oracle.nvfp4_quantize(x[small:small + 1])
    p_both = oracle.nvfp4_quantize(x)
    assert np.array_equal(p_alone[0][0], p_both[0][small])
