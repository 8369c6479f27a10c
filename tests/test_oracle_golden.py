"""The oracle reproduces the hand-worked blocks in tests/golden/ exactly."""
import numpy as np
import pytest

import oracle
from goldens import load

NV = load("nvfp4_worked_blocks.txt")
MX = load("mxfp4_resq_worked_block.txt")


@pytest.mark.parametrize("name", sorted(NV))
def test_nvfp4_worked_block(name):
    c = NV[name]
    x = c["x"][None, :]
    codes, scales, ts, dq = oracle.nvfp4_quantize(x, four_over_six=bool(c["four_over_six"]))
    assert ts.view(np.uint32)[0] == c["token_scale_bits"]
    np.testing.assert_array_equal(scales[0], c["scales"])
    np.testing.assert_array_equal(codes[0], c["codes"])
    np.testing.assert_array_equal(dq[0], c["dequant"])
    # the standalone dequant of the stored values gives the same BF16
    np.testing.assert_array_equal(oracle.nvfp4_dequantize(codes, scales, ts)[0], c["dequant"])
    if "err6" in c:
        x16 = (x[0, :16].astype(np.uint32) << 16).view(np.float32)
        blk = oracle.nvfp4_block(x16, ts[0], bool(c["four_over_six"]))
        assert blk.err[0] == np.float32(c["err6"])
        if "err4" in c:
            assert blk.err[1] == np.float32(c["err4"])


def test_mxfp4_resq_worked_block():
    c = MX["MX_first_group"]
    codes, scales, rc, rm, rs = oracle.mxfp4_resq_quantize(c["x"][None, :])
    np.testing.assert_array_equal(scales[0], c["scales"])
    np.testing.assert_array_equal(codes[0], c["codes"])
    np.testing.assert_array_equal(rs[0], c["res_scales"])
    np.testing.assert_array_equal(rc[0], c["res_codes"])
    np.testing.assert_array_equal(rm[0], c["res_meta"])
