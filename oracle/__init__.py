"""CPU oracle of the fused FP4 block quantizer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps the plain single-threaded C reference in
fp4_oracle.c (which cites the pages it follows) with numpy-level helpers.
It shares no code with the GPU library and never imports it.

BF16 tensors travel as numpy uint16 arrays of their bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        path = os.environ.get("FP4Q_ORACLE_LIB")  # a test may load another build
        if path is None:
            if not os.path.exists(_build.LIB_PATH):
                _build.build()
            path = _build.LIB_PATH
        L = ctypes.CDLL(path)
        c_f = ctypes.c_float
        c_i64 = ctypes.c_int64
        vp = ctypes.c_void_p
        L.oracle_e2m1_code.argtypes = [c_f]
        L.oracle_e2m1_code.restype = ctypes.c_int
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_e2m1_value.restype = c_f
        L.oracle_e4m3_encode.argtypes = [c_f]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = c_f
        L.oracle_bf16_rne.argtypes = [c_f]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_e8m0_exponent.argtypes = [c_f]
        L.oracle_e8m0_exponent.restype = ctypes.c_int
        L.oracle_fp16_rne.argtypes = [ctypes.c_double]
        L.oracle_fp16_rne.restype = ctypes.c_double
        L.oracle_nvfp4_block.argtypes = [vp, c_f, ctypes.c_int, vp]
        L.oracle_nvfp4_block.restype = None
        L.nvfp4_quantize_ref.argtypes = [vp, c_i64, c_i64, vp, c_i64,
                                         ctypes.c_int, vp, vp, vp, vp]
        L.nvfp4_quantize_ref.restype = ctypes.c_int
        L.nvfp4_dequantize_ref.argtypes = [vp, vp, vp, c_i64, c_i64, vp]
        L.nvfp4_dequantize_ref.restype = ctypes.c_int
        L.mxfp4_resq_quantize_ref.argtypes = [vp, c_i64, c_i64,
                                              vp, vp, vp, vp, vp]
        L.mxfp4_resq_quantize_ref.restype = ctypes.c_int
        L.mxfp4_resq_dense_quantize_ref.argtypes = [vp, c_i64, c_i64, vp, vp, vp, vp]
        L.mxfp4_resq_dense_quantize_ref.restype = ctypes.c_int
        L.mxfp4_resq_reconstruct_ref.argtypes = [vp, vp, vp, vp, vp, c_i64, c_i64,
                                                 ctypes.c_int, vp]
        L.mxfp4_resq_reconstruct_ref.restype = ctypes.c_int
        L.nvfp4_quantize_guided_ref.argtypes = [vp, c_i64, c_i64, vp, vp, vp, vp, vp]
        L.nvfp4_quantize_guided_ref.restype = ctypes.c_int
        L.nvfp4_quantize_global_ref.argtypes = [vp, c_i64, c_i64, ctypes.c_int, vp, vp, vp, vp]
        L.nvfp4_quantize_global_ref.restype = ctypes.c_int
        _lib = L
    return _lib


class NVFP4Block(ctypes.Structure):
    """Mirror of oracle_nvfp4_block_t (fp4_oracle.h)."""
    _fields_ = [
        ("t", ctypes.c_float * 2),
        ("e", ctypes.c_float * 2),
        ("e_byte", ctypes.c_uint8 * 2),
        ("err", ctypes.c_float * 2),
        ("err16", ctypes.c_float * 2),
        ("cand", (ctypes.c_float * 16) * 2),
        ("code", (ctypes.c_uint8 * 16) * 2),
        ("choice", ctypes.c_int),
    ]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(status, what):
    if status != 0:
        raise ValueError("%s rejected its arguments (status %d)" % (what, status))


def e2m1_code(a: float) -> int:
    return lib().oracle_e2m1_code(a)


def e2m1_value(q: int) -> float:
    return lib().oracle_e2m1_value(q)


def e4m3_encode(t: float) -> int:
    return lib().oracle_e4m3_encode(t)


def e4m3_decode(b: int) -> float:
    return lib().oracle_e4m3_decode(b)


def bf16_rne(f: float) -> int:
    return lib().oracle_bf16_rne(f)


def e8m0_exponent(b: float) -> int:
    return lib().oracle_e8m0_exponent(b)


def fp16_rne(v: float) -> float:
    return lib().oracle_fp16_rne(v)


def mode_of(four_over_six) -> int:
    """0: 6 only; 1: 4/6 on the FP32 error; 2 (or "fp16"): 4/6 on the FP16
    fast path's error."""
    if isinstance(four_over_six, str):
        return {"fp16": 2}[four_over_six]
    m = int(four_over_six)
    if m not in (0, 1, 2):
        raise ValueError("four_over_six must be 0, 1, 2 or 'fp16'")
    return m


def nvfp4_block(x16, s: float, four_over_six) -> NVFP4Block:
    """One 16-element block (FP32 values) with its internals."""
    x = np.ascontiguousarray(x16, dtype=np.float32)
    assert x.shape == (16,)
    out = NVFP4Block()
    lib().oracle_nvfp4_block(_ptr(x), float(np.float32(s)), mode_of(four_over_six),
                             ctypes.byref(out))
    return out


def nvfp4_quantize(x_bits, four_over_six=True, offsets=None, dequant=True,
                   outputs=None):
    """x_bits: uint16 [rows, hidden] BF16 patterns.

    Returns (codes u8 [rows, hidden/2], scales u8 [rows, hidden/16],
    token_scales f32 [rows], dequant u16 [rows, hidden] or None).  With
    ``outputs`` the given arrays are written in place (rows outside the
    ragged range keep their contents)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, hidden = x.shape
    if outputs is None:
        codes = np.zeros((rows, hidden // 2), np.uint8)
        scales = np.zeros((rows, hidden // 16), np.uint8)
        ts = np.zeros((rows,), np.float32)
        dq = np.zeros((rows, hidden), np.uint16) if dequant else None
    else:
        codes, scales, ts, dq = outputs
    off = None
    ng = 0
    if offsets is not None:
        off = np.ascontiguousarray(offsets, dtype=np.int64)
        ng = off.shape[0] - 1
    st = lib().nvfp4_quantize_ref(_ptr(x), rows, hidden, _ptr(off), ng,
                                  mode_of(four_over_six), _ptr(codes),
                                  _ptr(scales), _ptr(ts), _ptr(dq))
    _check(st, "nvfp4_quantize_ref")
    return codes, scales, ts, dq


def nvfp4_dequantize(codes, scales, token_scales):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    ts = np.ascontiguousarray(token_scales, dtype=np.float32)
    rows = codes.shape[0]
    hidden = codes.shape[1] * 2
    out = np.zeros((rows, hidden), np.uint16)
    st = lib().nvfp4_dequantize_ref(_ptr(codes), _ptr(scales), _ptr(ts), rows,
                                    hidden, _ptr(out))
    _check(st, "nvfp4_dequantize_ref")
    return out


def mxfp4_resq_quantize(x_bits):
    """Returns (codes [R,H/2], scales [R,H/32], res_codes [R,H/4],
    res_meta [R,H/8], res_scales [R,H/32]), all uint8."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, hidden = x.shape
    codes = np.zeros((rows, hidden // 2), np.uint8)
    scales = np.zeros((rows, hidden // 32), np.uint8)
    rc = np.zeros((rows, hidden // 4), np.uint8)
    rm = np.zeros((rows, hidden // 8), np.uint8)
    rs = np.zeros((rows, hidden // 32), np.uint8)
    st = lib().mxfp4_resq_quantize_ref(_ptr(x), rows, hidden, _ptr(codes),
                                       _ptr(scales), _ptr(rc), _ptr(rm), _ptr(rs))
    _check(st, "mxfp4_resq_quantize_ref")
    return codes, scales, rc, rm, rs


def mxfp4_resq_dense_quantize(x_bits):
    """Rollout-ResQ-Dense.  Returns (codes [R,H/2], scales [R,H/32],
    res_codes [R,H/2], res_scales [R,H/32]), all uint8."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, hidden = x.shape
    codes = np.zeros((rows, hidden // 2), np.uint8)
    scales = np.zeros((rows, hidden // 32), np.uint8)
    rc = np.zeros((rows, hidden // 2), np.uint8)
    rs = np.zeros((rows, hidden // 32), np.uint8)
    st = lib().mxfp4_resq_dense_quantize_ref(_ptr(x), rows, hidden, _ptr(codes), _ptr(scales),
                                             _ptr(rc), _ptr(rs))
    _check(st, "mxfp4_resq_dense_quantize_ref")
    return codes, scales, rc, rs


def mxfp4_resq_reconstruct(codes, scales, res_codes=None, res_meta=None, res_scales=None,
                           residual=0):
    """FP32 [R, H]: DQ(Q(X)) (+ the sparse (1) or dense (2) residual)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, hidden = codes.shape[0], codes.shape[1] * 2
    arrs = [None if a is None else np.ascontiguousarray(a, dtype=np.uint8)
            for a in (res_codes, res_meta, res_scales)]
    out = np.zeros((rows, hidden), np.float32)
    st = lib().mxfp4_resq_reconstruct_ref(_ptr(codes), _ptr(scales), *[_ptr(a) for a in arrs],
                                          rows, hidden, int(residual), _ptr(out))
    _check(st, "mxfp4_resq_reconstruct_ref")
    return out


def nvfp4_quantize_guided(x_bits, guide_codes, block_scales, token_scales, dequant=True):
    """TRACE rollout-guided rounding of x under the rollout's scales
    (guide_codes None: round-to-nearest under those scales).
    Returns (codes u8 [R, H/2], dequant u16 [R, H] or None)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, hidden = x.shape
    g = None if guide_codes is None else np.ascontiguousarray(guide_codes, dtype=np.uint8)
    bs = np.ascontiguousarray(block_scales, dtype=np.uint8)
    ts = np.ascontiguousarray(token_scales, dtype=np.float32)
    codes = np.zeros((rows, hidden // 2), np.uint8)
    dq = np.zeros((rows, hidden), np.uint16) if dequant else None
    st = lib().nvfp4_quantize_guided_ref(_ptr(x), rows, hidden, _ptr(g), _ptr(bs), _ptr(ts),
                                         _ptr(codes), _ptr(dq))
    _check(st, "nvfp4_quantize_guided_ref")
    return codes, dq


def nvfp4_quantize_global(x_bits, four_over_six=True, dequant=True):
    """One FP32 scale for the whole tensor.  Returns (codes, scales,
    tensor_scale f32 [1], dequant u16 or None)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, hidden = x.shape
    codes = np.zeros((rows, hidden // 2), np.uint8)
    scales = np.zeros((rows, hidden // 16), np.uint8)
    ts = np.zeros((1,), np.float32)
    dq = np.zeros((rows, hidden), np.uint16) if dequant else None
    st = lib().nvfp4_quantize_global_ref(_ptr(x), rows, hidden, mode_of(four_over_six),
                                         _ptr(codes), _ptr(scales), _ptr(ts), _ptr(dq))
    _check(st, "nvfp4_quantize_global_ref")
    return codes, scales, ts, dq
