"""MI355X (gfx950) fused FP4 block quantizer -- Python binding.

Argument marshalling only: every step of the quantizer runs in the HIP
kernels of libfp4q.so (C ABI in include/fp4q.h).  PyTorch supplies device
memory and the current stream.  There is no CPU fallback: if the library is
not built, or a tensor is not on a GPU, the call raises.

Calls (same names as the C ABI):
  nvfp4_quantize(x, four_over_six=True, offsets=None, dequant=True)
      four_over_six: True/1, "fp16"/2 (FP16 fast-path decision), False/0
      -> codes u8 [R, H/2], block_scales u8 [R, H/16] (E4M3FN bits),
         token_scales f32 [R], dequant bf16 [R, H] or None
  nvfp4_dequantize(codes, block_scales, token_scales) -> bf16 [R, H]
  mxfp4_resq_quantize(x)
      -> codes u8 [R, H/2], scales u8 [R, H/32], res_codes u8 [R, H/4],
         res_meta u8 [R, H/8], res_scales u8 [R, H/32]
  mxfp4_resq_dense_quantize(x)
      -> codes u8 [R, H/2], scales u8 [R, H/32], res_codes u8 [R, H/2],
         res_scales u8 [R, H/32]
  mxfp4_resq_reconstruct(codes, scales, res_codes, res_meta, res_scales,
                         residual) -> f32 [R, H]
"""
import ctypes
import os

import torch

from . import _build

__all__ = ["lib", "nvfp4_quantize", "nvfp4_dequantize", "nvfp4_quantize_guided",
           "nvfp4_quantize_global",
           "mxfp4_resq_quantize",
           "mxfp4_resq_dense_quantize", "mxfp4_resq_reconstruct", "Fp4qError", "LIB_PATH"]

LIB_PATH = _build.LIB_PATH
_lib = None


class Fp4qError(RuntimeError):
    pass


# Bytes of device workspace nvfp4_quantize_global needs (fp4q.h)
GLOBAL_WORKSPACE_BYTES = 1024


def declare(L):
    """Argument and result types of every C-ABI call on a loaded library
    (libfp4q.so, or a build of the same sources with other knobs)."""
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.nvfp4_quantize.argtypes = [vp, i64, i64, vp, i64, ci, vp, vp, vp, vp, vp]
    L.nvfp4_dequantize.argtypes = [vp, vp, vp, i64, i64, vp, vp]
    L.mxfp4_resq_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, vp]
    L.nvfp4_quantize_global.argtypes = [vp, i64, i64, ci, vp, vp, vp, vp, vp, vp]
    L.nvfp4_quantize_guided.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, vp]
    L.mxfp4_resq_dense_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
    L.mxfp4_resq_reconstruct.argtypes = [vp, vp, vp, vp, vp, i64, i64, ci, vp, vp]
    for name in ("nvfp4_quantize", "nvfp4_dequantize", "mxfp4_resq_quantize",
                 "nvfp4_quantize_global", "nvfp4_quantize_guided", "mxfp4_resq_dense_quantize",
                 "mxfp4_resq_reconstruct"):
        getattr(L, name).restype = ci
    L.fp4q_status_string.argtypes = [ci]
    L.fp4q_status_string.restype = ctypes.c_char_p
    return L


def lib():
    """The loaded libfp4q.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Fp4qError(
                "libfp4q.so is not built (%s); run __graft_entry__.build() or "
                "python fp4_block_quantization_amd/_build.py" % LIB_PATH)
        _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(status, what):
    if status != 0:
        msg = lib().fp4q_status_string(status).decode()
        raise Fp4qError("%s failed: %s (status %d)" % (what, msg, status))


# The current stream's handle on a device: torch's raw getter takes ~0.15 us
# a call, the public torch.cuda.current_stream(...).cuda_stream ~2 us (it
# builds a Stream object), which is most of a tiny call's budget.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t):
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t, name, dtype):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise Fp4qError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise Fp4qError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise Fp4qError("%s must be contiguous" % name)
    return t


def _same_device(x, *ts):
    d = x.get_device()
    for t in ts:
        if t is not None and t.get_device() != d:
            raise Fp4qError("all tensors must be on %s, got one on %s" % (x.device, t.device))


def _sized(t, name, dtype, numel):
    """A caller-supplied tensor: on a GPU, of dtype, contiguous, holding
    exactly numel elements (the kernels write or read that many)."""
    _dev(t, name, dtype)
    if t.numel() != numel:
        raise Fp4qError("%s must hold %d elements, got %d" % (name, numel, t.numel()))
    return t


def _rows_hidden(codes):
    """rows and hidden of a [rows, hidden/2] code tensor."""
    if codes.dim() != 2:
        raise Fp4qError("codes must be 2-D [rows, hidden/2]")
    return codes.shape[0], 2 * codes.shape[1]


def _p(t):
    return None if t is None else t.data_ptr()


def _mode(four_over_six):
    if isinstance(four_over_six, str):
        if four_over_six != "fp16":
            raise Fp4qError("four_over_six must be True/False/0/1/2 or 'fp16'")
        return 2
    return int(four_over_six)  # the library rejects values other than 0, 1, 2


def nvfp4_quantize(x, four_over_six=True, offsets=None, dequant=True, out=None):
    """Per-token NVFP4 with Four-Over-Six of a BF16 [rows, hidden] tensor.

    four_over_six: True/1 (4/6 on the FP32 error), "fp16"/2 (4/6 on the FP16
    fast path's error), False/0 (6 only).  offsets: optional int64 GPU
    tensor [groups + 1] (ragged routed rows); only rows [offsets[0],
    offsets[-1]) are written.  out: optional tuple (codes, block_scales,
    token_scales, dequant-or-None) to write into."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise Fp4qError("x must be 2-D [rows, hidden]")
    rows, hidden = x.shape
    if out is None:
        codes = torch.empty((rows, hidden // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((rows, hidden // 16), dtype=torch.uint8, device=x.device)
        ts = torch.empty((rows,), dtype=torch.float32, device=x.device)
        dq = torch.empty_like(x) if dequant else None
    else:
        codes, scales, ts, dq = out
        _sized(codes, "codes", torch.uint8, rows * (hidden // 2))
        _sized(scales, "block_scales", torch.uint8, rows * (hidden // 16))
        _sized(ts, "token_scales", torch.float32, rows)
        if dq is not None:
            _sized(dq, "dequant", torch.bfloat16, rows * hidden)
    ng = 0
    if offsets is not None:
        _dev(offsets, "offsets", torch.int64)
        ng = offsets.numel() - 1
        if ng < 1:
            raise Fp4qError("offsets needs at least two entries")
    _same_device(x, codes, scales, ts, dq, offsets)
    st = lib().nvfp4_quantize(_p(x), rows, hidden, _p(offsets), ng, _mode(four_over_six),
                              _p(codes), _p(scales), _p(ts), _p(dq), _stream(x))
    _check(st, "nvfp4_quantize")
    return codes, scales, ts, dq


def nvfp4_dequantize(codes, block_scales, token_scales, out=None):
    _dev(codes, "codes", torch.uint8)
    rows, hidden = _rows_hidden(codes)
    _sized(block_scales, "block_scales", torch.uint8, rows * (hidden // 16))
    _sized(token_scales, "token_scales", torch.float32, rows)
    if out is None:
        out = torch.empty((rows, hidden), dtype=torch.bfloat16, device=codes.device)
    _sized(out, "out", torch.bfloat16, rows * hidden)
    _same_device(codes, block_scales, token_scales, out)
    st = lib().nvfp4_dequantize(_p(codes), _p(block_scales), _p(token_scales), rows, hidden,
                                _p(out), _stream(codes))
    _check(st, "nvfp4_dequantize")
    return out


def mxfp4_resq_quantize(x, out=None):
    """MXFP4 + Rollout-ResQ residual with 2:4 sparsity of a BF16 [rows, hidden]."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise Fp4qError("x must be 2-D [rows, hidden]")
    rows, hidden = x.shape
    if out is None:
        kw = dict(dtype=torch.uint8, device=x.device)
        out = (torch.empty((rows, hidden // 2), **kw), torch.empty((rows, hidden // 32), **kw),
               torch.empty((rows, hidden // 4), **kw), torch.empty((rows, hidden // 8), **kw),
               torch.empty((rows, hidden // 32), **kw))
    if len(out) != 5:
        raise Fp4qError("out must be (codes, scales, res_codes, res_meta, res_scales)")
    sizes = (hidden // 2, hidden // 32, hidden // 4, hidden // 8, hidden // 32)
    for t, n, k in zip(out, ("codes", "scales", "res_codes", "res_meta", "res_scales"), sizes):
        _sized(t, n, torch.uint8, rows * k)
    _same_device(x, *out)
    st = lib().mxfp4_resq_quantize(_p(x), rows, hidden, *[_p(t) for t in out], _stream(x))
    _check(st, "mxfp4_resq_quantize")
    return out


def mxfp4_resq_dense_quantize(x, out=None):
    """MXFP4 + Rollout-ResQ-Dense residual (every residual code kept)."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise Fp4qError("x must be 2-D [rows, hidden]")
    rows, hidden = x.shape
    if out is None:
        kw = dict(dtype=torch.uint8, device=x.device)
        out = (torch.empty((rows, hidden // 2), **kw), torch.empty((rows, hidden // 32), **kw),
               torch.empty((rows, hidden // 2), **kw), torch.empty((rows, hidden // 32), **kw))
    if len(out) != 4:
        raise Fp4qError("out must be (codes, scales, res_codes, res_scales)")
    sizes = (hidden // 2, hidden // 32, hidden // 2, hidden // 32)
    for t, n, k in zip(out, ("codes", "scales", "res_codes", "res_scales"), sizes):
        _sized(t, n, torch.uint8, rows * k)
    _same_device(x, *out)
    st = lib().mxfp4_resq_dense_quantize(_p(x), rows, hidden, *[_p(t) for t in out], _stream(x))
    _check(st, "mxfp4_resq_dense_quantize")
    return out


def mxfp4_resq_reconstruct(codes, scales, res_codes=None, res_meta=None, res_scales=None,
                           residual=0, out=None):
    """FP32 X_hat = DQ(Q(X)) (+ DQ(S(Q(dX))) for residual 1, + DQ(Q(dX)) for
    residual 2, from the sparse or dense quantize outputs)."""
    _dev(codes, "codes", torch.uint8)
    rows, hidden = _rows_hidden(codes)
    _sized(scales, "scales", torch.uint8, rows * (hidden // 32))
    # the residual tensors the mode reads: S2:4 (1) kept codes, metadata and
    # scales; dense (2) every residual code and the scales
    mode = int(residual)
    if mode in (1, 2):
        need = [("res_codes", res_codes, hidden // (4 if mode == 1 else 2)),
                ("res_scales", res_scales, hidden // 32)]
        if mode == 1:
            need.append(("res_meta", res_meta, hidden // 8))
        for n, t, k in need:
            if t is None:
                raise Fp4qError("%s is required for residual=%d" % (n, mode))
            _sized(t, n, torch.uint8, rows * k)
    if out is None:
        out = torch.empty((rows, hidden), dtype=torch.float32, device=codes.device)
    _sized(out, "out", torch.float32, rows * hidden)
    _same_device(codes, scales, res_codes, res_meta, res_scales, out)
    st = lib().mxfp4_resq_reconstruct(_p(codes), _p(scales), _p(res_codes), _p(res_meta),
                                      _p(res_scales), rows, hidden, mode, _p(out),
                                      _stream(codes))
    _check(st, "mxfp4_resq_reconstruct")
    return out


def nvfp4_quantize_guided(x, guide_codes, block_scales, token_scales, dequant=True, out=None):
    """TRACE rollout-guided rounding of x (BF16 [rows, hidden]) under the
    rollout's scales, toward the rollout's codes (guide_codes None: round to
    nearest under those scales).  Returns (codes u8 [R, H/2], dequant bf16
    [R, H] or None)."""
    _dev(x, "x", torch.bfloat16)
    if guide_codes is not None:
        _dev(guide_codes, "guide_codes", torch.uint8)
    _dev(block_scales, "block_scales", torch.uint8)
    _dev(token_scales, "token_scales", torch.float32)
    if x.dim() != 2:
        raise Fp4qError("x must be 2-D [rows, hidden]")
    rows, hidden = x.shape
    if guide_codes is not None:
        _sized(guide_codes, "guide_codes", torch.uint8, rows * (hidden // 2))
    _sized(block_scales, "block_scales", torch.uint8, rows * (hidden // 16))
    _sized(token_scales, "token_scales", torch.float32, rows)
    if out is None:
        codes = torch.empty((rows, hidden // 2), dtype=torch.uint8, device=x.device)
        dq = torch.empty_like(x) if dequant else None
    else:
        codes, dq = out
        _sized(codes, "codes", torch.uint8, rows * (hidden // 2))
        if dq is not None:
            _sized(dq, "dequant", torch.bfloat16, rows * hidden)
    _same_device(x, guide_codes, block_scales, token_scales, codes, dq)
    st = lib().nvfp4_quantize_guided(_p(x), rows, hidden, _p(guide_codes), _p(block_scales),
                                     _p(token_scales), _p(codes), _p(dq), _stream(x))
    _check(st, "nvfp4_quantize_guided")
    return codes, dq


def nvfp4_quantize_global(x, four_over_six=True, dequant=True, out=None, workspace=None):
    """NVFP4 with one FP32 scale for the whole tensor (the naive baseline).
    Returns (codes, block_scales, tensor_scale f32 [1], dequant or None).
    workspace: optional uint8 GPU tensor of GLOBAL_WORKSPACE_BYTES (else one
    is allocated), the partial maxima between the call's two kernels; calls
    in flight at the same time must not share one."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise Fp4qError("x must be 2-D [rows, hidden]")
    rows, hidden = x.shape
    if out is None:
        codes = torch.empty((rows, hidden // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((rows, hidden // 16), dtype=torch.uint8, device=x.device)
        ts = torch.empty((1,), dtype=torch.float32, device=x.device)
        dq = torch.empty_like(x) if dequant else None
    else:
        codes, scales, ts, dq = out
        _sized(codes, "codes", torch.uint8, rows * (hidden // 2))
        _sized(scales, "block_scales", torch.uint8, rows * (hidden // 16))
        _sized(ts, "tensor_scale", torch.float32, 1)
        if dq is not None:
            _sized(dq, "dequant", torch.bfloat16, rows * hidden)
    if workspace is None:
        workspace = torch.empty(GLOBAL_WORKSPACE_BYTES, dtype=torch.uint8, device=x.device)
    _sized(workspace, "workspace", torch.uint8, GLOBAL_WORKSPACE_BYTES)
    _same_device(x, codes, scales, ts, dq, workspace)
    st = lib().nvfp4_quantize_global(_p(x), rows, hidden, _mode(four_over_six), _p(codes),
                                     _p(scales), _p(ts), _p(dq), _p(workspace), _stream(x))
    _check(st, "nvfp4_quantize_global")
    return codes, scales, ts, dq
