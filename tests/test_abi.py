"""The C-ABI library loads, exports every call include/*.h declares, and
rejects bad arguments on the host before any HIP call (so these run
without a GPU; nothing here launches a kernel)."""
import ctypes
import glob
import os
import re

import pytest

import fp4_block_quantization_amd as fq
from fp4_block_quantization_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SUCCESS, NULL, SHAPE, MISALIGNED, LAUNCH, INVALID = 0, 1, 2, 3, 4, 5


def declared_functions(header):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:FP4Q_API\s+)?(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*"
                       r"([A-Za-z_][A-Za-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


# each header under include/ and the library that exports its calls
HEADER_LIBS = {"fp4q.h": _build.LIB_PATH, "fp4q_membench.h": _build.MEMBENCH_PATH}


def test_every_header_has_its_library():
    assert sorted(os.path.basename(h) for h in glob.glob(os.path.join(ROOT, "include", "*.h"))) \
        == sorted(HEADER_LIBS)


def test_library_exports_every_declared_call():
    names = declared_functions("fp4q.h")
    assert len(names) == 9, names
    assert {"nvfp4_quantize", "nvfp4_dequantize", "mxfp4_resq_quantize",
            "mxfp4_resq_dense_quantize", "mxfp4_resq_reconstruct", "nvfp4_quantize_guided",
            "nvfp4_quantize_global", "nvfp4_quantize_global_noalloc",
            "fp4q_status_string"} <= set(names)
    L = fq.lib()
    for n in names:
        assert hasattr(L, n), n
    # the stand-in and exact-decision builds of the same sources export the
    # same calls
    for path in (_build.STANDIN_PATH, _build.EXACTDECISION_PATH):
        S = ctypes.CDLL(path)
        for n in names:
            assert hasattr(S, n), (path, n)


def test_membench_library_exports_and_rejects():
    names = declared_functions("fp4q_membench.h")
    assert names == ["fp4q_k0_copy", "fp4q_k0_copy_stream", "fp4q_k0_mix", "fp4q_k0_read",
                     "fp4q_k0_write"], names
    M = ctypes.CDLL(_build.MEMBENCH_PATH)
    P, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    M.fp4q_k0_copy.argtypes = [P, P, i64, ci, P]
    M.fp4q_k0_read.argtypes = [P, i64, ci, ci, P, P]
    M.fp4q_k0_write.argtypes = [P, i64, ci, P]
    M.fp4q_k0_copy_stream.argtypes = [P, P, i64, ci, ci, P]
    M.fp4q_k0_mix.argtypes = [P, P, i64, ci, ci, P]
    a16 = P(0x10000)
    assert M.fp4q_k0_mix(a16, a16, 4096, 3, 1, None) == INVALID
    assert M.fp4q_k0_mix(a16, a16, 4096, 4, 3, None) == INVALID
    assert M.fp4q_k0_mix(a16, a16, 2048, 4, 1, None) == SHAPE
    assert M.fp4q_k0_mix(None, a16, 4096, 4, 1, None) == NULL
    assert M.fp4q_k0_mix(a16, P(0x10004), 4096, 4, 1, None) == MISALIGNED
    assert M.fp4q_k0_mix(None, None, 0, 4, 1, None) == SUCCESS
    assert M.fp4q_k0_copy_stream(a16, a16, 32, 1, 0, None) == INVALID
    assert M.fp4q_k0_copy_stream(a16, a16, 24, 1, 8, None) == SHAPE
    assert M.fp4q_k0_copy(a16, a16, 24, 1, None) == SHAPE
    assert M.fp4q_k0_copy(None, a16, 32, 1, None) == NULL
    assert M.fp4q_k0_copy(P(0x10008), a16, 32, 1, None) == MISALIGNED
    assert M.fp4q_k0_copy(None, None, 0, 1, None) == SUCCESS
    assert M.fp4q_k0_read(a16, 64, 3, 0, a16, None) == INVALID
    assert M.fp4q_k0_read(a16, 6, 4, 0, a16, None) == SHAPE
    assert M.fp4q_k0_read(a16, 64, 4, 0, None, None) == NULL
    assert M.fp4q_k0_read(P(0x10002), 64, 4, 0, a16, None) == MISALIGNED
    assert M.fp4q_k0_write(a16, -16, 1, None) == SHAPE
    assert M.fp4q_k0_write(None, 16, 1, None) == NULL
    # store modes 0, 1 and 2 only
    assert M.fp4q_k0_write(a16, 16, 3, None) == INVALID
    assert M.fp4q_k0_copy(a16, a16, 32, -1, None) == INVALID
    assert M.fp4q_k0_copy_stream(a16, a16, 32, 3, 8, None) == INVALID


def test_status_strings():
    L = fq.lib()
    for s in range(6):
        assert L.fp4q_status_string(s) != b"unknown status"
    assert L.fp4q_status_string(99) == b"unknown status"


P = ctypes.c_void_p
A16 = P(0x10000)  # aligned fake pointers: never dereferenced by a rejected call
A8 = P(0x10008)
ODD = P(0x10001)


def nvq(x=A16, rows=4, hidden=64, offs=None, ng=0, fos=1, codes=A16, scales=A16, ts=A16,
        dq=A16):
    return fq.lib().nvfp4_quantize(x, rows, hidden, offs, ng, fos, codes, scales, ts, dq, None)


def test_nvfp4_quantize_rejects():
    assert nvq(hidden=24) == SHAPE
    assert nvq(hidden=0) == SHAPE
    assert nvq(rows=-1) == SHAPE
    assert nvq(ng=-1) == SHAPE
    assert nvq(ng=2) == NULL  # groups without offsets
    assert nvq(offs=A8, ng=0) == SHAPE  # offsets without groups
    assert nvq(x=None) == NULL
    assert nvq(codes=None) == NULL
    assert nvq(scales=None) == NULL
    assert nvq(ts=None) == NULL
    assert nvq(x=A8) == MISALIGNED
    assert nvq(dq=A8) == MISALIGNED
    assert nvq(codes=P(0x10004)) == MISALIGNED
    assert nvq(ts=P(0x10002)) == MISALIGNED
    assert nvq(offs=P(0x10004), ng=1) == MISALIGNED
    assert nvq(rows=1 << 33) == SHAPE
    assert nvq(fos=3) == INVALID
    assert nvq(fos=-1) == INVALID
    # empty input: success, nothing launched, pointers may be NULL
    assert nvq(rows=0, x=None, codes=None, scales=None, ts=None, dq=None) == SUCCESS


def test_nvfp4_dequantize_rejects():
    L = fq.lib()
    assert L.nvfp4_dequantize(A16, A16, A16, 4, 40, A16, None) == SHAPE
    assert L.nvfp4_dequantize(None, A16, A16, 4, 64, A16, None) == NULL
    assert L.nvfp4_dequantize(A16, A16, A16, 4, 64, A8, None) == MISALIGNED
    assert L.nvfp4_dequantize(None, None, None, 0, 64, None, None) == SUCCESS


def test_mxfp4_resq_rejects():
    L = fq.lib()
    f = L.mxfp4_resq_quantize
    assert f(A16, 4, 48, A16, A16, A16, A16, A16, None) == SHAPE  # not a multiple of 32
    assert f(A16, 4, 64, A16, A16, None, A16, A16, None) == NULL
    assert f(A16, 4, 64, A8, A16, A16, A16, A16, None) == MISALIGNED
    assert f(A16, 4, 64, A16, A16, A16, P(0x10002), A16, None) == MISALIGNED
    assert f(None, 0, 64, None, None, None, None, None, None) == SUCCESS


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(fq.Fp4qError):
        fq.nvfp4_quantize(torch.zeros(4, 64, dtype=torch.bfloat16))
    with pytest.raises(fq.Fp4qError):
        fq.mxfp4_resq_quantize(torch.zeros(4, 64, dtype=torch.bfloat16))


def test_mxfp4_resq_dense_and_reconstruct_reject():
    L = fq.lib()
    dense = lambda **k: L.mxfp4_resq_dense_quantize(
        k.get("x", A16), k.get("rows", 4), k.get("hidden", 64), k.get("codes", A16), A16,
        k.get("rc", A16), A16, None)
    assert dense(hidden=48) == SHAPE
    assert dense(x=None) == NULL
    assert dense(rc=A8) == MISALIGNED
    assert dense(rows=0, x=None) == SUCCESS
    rec = lambda **k: L.mxfp4_resq_reconstruct(
        k.get("codes", A16), A16, k.get("rc", A16), k.get("rm", A16), k.get("rs", A16),
        k.get("rows", 4), k.get("hidden", 64), k.get("res", 1), k.get("out", A16), None)
    assert rec(res=3) == INVALID
    assert rec(res=-1) == INVALID
    assert rec(hidden=16) == SHAPE
    assert rec(out=None) == NULL
    assert rec(rm=None) == NULL          # sparse residual needs its metadata
    assert rec(res=2, rc=None) == NULL
    assert rec(res=2, rc=A8) == MISALIGNED
    assert rec(res=1, rc=P(0x10004)) == MISALIGNED
    assert rec(out=A8) == MISALIGNED
    assert rec(rows=0, codes=None, out=None) == SUCCESS


def test_nvfp4_quantize_guided_rejects():
    L = fq.lib()
    g = lambda **k: L.nvfp4_quantize_guided(
        k.get("x", A16), k.get("rows", 4), k.get("hidden", 64), k.get("guide", A16), A16,
        k.get("ts", A16), k.get("codes", A16), k.get("dq", A16), None)
    assert g(hidden=24) == SHAPE
    assert g(x=None) == NULL
    assert g(codes=None) == NULL
    # no guide is a valid call (round to nearest); it is still checked in
    # full before anything is launched
    assert g(guide=None, codes=None) == NULL
    assert g(guide=None, x=A8) == MISALIGNED
    assert g(x=A8) == MISALIGNED
    assert g(guide=P(0x10002)) == MISALIGNED
    assert g(dq=A8) == MISALIGNED
    assert g(rows=0, x=None, guide=None, codes=None) == SUCCESS


def test_nvfp4_quantize_global_rejects():
    L = fq.lib()
    g = lambda **k: L.nvfp4_quantize_global(
        k.get("x", A16), k.get("rows", 4), k.get("hidden", 64), k.get("fos", 1),
        k.get("codes", A16), A16, k.get("ts", A16), k.get("dq", A16), k.get("ws", A16), None)
    assert g(hidden=24) == SHAPE
    assert g(ws=None) == NULL
    assert g(ws=P(0x10002)) == MISALIGNED
    assert g(ws=P(0x10008)) == MISALIGNED  # 16-byte alignment
    assert g(fos=3) == INVALID
    assert g(x=None) == NULL
    assert g(ts=None) == NULL
    assert g(ts=P(0x10002)) == MISALIGNED
    assert g(dq=A8) == MISALIGNED
    assert g(rows=0, x=None, codes=None, ts=None, ws=None) == SUCCESS


def test_nvfp4_quantize_global_noalloc_rejects():
    # the same validation as the workspace form, without the workspace
    # argument; every case returns before any HIP call
    L = fq.lib()
    f = L.nvfp4_quantize_global_noalloc
    f.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int] + [P] * 5
    f.restype = ctypes.c_int
    g = lambda **k: f(
        k.get("x", A16), k.get("rows", 4), k.get("hidden", 64), k.get("fos", 1),
        k.get("codes", A16), A16, k.get("ts", A16), k.get("dq", A16), None)
    assert g(hidden=24) == SHAPE
    assert g(rows=-1) == SHAPE
    assert g(fos=3) == INVALID
    assert g(fos=-1) == INVALID
    assert g(x=None) == NULL
    assert g(codes=None) == NULL
    assert g(ts=None) == NULL
    assert g(x=P(0x10008)) == MISALIGNED
    assert g(codes=P(0x10004)) == MISALIGNED
    assert g(ts=P(0x10002)) == MISALIGNED
    assert g(dq=A8) == MISALIGNED
    assert g(rows=0, x=None, codes=None, ts=None) == SUCCESS
