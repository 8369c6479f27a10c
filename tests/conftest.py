import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TESTS = os.path.dirname(os.path.abspath(__file__))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def pins():
    """The exhaustive pin helpers (tests/pins/pins.c), compiled per session."""
    out_dir = os.path.join(TESTS, "_build")
    os.makedirs(out_dir, exist_ok=True)
    so = os.path.join(out_dir, "libpins.%d.so" % os.getpid())
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared",
                    "-ffp-contract=off", "-fopenmp", os.path.join(TESTS, "pins", "pins.c"),
                    "-lm", "-o", so], check=True)
    L = ctypes.CDLL(so)
    os.unlink(so)
    u32 = ctypes.c_uint32
    for name in ("pin_e2m1", "pin_e4m3", "pin_bf16"):
        fn = getattr(L, name)
        fn.argtypes = [ctypes.c_void_p, u32, u32, ctypes.POINTER(u32)]
        fn.restype = ctypes.c_int64
    L.pin_fp16.argtypes = [ctypes.c_void_p, u32, u32, ctypes.POINTER(u32)]
    L.pin_fp16.restype = ctypes.c_int64
    L.pin_e8m0.argtypes = [ctypes.c_void_p, u32, u32, u32, ctypes.POINTER(u32)]
    L.pin_e8m0.restype = ctypes.c_int64
    u64p = ctypes.POINTER(ctypes.c_uint64)
    L.cmp_fp4.argtypes = [ctypes.c_void_p, u32, u32, ctypes.c_uint64, ctypes.c_void_p, u64p]
    L.cmp_fp4.restype = ctypes.c_int64
    L.cmp_fp4_floor.argtypes = [u32, ctypes.c_uint64, ctypes.c_void_p, u64p]
    L.cmp_fp4_floor.restype = ctypes.c_int64
    L.cmp_fp4_scaled.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p,
                                 u64p]
    L.cmp_fp4_scaled.restype = ctypes.c_int64
    L.cmp_recip.argtypes = [u32, ctypes.c_uint64, ctypes.c_void_p, u64p]
    L.cmp_recip.restype = ctypes.c_int64
    for name in ("cmp_bf16", "cmp_fp8"):
        fn = getattr(L, name)
        fn.argtypes = [ctypes.c_void_p, u32, ctypes.c_uint64, ctypes.c_void_p, u64p]
        fn.restype = ctypes.c_int64
    return L


@pytest.fixture(scope="session")
def olib():
    import oracle
    return oracle.lib()


def fnptr(lib, name):
    return ctypes.cast(getattr(lib, name), ctypes.c_void_p)
