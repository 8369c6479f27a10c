"""Seeded synthetic workloads for the FP4 quantizer (tests and benchmark).

This module holds no quantizer arithmetic.  It draws FP32 values from
gen.c (row-addressable seeded streams), and the BF16 inputs are produced
from them by torch's own FP32 -> BF16 cast.

The workloads stand in for the pages' data: MoE expert activations and
weights inside RL training and rollouts (humans& article, sections 1 and 3;
NVFP4-RL blog, sections 2 and 4), ragged routed tokens of a per-token MoE
kernel (humans& article, PR list), and rollout linear-layer activations with
channel outliers (HiFloat4 page, underflow diagnosis and Rollout-ResQ).

Named workloads (seed = workload number):
  tiny_ref         256 x 2048,  N(0,1), 1% of channels (20) x 50
  moe_act          8192 x 7168, Student-t(3) x LogNormal(0, 0.5) row gain
  expert_weights   32 experts x 2048 x 7168 = 65536 x 7168 rows,
                   0.02 N(0,1), each entry x 20 with probability 0.001
  ragged_routed    65536 x 2048, N(0,1) x LogNormal(0, 1) row gain,
                   64 expert groups (top-8 routing of 8192 tokens)
  resq_act         8192 x 7168, N(0,1), 0.5% of channels (35) x 100
"""
import ctypes
import os
import subprocess

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libworkloads.so")

WORKLOADS = {
    "tiny_ref": dict(seed=1, rows=256, hidden=2048, dist=0, scale=1.0,
                     row_gain_sigma=0.0, channel_frac=0.01, channel_mult=50.0),
    "moe_act": dict(seed=2, rows=8192, hidden=7168, dist=1, scale=1.0,
                    row_gain_sigma=0.5),
    "expert_weights": dict(seed=3, rows=32 * 2048, hidden=7168, dist=0,
                           scale=0.02, row_gain_sigma=0.0, elem_p=0.001,
                           elem_mult=20.0),
    "ragged_routed": dict(seed=4, rows=65536, hidden=2048, dist=0, scale=1.0,
                          row_gain_sigma=1.0, groups=64, tokens=8192, top_k=8),
    "resq_act": dict(seed=5, rows=8192, hidden=7168, dist=0, scale=1.0,
                     row_gain_sigma=0.0, channel_frac=0.005,
                     channel_mult=100.0),
}

_lib = None


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
           os.path.join(HERE, "gen.c"), "-lm", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, u64, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        L.wl_fill_rows.argtypes = [u64, i64, i64, i64, ctypes.c_int, d, d, d, d, vp, vp]
        L.wl_fill_rows.restype = None
        L.wl_pick_channels.argtypes = [u64, i64, i64, vp, vp]
        L.wl_pick_channels.restype = None
        L.wl_route_counts.argtypes = [u64, i64, ctypes.c_int, vp]
        L.wl_route_counts.restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def channel_multipliers(name: str):
    """FP32 per-channel multipliers (outlier channels) or None."""
    w = WORKLOADS[name]
    frac = w.get("channel_frac", 0.0)
    if frac <= 0.0:
        return None
    n = w["hidden"]
    count = int(np.floor(frac * n))
    picked = np.zeros(count, np.int64)
    scratch = np.zeros(n, np.int64)
    _L().wl_pick_channels(w["seed"], n, count, _p(picked), _p(scratch))
    mult = np.ones(n, np.float32)
    mult[picked] = w["channel_mult"]
    return mult


def fill_fp32(seed, row0, nrows, hidden, dist=0, scale=1.0, row_gain_sigma=0.0,
              elem_p=0.0, elem_mult=1.0, col_mult=None):
    out = np.empty((nrows, hidden), np.float32)
    cm = None if col_mult is None else np.ascontiguousarray(col_mult, np.float32)
    _L().wl_fill_rows(seed, row0, nrows, hidden, dist, scale, row_gain_sigma,
                      elem_p, elem_mult, _p(cm), _p(out))
    return out


def to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """FP32 array -> uint16 BF16 bit patterns via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rows(name: str, row0: int = 0, nrows: int = None) -> np.ndarray:
    """BF16 bit patterns (uint16 [nrows, hidden]) of rows [row0, row0+nrows)."""
    w = WORKLOADS[name]
    if nrows is None:
        nrows = w["rows"] - row0
    a = fill_fp32(w["seed"], row0, nrows, w["hidden"], w["dist"], w["scale"],
                  w["row_gain_sigma"], w.get("elem_p", 0.0),
                  w.get("elem_mult", 1.0), channel_multipliers(name))
    return to_bf16_bits(a)


def row_subset(name: str, indices) -> np.ndarray:
    """BF16 bits of the listed rows only (each row has its own stream)."""
    idx = np.asarray(indices, np.int64)
    w = WORKLOADS[name]
    out = np.empty((idx.shape[0], w["hidden"]), np.uint16)
    for j, r in enumerate(idx):
        out[j] = rows(name, int(r), 1)[0]
    return out


def tensor(name: str, device="cpu") -> torch.Tensor:
    """The whole workload as a torch.bfloat16 tensor [rows, hidden]."""
    bits = rows(name)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device != "cpu" else t


def group_offsets(name: str = "ragged_routed") -> np.ndarray:
    """int64 [groups + 1] exclusive prefix sum of the routed group sizes."""
    w = WORKLOADS[name]
    g = w["groups"]
    log2g = int(g).bit_length() - 1
    assert 1 << log2g == g
    counts = np.zeros(g, np.int64)
    _L().wl_route_counts(w["seed"], w["tokens"] * w["top_k"], log2g, _p(counts))
    assert counts.sum() == w["rows"]
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def random_rows(seed: int, nrows: int, hidden: int, dist=0, scale=1.0,
                row_gain_sigma=0.0, elem_p=0.0, elem_mult=1.0):
    """Free-form seeded rows (BF16 bits) for property tests."""
    return to_bf16_bits(fill_fp32(seed, 0, nrows, hidden, dist, scale,
                                  row_gain_sigma, elem_p, elem_mult))


def perturbed(x_bits: np.ndarray, seed: int, rel_sigma: float = 2.0 ** -8) -> np.ndarray:
    """A training-side copy of a rollout tensor: each BF16 value times
    (1 + rel_sigma * N(0, 1)), rounded back to BF16 (seeded; the draws come
    from numpy's PCG64)."""
    rng = np.random.default_rng(seed)
    x = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    noise = rng.standard_normal(x.shape).astype(np.float32)
    bf16_max = np.float32(3.3895313892515355e38)  # largest finite BF16: values stay finite
    with np.errstate(over="ignore"):
        y = x * (np.float32(1) + np.float32(rel_sigma) * noise)
    return to_bf16_bits(np.clip(y, -bf16_max, bf16_max))
