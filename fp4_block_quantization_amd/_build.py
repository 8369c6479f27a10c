"""Compile the gfx950 HIP library libfp4q.so in-tree (no JIT cache).

Flags that the bit-exact contract depends on:
  -ffp-contract=off            no FMA contraction of a*b+c
  -fhip-fp32-correctly-rounded-divide-sqrt
                               IEEE-rounded FP32 division
  -fno-gpu-flush-denormals-to-zero
                               FP32 subnormals kept
  -target-feature -packed-fp32-ops
                               no packed FP32 instructions
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libfp4q.so")
# the same sources with the per-block arithmetic compiled out
# (-DFP4Q_STANDIN=1): memory-pattern stand-ins, for measurement only
STANDIN_PATH = os.path.join(BUILD_DIR, "libfp4q_standin.so")
# the same sources deciding every 4/6 block from both exactly computed errors
# (-DFP4Q_NV_CERTIFY=0, the straightforward FP32 decision): measurement only
EXACTDECISION_PATH = os.path.join(BUILD_DIR, "libfp4q_exactdecision.so")
# K0, the HBM probes (copy, read-only, write-only)
MEMBENCH_PATH = os.path.join(BUILD_DIR, "libfp4q_membench.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["nvfp4.hip", "mxfp4_resq.hip", "fp4q_api.cpp"]
MEMBENCH_SOURCES = ["membench.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra_flags=(), out_path: str = None, sources=None) -> str:
    """Compile the sources (default: the quantizer's) and link libfp4q.so (or
    out_path, with extra_flags such as -D build knobs); returns the library
    path."""
    out_path = out_path or LIB_PATH
    sources = sources or SOURCES
    obj_dir = os.path.join(os.path.dirname(out_path), "obj_" + os.path.basename(out_path))
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    for src in sources:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, *HIP_FLAGS, *extra_flags, *lang, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build_all(verbose: bool = False):
    """libfp4q.so, the stand-in and exact-decision builds and the K0 probes."""
    return [build(verbose), build(verbose, ["-DFP4Q_STANDIN=1"], STANDIN_PATH),
            build(verbose, ["-DFP4Q_NV_CERTIFY=0"], EXACTDECISION_PATH),
            build(verbose, out_path=MEMBENCH_PATH, sources=MEMBENCH_SOURCES)]


if __name__ == "__main__":
    print(build_all(verbose=True))
