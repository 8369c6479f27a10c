"""Compile the test-only GPU libraries into tests/_build/: the conversion
probes, and libfp4q built with a launch limit of 4096 work-items so that
small calls exercise the split into several launches."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libprobes.so")
SPLIT_LIB_PATH = os.path.join(BUILD_DIR, "libfp4q_split4096.so")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
           "-shared", "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
           "-fno-gpu-flush-denormals-to-zero",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "fp4_block_quantization_amd", "csrc"),
           os.path.join(HERE, "probes.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "fp4q_lib_build", os.path.join(ROOT, "fp4_block_quantization_amd", "_build.py"))
    lib_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(lib_build)
    lib_build.build(verbose=verbose, extra_flags=["-DFP4Q_MAX_LAUNCH_ITEMS=4096"],
                    out_path=SPLIT_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
