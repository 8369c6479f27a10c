"""Every build-time knob of the HIP sources still compiles at its
non-default settings (device code for gfx950, compile only).  The knobs
select alternatives that were measured against the defaults -- load and
store paths, units per lane, launch shapes -- and are kept so that they can
be measured again; this keeps them buildable."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from fp4_block_quantization_amd import _build

KNOBS = {
    "nvfp4.hip": ["FP4Q_NV_NT_STORES=0", "FP4Q_NV_NT_BYTES=0", "FP4Q_NV_NT_BYTES=1",
                  "FP4Q_NV_NT_CODES=0", "FP4Q_NV_NT_CODES=1", "FP4Q_NV_NT_LOADS=0",
                  "FP4Q_NV_LDS_DQ=0", "FP4Q_NV_WG_WAVES=2", "FP4Q_NV_LDS_LOAD=0",
                  "FP4Q_NV_NB=1", "FP4Q_NV_NB=3", "FP4Q_NV_NB=4", "FP4Q_DQ_UNITS=1",
                  "FP4Q_DQ_UNITS=2", "FP4Q_GUIDED_UNITS=2", "FP4Q_DQ_NT_STORES=0", "FP4Q_DQ_NT_LOADS=3",
                  "FP4Q_GUIDED_NT_LOADS=0", "FP4Q_GUIDED_NT_LOADS=3", "FP4Q_GAMAX_NT=1",
                  "FP4Q_GAMAX_DEPTH=2", "FP4Q_GAMAX_GRID=256", "FP4Q_NV_STREAM=1",
                  "FP4Q_NV_STREAM_DEFER=0", "FP4Q_NV_STREAM_GRID=4096", "FP4Q_STANDIN=1",
                  "FP4Q_NV_DQ_POLICY=2", "FP4Q_NV_DQ_POLICY=-1", "FP4Q_NV_NT_POLICY=18",
                  "FP4Q_NV_PLAIN_POLICY=-1", "FP4Q_DQ_POLICY=19", "FP4Q_NV_LOAD_AUX=18",
                  "FP4Q_GLOBAL_REVERSE=0", "FP4Q_GLOBAL_LOAD_AUX=0", "FP4Q_GAMAX_THREADS=1024",
                  "FP4Q_GAMAX_CHUNKED=0", "FP4Q_NV_FLOAT_MAX=0", "FP4Q_NV_SCALE_NT_POLICY=16",
                  "FP4Q_NV_SCALE_PLAIN_POLICY=16", "FP4Q_GUIDED_CODE_POLICY=16",
                  "FP4Q_RTN_CODE_POLICY=2", "FP4Q_NV_CERTIFY=0"],
    "mxfp4_resq.hip": ["FP4Q_MX_LDS_STAGE=0", "FP4Q_MX_NT_LOADS=0", "FP4Q_MX_NT_STORES=0",
                       "FP4Q_MX_NT_SMALL=1", "FP4Q_MX_UNITS=1", "FP4Q_MX_UNITS=2",
                       "FP4Q_MX_UNITS=8", "FP4Q_MX_REC_STAGE=0", "FP4Q_MX_REC_NT=0",
                       "FP4Q_STANDIN=1", "FP4Q_MX_POLICY=18", "FP4Q_MX_SMALL_POLICY=18",
                       "FP4Q_MX_REC_POLICY=2", "FP4Q_MX_WG_WAVES=8", "FP4Q_MX_WG_WAVES=16",
                       "FP4Q_MX_FLOAT_MAX=0", "FP4Q_MX_STAGED_SMALL_POLICY=2"],
    "membench.hip": ["FP4Q_K0_UNITS=8", "FP4Q_K0_UNITS=16"],
}


def _compile(job, out_dir):
    src, knob = job
    out = os.path.join(out_dir, "%s_%s.o" % (src.split(".")[0], knob.replace("=", "_")))
    cmd = [_build.HIPCC, *_build.HIP_FLAGS, "--cuda-device-only", "-D" + knob,
           "-I", os.path.join(_build.ROOT, "include"), "-I", _build.CSRC,
           "-c", os.path.join(_build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return job, r.returncode, r.stderr


def test_every_knob_compiles(tmp_path):
    if not os.path.exists(_build.HIPCC):
        pytest.skip("hipcc not available")
    jobs = [(src, k) for src, ks in KNOBS.items() for k in ks]
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda j: _compile(j, str(tmp_path)), jobs))
    failed = [(job, err[-2000:]) for job, rc, err in results if rc != 0]
    assert not failed, failed
