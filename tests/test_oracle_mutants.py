"""The pins catch plausible mistakes in the oracle.

Each case below plants one mistake in a copy of oracle/fp4_oracle.c (on the
CPU, by text substitution), builds it with the oracle's own flags, and runs
the oracle pin suite against that build (FP4Q_ORACLE_LIB); the suite must
fail.  The unmodified copy, built the same way, must pass.  The cases are
the slips one could make while writing the oracle from the pages: a tie
direction, a constant, a comparison, a dropped sign or rounding, a wrong
operand order, a wrong scale."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fp4_oracle.c")
OUT = os.path.join(ROOT, "tests", "_build", "mutants")
# fastest first: a mutant stops the run at its first failing pin
PINS = ["tests/test_oracle_golden.py", "tests/test_oracle_trace.py",
        "tests/test_oracle_global.py", "tests/test_oracle_resq.py",
        "tests/test_oracle_properties.py", "tests/test_oracle_fp16.py",
        "tests/test_oracle_primitives.py"]

MUTANTS = {
    "e2m1_tie_0_75_down": ("q += (a >= 0.75f);", "q += (a > 0.75f);"),
    "e2m1_tie_5_up": ("q += (a > 5.0f);", "q += (a >= 5.0f);"),
    "token_scale_constant": ("float s = amax / (four_over_six ? 1536.0f : 2688.0f); /* 1 and 2",
                             "float s = amax / (four_over_six ? 1792.0f : 2688.0f); /* 1 and 2"),
    "ties_pick_4": ("out->choice = (four_over_six && out->err[1] < out->err[0]) ? 4 : 6;",
                    "out->choice = (four_over_six && out->err[1] <= out->err[0]) ? 4 : 6;"),
    "candidate_sign_dropped": ("      if (negative) c = -c;\n      float delta", "      float delta"),
    "candidate_rounding_order": ("      float ge = oracle_e2m1_value(q) * e; /* exact: <= 6 significant bits */\n      float c = ge * s;",
                                 "      float ge = oracle_e2m1_value(q) * e; /* exact: <= 6 significant bits */\n      float c = oracle_e2m1_value(q) * (e * s); (void)ge;"),
    "error_is_l1": ("      float sq = delta * delta;\n      err = err + sq;",
                    "      float sq = fabsf(delta);\n      err = err + sq;"),
    "e4m3_truncates": ("  double v = lo * step;\n  if (v > 448.0) v = 448.0;",
                       "  lo = floor(n);\n  double v = lo * step;\n  if (v > 448.0) v = 448.0;"),
    "bf16_truncates": ("  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;", ""),
    "mx_exponent_off_by_one": ("int k = (ex - 1) - 2;", "int k = (ex - 1) - 1;"),
    "s24_ties_to_higher_index": ("if (i0 < 0 || (grp[i] & 7) > (grp[i0] & 7)) i0 = i;",
                                 "if (i0 < 0 || (grp[i] & 7) >= (grp[i0] & 7)) i0 = i;"),
    # (the FP16 rounding of y - g e is exact -- |y - g e| <= y and g e has no
    # bits below y's last place -- so dropping it is not an observable mistake)
    "fp16_target_not_rounded": ("double y = oracle_fp16_rne((double)scaled);",
                                "double y = (double)scaled;"),
    "guided_picks_farther": ("q = (dhi < dlo) ? hi : lo;", "q = (dhi > dlo) ? hi : lo;"),
    "unguided_truncates": ("nearest = oracle_e2m1_code(v);", "nearest = lo;"),
    "reconstruct_wrong_scale": ("rv = mx_value((i % 2) ? (rb >> 4) : (rb & 15), res_scales[blk]);",
                                "rv = mx_value((i % 2) ? (rb >> 4) : (rb & 15), scales[blk]);"),
    "global_scale_constant": ("  float s = amax / (four_over_six ? 1536.0f : 2688.0f);\n  *tensor_scale = s;",
                              "  float s = amax / 2688.0f;\n  *tensor_scale = s;"),
}


def build_variant(name, text):
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    os.makedirs(OUT, exist_ok=True)
    src = os.path.join(OUT, name + ".c")
    with open(src, "w") as f:
        f.write(text)
    lib = os.path.join(OUT, "liboracle_%s.so" % name)
    subprocess.run(["gcc", *ob.CFLAGS, "-I", os.path.join(ROOT, "oracle"), src, "-lm", "-o", lib],
                   check=True, stderr=subprocess.DEVNULL)
    return lib


def run_pins(lib):
    env = dict(os.environ, FP4Q_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *PINS], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=900)
    return r.returncode, r.stdout.decode(errors="replace")[-400:]


def test_unmodified_copy_passes():
    code, tail = run_pins(build_variant("original", open(SRC).read()))
    assert code == 0, tail


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation site not found: %s" % name
    code, tail = run_pins(build_variant(name, text.replace(old, new, 1)))
    assert code != 0, "the pins did not catch mutant %s" % name
