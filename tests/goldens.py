"""Parser for the hand-worked fixtures under tests/golden/."""
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bf16_exact(v: float) -> int:
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    assert u & 0xFFFF == 0, "fixture value %r is not an exact BF16" % v
    assert struct.unpack("<f", struct.pack("<I", u))[0] == v or v != v
    return u >> 16


def load(name):
    """Return {case_name: {field: value}} with x as uint16 BF16 bits and byte
    fields as numpy arrays."""
    cases = {}
    cur = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("[case ") and line.endswith("]"):
                cur = cases.setdefault(line[6:-1], {})
                continue
            key, val = [p.strip() for p in line.split(":", 1)]
            if key == "x":
                cur[key] = np.array([_bf16_exact(float(t)) for t in val.split()], np.uint16)
            elif key in ("dequant",):
                cur[key] = np.array([int(t, 16) for t in val.split()], np.uint16)
            elif key == "token_scale_bits":
                cur[key] = int(val, 16)
            elif key in ("four_over_six", "hidden"):
                cur[key] = int(val)
            elif key.startswith("err"):
                cur[key] = float(val)
            else:
                cur[key] = np.array([int(t, 16) for t in val.split()], np.uint8)
    return cases
