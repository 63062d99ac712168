"""Reader for the small text fixtures under tests/golden."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_case(name):
    """key value... lines; repeated keys stack into a 2-D array."""
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            rows.setdefault(key, []).append([float(v) for v in vals])
    out = {}
    for k, v in rows.items():
        a = np.array(v)
        out[k] = a[0] if a.shape[0] == 1 else a
    return out


def load_pack_lines():
    cases = []
    with open(os.path.join(GOLDEN, "pack_words.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            b, codes, words = [p.strip() for p in line.split("|")]
            cases.append((int(b), [int(c) for c in codes.split()], [int(w, 16) for w in words.split()]))
    return cases
