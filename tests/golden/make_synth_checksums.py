"""Write synth_checksums.json: SHA-256 of every array of the five seeded workloads.

Run from the repository root: python tests/golden/make_synth_checksums.py
It calls only the input generator (no oracle, no GPU code); the test compares the
generator's current bytes against these digests so that a change of workload is never
silent.
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from synth import config_case  # noqa: E402


def digests(case):
    out = {}
    for field, val in sorted(vars(case).items()):
        if isinstance(val, np.ndarray):
            out[field] = hashlib.sha256(np.ascontiguousarray(val).tobytes()).hexdigest()
    return out


def main():
    res = {f"C{k}": digests(config_case(k)) for k in range(5)}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "synth_checksums.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    print("wrote", path)


if __name__ == "__main__":
    main()
