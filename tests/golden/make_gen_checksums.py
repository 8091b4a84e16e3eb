"""Writes tests/golden/gen_checksums.json: SHA-256 of every array the seeded
generators build for the five workloads at seed 0 (pattern, values and the
dense operands), so that a change in any generator, or in the libraries it
draws from, shows up as a failing pin.  Run from the repository root:
    python tests/golden/make_gen_checksums.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from unstructured_sparse_linear_amd import gen  # noqa: E402

KEYS = {1: ["A", "B", "Ad", "BT", "W"], 2: ["A", "B", "Ad", "BT", "W"],
        3: ["A", "B", "Ad", "BT"], 4: ["A", "B1", "B", "Ad", "BT"],
        5: ["A", "B", "Ad", "BT"]}


def digest(x: np.ndarray) -> str:
    x = np.ascontiguousarray(x)
    h = hashlib.sha256()
    h.update(str(x.dtype).encode() + str(x.shape).encode())
    h.update(x.tobytes())
    return h.hexdigest()


def checksums():
    out = {}
    for cfg, keys in KEYS.items():
        for dt in ((None, "bf16") if cfg == 3 else (None,)):
            w = gen.make_config(cfg, dt=dt)
            ent = {}
            for k in keys:
                a = w.get(k)
                if isinstance(a, gen.CSR):
                    ent[k + ".row_offsets"] = digest(a.row_offsets)
                    ent[k + ".col_idx"] = digest(a.col_idx)
                    ent[k + ".values"] = digest(a.values)
                else:
                    ent[k] = digest(a)
            out[w.name if cfg == 3 else gen.CONFIG_NAMES[cfg]] = ent
    return out


if __name__ == "__main__":
    path = os.path.join(ROOT, "tests", "golden", "gen_checksums.json")
    with open(path, "w") as f:
        json.dump(checksums(), f, indent=1, sort_keys=True)
    print("wrote", path)
