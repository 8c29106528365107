"""Writes the stored query-draw attempt tables tests/golden/gap_attempts/<workload>.json of the five workloads.

Each table holds, per decode step t, sequence b and KV head g, the first draw attempt of that group's query step for
which the oracle's plain block scores of the stored bytes have a relative gap above 1e-4 at the K-th/(K+1)-th
boundary (tests/gap_search.py). The input generator draws the queries by these attempts, so the selection must match
the oracle exactly on every instance that is not counted as banded. Only the oracle and the seeded input generator
are used.

    python tests/golden/make_gap_attempts.py [workload ...]      (default: all five)
"""
from __future__ import annotations

import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from dynamic_sparse_attention_decode_amd.inputs import WORKLOADS  # noqa: E402
from tests.gap_search import REL_GAP, search  # noqa: E402

CAP = 1024


def table_path(name: str) -> str:
    return os.path.join(HERE, "gap_attempts", f"{name}.json")


def make(name: str) -> dict:
    w = WORKLOADS[name]
    t0 = time.time()
    attempts, gaps = search(w, cap=CAP)
    banded = int((gaps <= REL_GAP).sum())
    d = {
        "name": name,
        "workload": w.key(),
        "rule": "first attempt per (step, sequence, KV head) whose plain-score relative gap at the K-th boundary "
                "exceeds 1e-4; after 1024 attempts the widest-gap one (counted as banded)",
        "cap": CAP,
        "shape": list(attempts.shape),
        "instances": int(attempts.size),
        "banded": banded,
        "min_gap": float(gaps.min()),
        "mean_attempt": float(attempts.mean()),
        "max_attempt": int(attempts.max()),
        "command": f"python tests/golden/make_gap_attempts.py {name}",
        "attempts": attempts.ravel().tolist(),
    }
    with open(table_path(name), "w") as f:
        json.dump(d, f, separators=(",", ":"))
        f.write("\n")
    print(f"{name}: {attempts.size} instances, banded {banded}, mean attempt {attempts.mean():.2f}, "
          f"max {attempts.max()}, min gap {gaps.min():.3e} ({time.time() - t0:.1f} s)", flush=True)
    return d


if __name__ == "__main__":
    for n in sys.argv[1:] or list(WORKLOADS):
        make(n)
