"""Writes oracle_samples_n196.json: sampled fp64 oracle outputs on the tiny
Laplacian workload (14x14 grid, d=32, 2x2 pool).  Calls only the oracle and
the seeded input generator; rerun it only when the oracle's arithmetic is
changed on purpose (and say why in the commit)."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from nystr_linear_attention_amd import workloads as wl  # noqa: E402


def main():
    w = wl.WORKLOADS[0]
    x = wl.make_inputs(w)
    res = oracle.forward_workload(w, x, stages=True)[(0, 0)]
    rows = [0, 1, 13, 14, 97, 195]
    out = {
        "workload": w.name,
        "seed": w.seed,
        "rows": rows,
        "O_rows": res["O"][rows].tolist(),
        "L_row0": res["L"][0].tolist(),
        "A_diag": np.diag(res["A"]).tolist(),
        "X_trace": float(np.trace(res["X"])),
        "W_sum": float(res["W"].sum()),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_samples_n196.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
