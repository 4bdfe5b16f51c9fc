"""Write stored expected values for the full-size workloads (test infrastructure).

Calls only the oracle and the seeded input generators. For each large
workload it stores, under ``tests/golden/``:

* ``lse_<name>.npy``: float64 lse_i of every row (row-blocked float64 pass);
* ``<name>.json``: n_valid, the exact total loss (sum of l_i), the sha256 of
  the generated input bits (so a test can tell if the generator drifted),
  and the command that made it.

The GPU tests need every row's lse to evaluate grad_weight on a subset of
vocabulary ids (grad_weight[j] sums over all rows), and recomputing it takes
tens of CPU-minutes, so it is computed once here.

Usage: python -m oracle.make_golden [workload ...]
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

from lce_inputs import IGNORE_INDEX, WORKLOADS, make_inputs
from oracle import lce_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden")
LARGE = ["qwen3_4b_32k", "qwen3_8b_1m_shard", "qwen3_4b_160k"]


def write(name: str) -> None:
    w = WORKLOADS[name]
    t0 = time.time()
    inp = make_inputs(w)
    h = inp.hidden_f32()
    w64 = inp.weight_f32().astype(np.float64)
    b = inp.bias_f32()
    print(f"[{name}] inputs ready in {time.time() - t0:.1f}s", flush=True)
    last = [time.time()]

    def progress(done, total):
        if time.time() - last[0] > 30:
            last[0] = time.time()
            print(f"[{name}] lse rows {done}/{total} ({time.time() - t0:.0f}s)", flush=True)

    lse = O.lse_rows_blocked(h, None, b, block_rows=2048, weight64=w64, progress=progress)
    valid = O.valid_rows(inp.labels, w.vocab)
    rows = np.flatnonzero(valid)
    zy = np.einsum("ij,ij->i", h[rows].astype(np.float64), w64[inp.labels[rows]])
    if b is not None:
        zy += b.astype(np.float64)[inp.labels[rows]]
    row_loss = np.zeros(w.n_rows)
    row_loss[rows] = lse[rows] - zy
    meta = {
        "workload": name,
        "n_rows": w.n_rows, "hidden": w.hidden, "vocab": w.vocab,
        "n_valid": int(valid.sum()),
        "loss_sum": float(np.sum(row_loss)),
        "ignore_index": IGNORE_INDEX,
        "inputs_sha256": inp.digest(),
        "made_by": "python -m oracle.make_golden " + name,
        "seconds": round(time.time() - t0, 1),
    }
    np.save(os.path.join(GOLDEN, f"lse_{name}.npy"), lse)
    with open(os.path.join(GOLDEN, f"{name}.json"), "w") as f:
        json.dump(meta, f, indent=1)
    print(f"[{name}] done: {meta}", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or LARGE):
        write(n)
