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

Usage: python -m oracle.make_golden [--reuse-lse] [workload ...]
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


def compute(inp, progress=None) -> tuple[np.ndarray, dict]:
    """Every row's lse and the exact loss sum of one workload's inputs, from
    the oracle's row-blocked lse and its label-logit gather only."""
    w = inp.workload
    h = inp.hidden_f32()
    w64 = inp.weight_f32().astype(np.float64)
    b = inp.bias_f32()
    lse = O.lse_rows_blocked(h, None, b, block_rows=2048, weight64=w64, progress=progress)
    loss_sum, n_valid = O.loss_sum_from_lse(h, w64, b, inp.labels, lse, ignore_index=IGNORE_INDEX)
    meta = {
        "workload": w.name,
        "n_rows": w.n_rows, "hidden": w.hidden, "vocab": w.vocab,
        "n_valid": n_valid,
        "loss_sum": loss_sum,
        "ignore_index": IGNORE_INDEX,
        "inputs_sha256": inp.digest(),
        "made_by": "python -m oracle.make_golden " + w.name,
    }
    return lse, meta


def write(name: str, reuse_lse: bool = False) -> None:
    """Compute and store one workload's values. With ``reuse_lse`` the stored
    lse (written by an earlier run of this script) is kept and only the
    loss sum and the metadata are recomputed from it."""
    w = WORKLOADS[name]
    t0 = time.time()
    inp = make_inputs(w)
    print(f"[{name}] inputs ready in {time.time() - t0:.1f}s", flush=True)
    last = [time.time()]

    def progress(done, total):
        if time.time() - last[0] > 30:
            last[0] = time.time()
            print(f"[{name}] lse rows {done}/{total} ({time.time() - t0:.0f}s)", flush=True)

    lse_path = os.path.join(GOLDEN, f"lse_{name}.npy")
    if reuse_lse:
        old = json.load(open(os.path.join(GOLDEN, f"{name}.json")))
        if old["inputs_sha256"] != inp.digest():
            raise RuntimeError(f"{name}: inputs changed since the stored lse was written")
        lse = np.load(lse_path)
        loss_sum, n_valid = O.loss_sum_from_lse(inp.hidden_f32(), inp.weight_f32(), inp.bias_f32(), inp.labels,
                                                lse, ignore_index=IGNORE_INDEX)
        meta = dict(old, n_valid=n_valid, loss_sum=loss_sum,
                    made_by="python -m oracle.make_golden " + name + " (loss sum: --reuse-lse)")
    else:
        lse, meta = compute(inp, progress)
        meta["seconds"] = round(time.time() - t0, 1)
        np.save(lse_path, lse)
    with open(os.path.join(GOLDEN, f"{name}.json"), "w") as f:
        json.dump(meta, f, indent=1)
    print(f"[{name}] done: {meta}", flush=True)


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    for n in (args or LARGE):
        write(n, reuse_lse="--reuse-lse" in sys.argv)
