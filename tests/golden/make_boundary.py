"""Writes down_proj_boundary.json: the oracle's boundary-search v_s for the down_proj sweep.

Calls only the seeded input generator and the CPU oracle.  Workload: LLaMA-7B
down_proj 4096x11008 with 5% outlier columns x10, importance W*W, tile_rows 64,
seed 0, t_s in {0.6, 0.7, 0.8} (FlexHiNM-GP notes, key design 1: search v_s
from t_s downwards, stop at the first decrease of the retained importance).
Run from the repository root:  python tests/golden/make_boundary.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle.hinm as oh  # noqa: E402
import synth  # noqa: E402


def main():
    out = {"workload": "down_proj 4096x11008, 5% outlier columns x10, importance W*W, tile_rows 64, seed 0",
           "step": 0.01, "results": []}
    for t_s in (0.6, 0.7, 0.8):
        w = synth.down_proj_sweep(t_s)
        v, trace = oh.boundary_search(w.importance.numpy(), w.perm.numpy(), w.cout, w.cin, 64, t_s)
        p = oh.plan(w.cout, w.cin, 64, t_s, v)
        out["results"].append({"t_s": t_s, "v_s": v, "n_dense": p.n_dense, "n_24": p.n_24,
                               "n_pruned": p.n_pruned, "trace": [[a, b] for a, b in trace]})
        print(t_s, v, p.n_dense, p.n_24, p.n_pruned, len(trace), flush=True)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "down_proj_boundary.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
