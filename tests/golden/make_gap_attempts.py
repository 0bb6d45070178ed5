"""Write tests/golden/gap_attempts.json: per workload, the redraw index of every
token row whose first draw leaves the 8th and 9th router probabilities closer
than 1e-3.

The gap is measured with the CPU oracle (double precision, on the rounded
inputs the GPU receives): token rows are redrawn with the next attempt index
until sigmoid(z_8) - sigmoid(z_9) > 1e-3.  Only the oracle and the input
generator are called.  For the stacked workload only the first layer's input
is filtered (later layers' inputs are computed, not drawn).

Usage:  python tests/golden/make_gap_attempts.py  [names...]
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def attempts_for(name, max_attempts=64):
    cfg = synth.CONFIGS[name]
    T, D, E, K = cfg["T"], cfg["D"], cfg["E"], cfg["K"]
    wr = synth.normal(synth.key(cfg, 0, synth.WR), E, D, 1.0 / np.sqrt(D), cfg["dtype"])
    b = synth.bias(cfg, 0)
    att = np.zeros(T, np.int32)
    todo = np.arange(T)
    first_fail = None
    for _ in range(max_attempts):
        x = synth.x_rows(cfg, att)
        z = oracle.router_logits(x[todo], wr, b, len(todo), D, E)
        gap = oracle.sigma_gap(z, K)
        bad = todo[gap <= synth.GAP_MIN]
        if first_fail is None:
            first_fail = int(len(bad))
        if len(bad) == 0:
            break
        att[bad] += 1
        todo = bad
    else:
        raise RuntimeError(f"{name}: tokens still inside the gap after {max_attempts} draws")
    x = synth.x_rows(cfg, att)
    gap = oracle.sigma_gap(oracle.router_logits(x, wr, b, T, D, E), K)
    return att, float(gap.min()), first_fail


def main(names):
    path = os.path.join(HERE, "gap_attempts.json")
    table = {}
    if os.path.exists(path):
        with open(path) as f:
            table = json.load(f)
    for name in names:
        att, gmin, nfail = attempts_for(name)
        table[name] = {
            "attempts": {str(t): int(a) for t, a in enumerate(att) if a},
            "min_gap": gmin,
            "tokens_redrawn": nfail,
            "T": int(len(att)),
            "note": "written by tests/golden/make_gap_attempts.py with the oracle; seed 0",
        }
        print(f"{name}: {nfail}/{len(att)} rows redrawn, min sigma gap {gmin:.3e}", flush=True)
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(synth.CONFIGS))
