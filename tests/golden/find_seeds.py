"""Finds the seeds of the naturally routed workloads ("tiny", "prefill").

Calls only the oracle's router on the generator's inputs.  Conditions (from
the workload description): every complete chunk's score margin |s_sm - s_lin|
exceeds 1e-3 (so a correct router's decision is never a coin flip), both
routes occur, and for "prefill" the softmax share lies in [0.45, 0.55].
Prints the first qualifying seed at or above each workload's base seed; the
result is recorded in workloads.WORKLOADS and re-checked by the tests.

    python tests/golden/find_seeds.py
"""
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))
import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as W  # noqa: E402

CONDITIONS = {"tiny": (1e-3, None), "prefill": (1e-3, (0.45, 0.55))}


def ok(name, seed):
    wl = W.WORKLOADS[name]
    inp = W.make_prefill(wl, seed=seed, routing="natural")
    r, m = oracle.route(inp["x"], inp["w_score"], inp["b_score"])
    min_margin, frac = CONDITIONS[name]
    f = float((r == oracle.SM).mean())
    good = np.abs(m).min() > min_margin and 0 < f < 1
    if frac is not None:
        good = good and frac[0] <= f <= frac[1]
    return good, float(np.abs(m).min()), f


if __name__ == "__main__":
    for name, base in (("tiny", 0), ("prefill", 1)):
        s = base
        while True:
            good, mm, f = ok(name, s)
            print(f"{name} seed {s}: min|margin| {mm:.2e} sm_frac {f:.3f} {'OK' if good else ''}", flush=True)
            if good:
                break
            s += 100
