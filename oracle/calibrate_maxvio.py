"""Find the router-bias strength beta that gives the MoonEP-shape workload a target maxvio.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): run by hand, never by
the HIP library.  Writes ``synth/maxvio_beta.json``, which the seeded input
generators read to build the skewed workloads.

The workload is the single-GPU share of the MoonEP benchmark shape (S=8192,
E=384, H=7168, K=8).  Its router adds bias_e = -beta * ln(1 + pi(e)) to every
token's logits, pi a seeded permutation of the experts, so expert pi^-1(0) is
the hot one.  maxvio = max_e c_e / (S K / E) - 1 is the load-skew measure of
the MoonEP page ("Moonshot AI opened MoonEP...", step-by-step guide, the
problem statement and its benchmark step); 0 is perfect balance.

The routing is the oracle's: float64 logits rounded to float32 (the width the
GPU router produces) and the oracle's top-K with its tie rule.  maxvio is not
continuous in beta (counts are integers), so the bisection stops at the first
beta whose maxvio lies within 1% of the target (0.005 absolute for small
targets) or after 60 halvings, and the table records the maxvio reached.

A level below the natural skew of the unbiased router (about 0.34 here: the
columns of W_g differ in norm, so some experts win more often) cannot be
reached by the one-parameter skew.  For such a level the table stores a
per-expert balancing bias instead: starting from zero, each expert's bias is
lowered by eta * ln((c_e + 1) / (mean + 1)) per iteration (overloaded experts
down, idle ones up), and the first vector whose maxvio is within the tolerance
of the target (or the closest after 400 iterations) is kept.

    python -m oracle.calibrate_maxvio            # levels 0.2 1 10 20
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle.moe import expert_counts, maxvio, router_logits, topk_experts  # noqa: E402
from synth.inputs import CONFIGS, make_workload, zipf_bias  # noqa: E402

OUT = os.path.join(ROOT, "synth", "maxvio_beta.json")


def maxvio_at(base, E, K, beta, seed):
    """maxvio of the oracle routing with bias strength beta on precomputed unbiased logits."""
    bias = zipf_bias(E, beta, seed).astype(np.float64)
    logits = (base + bias[None, :]).astype(np.float32)
    counts, _ = expert_counts(topk_experts(logits, K), E)
    return float(maxvio(counts))


def maxvio_vec(base, E, K, bias):
    logits = (base + bias.astype(np.float32).astype(np.float64)[None, :]).astype(np.float32)
    counts, _ = expert_counts(topk_experts(logits, K), E)
    return float(maxvio(counts)), counts


def balance(base, E, K, target, tol, eta=0.05, iters=400):
    """Per-expert bias that lowers maxvio to the target (see the module docstring)."""
    b = np.zeros(E, np.float64)
    best = None
    for _ in range(iters):
        v, counts = maxvio_vec(base, E, K, b)
        if best is None or abs(v - target) < abs(best[1] - target):
            best = (b.astype(np.float32).copy(), v)
        if abs(v - target) <= tol:
            break
        mean = counts.mean()
        b = b - eta * np.log((counts + 1.0) / (mean + 1.0))
    return best


def calibrate(levels, name="c4"):
    cfg = CONFIGS[name]
    wl = make_workload(name, beta=0.0, host_weights=False)
    E, K, seed = wl.E, wl.K, cfg["seed"]
    # x Wg accumulated in float64; the bias is added per level (same sum order
    # as the oracle's router_logits, which adds it after the product)
    base = router_logits(wl.x, wl.Wg, None, out_dtype=np.float64)
    natural = maxvio_at(base, E, K, 0.0, seed)
    print(f"beta=0: maxvio {natural:.4f}", flush=True)
    table = {"workload": cfg["workload"], "natural_maxvio": natural, "beta": {}, "reached": {},
             "bias": {}}
    for t in levels:
        tol = max(0.01 * t, 0.005)
        if t < natural - tol:
            vec, v = balance(base, E, K, t, tol)
            table["bias"][f"{t:g}"] = [float(z) for z in vec]
            table["beta"][f"{t:g}"], table["reached"][f"{t:g}"] = 0.0, v
            print(f"target {t:g}: balancing bias -> maxvio {v:.4f}", flush=True)
            continue
        lo, hi = 0.0, 1.0
        while maxvio_at(base, E, K, hi, seed) < t:
            lo, hi = hi, hi * 2.0
        best = (hi, maxvio_at(base, E, K, hi, seed))
        for _ in range(60):
            mid = 0.5 * (lo + hi)
            v = maxvio_at(base, E, K, mid, seed)
            if abs(v - t) < abs(best[1] - t):
                best = (mid, v)
            if abs(v - t) <= tol:
                break
            if v < t:
                lo = mid
            else:
                hi = mid
        table["beta"][f"{t:g}"], table["reached"][f"{t:g}"] = best[0], best[1]
        print(f"target {t:g}: beta {best[0]:.6f} -> maxvio {best[1]:.4f}", flush=True)
    return table


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("levels", nargs="*", type=float, default=[0.2, 1.0, 10.0, 20.0])
    args = ap.parse_args()
    table = calibrate(args.levels)
    with open(OUT, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
