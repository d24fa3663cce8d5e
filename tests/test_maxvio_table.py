"""The stored router-bias table reproduces its maxvio levels under the oracle's routing.

The table (synth/maxvio_beta.json) is written by oracle/calibrate_maxvio.py;
this re-derives each level's counts from the seeded inputs with the oracle's
float64 router and top-K, so a stale or hand-edited table fails here.
"""
import json
import os

import numpy as np
import pytest

import oracle
from synth import make_workload
from synth.inputs import _BETA_FILE


@pytest.fixture(scope="module")
def base_logits():
    wl = make_workload("c4", beta=0.0, host_weights=False)
    return wl, oracle.router_logits(wl.x, wl.Wg, None, out_dtype=np.float64)


def test_table_levels_reproduce(base_logits):
    wl0, base = base_logits
    assert os.path.exists(_BETA_FILE)
    with open(_BETA_FILE) as f:
        table = json.load(f)
    mean = wl0.S * wl0.K / wl0.E
    for level, reached in table["reached"].items():
        wl = make_workload("c4", S=None, maxvio=float(level), host_weights=False)
        np.testing.assert_array_equal(wl.x, wl0.x)
        logits = (base + wl.bias.astype(np.float64)[None, :]).astype(np.float32)
        counts, cu = oracle.expert_counts(oracle.topk_experts(logits, wl.K), wl.E)
        assert cu[-1] == wl.S * wl.K
        mv = oracle.maxvio(counts)
        # one flipped pick moves the hot expert's count by one row
        assert abs(mv - reached) <= 2.0 / mean, (level, mv, reached)
        assert abs(mv - float(level)) <= max(0.02 * float(level), 0.02), (level, mv)
