"""GPU parity of the Mixture-of-Depths block (select -> MoE -> merge, and its backward).

Through the C ABI against the oracle: the score r to 1e-5 (fp32 from exact
bf16 inputs on both sides), the keep set bit for bit (the oracle selects
from the GPU's fp32 scores, so both take the integer decision in the same
precision), xk bitwise, and every float output normwise to 2e-2 (bf16
storage).  The oracle chain is: MoE forward on x[keep] with the routing
re-selected from the GPU's logits, merge, then dm = r dout on the kept
rows, the MoE backward on dm, and the merge/score backward.
"""
import sys

import numpy as np
import pytest

import oracle
from synth import make_workload
from tests.moe_testutil import BF16_TOL, F32_TOL, assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from routing_dispatch_grouped_moe_amd import MoDMoELayer  # noqa: E402
from routing_dispatch_grouped_moe_amd import _lib as L  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_and_check(wl, C=None, zero_scores=False, flags=L.MOE_F_RENORM):
    B, T = wl.cfg["B"], wl.cfg["T"]
    C = wl.cfg["C"] if C is None else C
    H, Hf, E, K = wl.H, wl.Hf, wl.E, wl.K
    w_r = np.zeros_like(wl.w_r) if zero_scores else wl.w_r
    dev = lambda a: to_dev(a, "bf16")  # noqa: E731
    x, wr_t, Wg = dev(wl.x), dev(w_r), dev(wl.Wg)
    W1, W3, W2, dout = dev(wl.W1), dev(wl.W3), dev(wl.W2), dev(wl.dout)
    layer = MoDMoELayer(B, T, C, H, Hf, E, K, "bf16", flags=flags)
    renorm = bool(flags & L.MOE_F_RENORM)
    L.moe_clear_status(layer.moe.ws)
    layer.forward(x, wr_t, Wg, None, W1, W3, W2)
    layer.backward(dout, x, wr_t, Wg, W1, W3, W2)
    torch.cuda.synchronize()
    assert layer.moe.status() == 0

    r = to_host(layer.r)
    assert_close("r", r, oracle.mod_scores(wl.x, w_r), F32_TOL)
    keep = oracle.mod_keep(r, B, T, C)
    np.testing.assert_array_equal(to_host(layer.keep)[:B * C], keep, err_msg="keep_idx")
    xk = np.asarray(wl.x)[keep]
    np.testing.assert_array_equal(to_host(layer.xk), xk, err_msg="xk")

    logits = to_host(layer.moe.logits)
    idx = oracle.topk_experts(logits, K)
    np.testing.assert_array_equal(to_host(layer.moe.topk_idx), idx, err_msg="topk_idx")
    fw = oracle.moe_forward(xk, wl.Wg, None, wl.W1, wl.W3, wl.W2, K, idx=idx, logits=logits,
                            renorm=renorm)
    m = fw["out"]
    assert_close("m (MoE out)", to_host(layer.moe.out), m, BF16_TOL)
    out = oracle.mod_merge(wl.x, r, keep, m)
    got_out = to_host(layer.out)
    assert_close("out", got_out, out, BF16_TOL)
    dropped = np.setdiff1d(np.arange(B * T), keep)
    np.testing.assert_array_equal(got_out[dropped], np.asarray(wl.x)[dropped],
                                  err_msg="dropped tokens must pass through unchanged")

    dm, dr, _, _ = oracle.mod_backward(wl.x, w_r, r, keep, m, wl.dout, None)
    bw = oracle.moe_backward(fw, dm, xk, wl.Wg, wl.W1, wl.W3, wl.W2, K, renorm=renorm)
    _, _, dx, dw_r = oracle.mod_backward(wl.x, w_r, r, keep, m, wl.dout, bw["dx"])
    errs = {}
    errs["dm"] = assert_close("dm", to_host(layer.dm), dm, BF16_TOL)
    errs["dr"] = assert_close("dr", to_host(layer.dr)[:B * C], dr, BF16_TOL)
    errs["dx"] = assert_close("dx", to_host(layer.dx), dx, BF16_TOL)
    errs["dw_r"] = assert_close("dw_r", to_host(layer.dw_r), dw_r, BF16_TOL)
    for n, key in (("dW1", "dW1"), ("dW3", "dW3"), ("dW2", "dW2"), ("dWg", "dWg")):
        errs[n] = assert_close(n, to_host(getattr(layer.moe, n)), bw[key], BF16_TOL)
    got_dx = to_host(layer.dx)
    np.testing.assert_array_equal(got_dx[dropped], np.asarray(wl.dout)[dropped],
                                  err_msg="dropped tokens: dx must equal dout")
    return errs


CASES = [
    # (id, S_in = B*T, overrides): T = S_in / 4 per sequence, C = T // 2 kept
    ("mod_T128", 512, dict(H=256, Hf=384)),
    ("mod_T100_ragged", 400, dict(H=256, Hf=256)),
    ("mod_T37_odd", 148, dict(H=128, Hf=256, E=8)),
    # the longest sequence the selection accepts (T = 8192: the keys fill
    # the whole LDS key array), and T = 5000 (not a power of two; each
    # thread owns a run of five positions)
    ("mod_T8192_longest", 32768, dict(H=128, Hf=128)),
    ("mod_T5000_not_pow2", 20000, dict(H=128, Hf=128)),
]


@pytest.mark.parametrize("cid,S,ov", CASES, ids=[c[0] for c in CASES])
def test_mod_parity(cid, S, ov):
    _say(f"[mod] {cid} S_in={S} {ov}")
    wl = make_workload("c5", S=S, host_weights=True, **ov)
    errs = run_and_check(wl)
    _say(f"[mod] {cid} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_mod_all_kept():
    wl = make_workload("c5", S=256, H=128, Hf=128, E=4, host_weights=True)
    run_and_check(wl, C=wl.cfg["T"])


def test_mod_keep_one():
    # C = 1: the selection descends all eight digit passes to a single key
    wl = make_workload("c5", S=1024, H=128, Hf=128, E=4, host_weights=True)
    run_and_check(wl, C=1)


def test_mod_tied_scores():
    # scores from three values: the C-th key falls inside a tie group, so the
    # selection's digit passes descend into the position bits
    wl = make_workload("c5", S=1024, H=128, Hf=128, E=4, host_weights=True)
    rng = np.random.default_rng(7)
    x = np.array(wl.x, dtype=np.float32, copy=True)
    x[:, 0] = rng.integers(-1, 2, size=x.shape[0]).astype(np.float32)
    wl.x = x
    w = np.zeros_like(wl.w_r)
    w[0] = 1.0
    wl.w_r = w
    run_and_check(wl)


def test_mod_zero_scores_keep_first_positions():
    # every score is 0: the tie rule keeps the first C positions of each sequence
    wl = make_workload("c5", S=256, H=128, Hf=128, E=4, host_weights=True)
    run_and_check(wl, zero_scores=True)


def test_mod_raw_gates_and_recompute():
    # the MoD block over a MoE layer with raw softmax gates that keeps no h1/h3
    wl = make_workload("c5", S=512, H=256, Hf=384, host_weights=True)
    errs = run_and_check(wl, flags=L.MOE_F_RECOMPUTE)
    _say("[mod] raw gates + recompute " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
