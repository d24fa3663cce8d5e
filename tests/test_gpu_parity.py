"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Integer outputs (top-K indices, counts, cu_seqlens, the permutation) must be
bit-exact; xd must be a bitwise copy; float outputs are compared normwise
(max |gpu - oracle| / max |oracle|) with 2e-2 for bf16 storage and 1e-5 for
fp32 storage.  The top-K is checked against the oracle's selection on the
GPU's own float32 logits (the logits themselves are checked to 1e-5: both
sides accumulate the router product in at least fp32); everything downstream
is the oracle's float64 arithmetic on the exact inputs and that routing.
"""
import sys

import numpy as np
import pytest

import oracle
from synth import make_workload
from tests.moe_testutil import (BF16_TOL, F32_TOL, assert_close, oracle_on_gpu_routing, to_dev,
                                to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from routing_dispatch_grouped_moe_amd import MoELayer  # noqa: E402
from routing_dispatch_grouped_moe_amd import _lib as L  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_layer(wl, W1=None, W3=None, W2=None, bias=None, backward=True, flags=L.MOE_F_RENORM):
    """Upload a workload, run the GPU forward (+ backward); return host copies."""
    dt = wl.dtype
    x = to_dev(wl.x, dt)
    Wg = to_dev(wl.Wg, dt)
    b = None if wl.bias is None else torch.from_numpy(wl.bias.astype(np.float32)).cuda()
    W1 = to_dev(wl.W1, dt); W3 = to_dev(wl.W3, dt); W2 = to_dev(wl.W2, dt)
    dout = to_dev(wl.dout, dt)
    layer = MoELayer(wl.S, wl.H, wl.Hf, wl.E, wl.K, dt, flags=flags)
    L.moe_clear_status(layer.ws)
    layer.forward(x, Wg, b, W1, W3, W2)
    if backward:
        layer.backward(dout, x, Wg, W1, W3, W2)
    torch.cuda.synchronize()
    names = ["logits", "topk_idx", "gates", "counts", "cu", "row_of", "tok_of", "xd", "h1", "h3",
             "a", "y", "out"]
    if backward:
        names += ["dy", "dh1", "dh3", "dxd", "dgates", "dlogits", "dx", "dWg", "dW1", "dW3", "dW2"]
    got = {n: to_host(getattr(layer, n)) for n in names if getattr(layer, n) is not None}
    got["status"] = layer.status()
    return got


def check_against_oracle(wl, got, tol, backward=True, renorm=True):
    x, Wg, bias = wl.x, wl.Wg, wl.bias
    S, E, K = wl.S, wl.E, wl.K
    # router logits: fp32 accumulation on both sides
    want_logits = oracle.router_logits(x, Wg, bias)
    assert_close("logits", got["logits"], want_logits, 1e-5)
    fw, bw = oracle_on_gpu_routing(x, Wg, bias, wl.W1, wl.W3, wl.W2, K, got["logits"], wl.dout,
                                   renorm=renorm)
    np.testing.assert_array_equal(got["topk_idx"], fw["idx"], err_msg="topk_idx")
    assert_close("gates", got["gates"], fw["gates"], 1e-5)
    np.testing.assert_array_equal(got["counts"], fw["counts"], err_msg="counts")
    np.testing.assert_array_equal(got["cu"], fw["cu"], err_msg="cu_seqlens")
    np.testing.assert_array_equal(got["row_of"], fw["row_of"], err_msg="row_of")
    np.testing.assert_array_equal(got["tok_of"], fw["tok_of"], err_msg="tok_of")
    np.testing.assert_array_equal(got["xd"], np.asarray(x, np.float32)[fw["tok_of"]], err_msg="xd")
    errs = {}
    for n in ("h1", "h3", "a", "y"):
        errs[n] = assert_close(n, got[n], fw[n], tol)
    errs["out"] = assert_close("out", got["out"], fw["out"], tol)
    if backward:
        for n, key in (("dy", "dy"), ("dgates", "dg"), ("dlogits", "dlogits"), ("dh1", "dh1"),
                       ("dh3", "dh3"), ("dxd", "dxd"), ("dx", "dx"), ("dWg", "dWg"),
                       ("dW1", "dW1"), ("dW3", "dW3"), ("dW2", "dW2")):
            errs[n] = assert_close(n, got[n], bw[key], tol)
        # each expert's weight gradient against its own scale (a cold
        # expert's error must not hide under a hot expert's maximum)
        for n in ("dW1", "dW3", "dW2"):
            for e in np.nonzero(fw["counts"] > 0)[0]:
                errs[f"{n}[{e}]"] = assert_close(f"{n}[{e}]", got[n][e], bw[n][e], tol)
    # end-to-end routing: the oracle's own logits vs the GPU's choice
    own = oracle.topk_experts(want_logits, K)
    flips = int(np.sum(np.any(own != got["topk_idx"], axis=1)))
    return errs, flips


CASES = [
    # (id, config, overrides): reduced sizes span several tiles and ragged tails
    ("c1_tiny_fp32", "c1", {}),
    ("c2_mixtral_shape_small", "c2", dict(S=300, H=256, Hf=384)),
    # 525 rows per expert: three M tiles each, the last ragged; above the
    # few-rows bound of the weight-gradient products (smaller shares use the
    # small-tile form)
    ("c2_mixtral_shape_multi_tile", "c2", dict(S=2100, H=256, Hf=384)),
    # about 24 tiles, under half a wave of 256 compute units: the down and dxd
    # products split every tile along K (2 and 4 parts; H' = 2048 gives 32
    # and 64 K steps) and sum fp32 partial tiles in a second kernel
    ("c2_k_split_last_wave", "c2", dict(S=2100, H=256, Hf=2048, E=12)),
    # the same with one M tile per expert (about 167 rows each): the
    # M-grouped products walk groups of one M tile, and the split tail
    # follows that order
    ("c2_k_split_single_tiles", "c2", dict(S=1000, H=256, Hf=2048, E=12)),
    # and with most experts at one M tile but two at four (groups of two M
    # tiles, 13 tiles in all)
    ("c4_k_split_pairs", "c4", dict(S=1000, H=256, Hf=2048, E=12, K=2, beta=1.0)),
    ("c3_zipf_small", "c3", dict(S=257, H=256, Hf=256)),
    ("c4_moonep_small", "c4", dict(S=200, H=512, Hf=256, beta=1.0)),
    ("c4_moonep_skewed_small", "c4", dict(S=640, H=256, Hf=384, beta=4.0)),
    # decode shape: about one row per expert, many experts empty; the
    # M-grouped products take 64-row tiles (at most 32 rows per expert on
    # average), forward and backward
    ("c6_decode_small", "c6", dict(S=48, H=512, Hf=256)),
    # 64-row tiles with a hot expert spanning several of them (ragged tail):
    # 400 rows over 16 experts, the Zipf-biased top expert takes most tokens
    ("c4_few_rows_hot_expert", "c4", dict(S=200, H=256, Hf=384, E=16, K=2, beta=4.0)),
    # the tiled router (2048 tokens, 256 experts) inside the whole layer
    ("c4_tiled_router", "c4", dict(S=2048, H=256, Hf=256, E=256, beta=1.0)),
    # dW2's XCD dealing with 8 tiles per expert and 12 experts (not a
    # multiple of 8): the two heavy experts (more than twice the mean rows)
    # plus two more split eight ways, the other eight whole, one per XCD,
    # some of them empty; few rows (eight-wavefront tiles) and many rows
    # (one wavefront per SIMD)
    ("c4_dw2_dealing_few_rows", "c4", dict(S=1000, H=1024, Hf=512, E=12, K=2, beta=2.0)),
    ("c4_dw2_dealing_many_rows", "c4", dict(S=4096, H=1024, Hf=512, E=12, K=2, beta=2.0)),
    # the largest expert count and top-K the library accepts (1024 experts,
    # top-16; 2080 rows): spread over ~850 experts of at most ten rows each,
    # and Zipf-concentrated on ~28 experts with every token in the hottest
    # ones (several 64-row tiles each) and ~1000 experts empty
    # Zipf-skewed with at least 512 rows per expert: the one-wavefront-per-
    # SIMD weight gradients, dW1/dW3 in patches (the hottest expert holds
    # half the rows)
    ("c3_many_rows_skewed", "c3", dict(S=2100, H=256, Hf=384, E=8, K=2)),
    ("max_experts_top16_spread", "c4", dict(S=130, H=128, Hf=128, E=1024, K=16, beta=0.0)),
    ("max_experts_top16_zipf", "c3", dict(S=130, H=128, Hf=128, E=1024, K=16)),
]


@pytest.mark.parametrize("cid,cfg,ov", CASES, ids=[c[0] for c in CASES])
def test_layer_parity(cid, cfg, ov):
    _say(f"[parity] {cid} {ov}")
    wl = make_workload(cfg, **ov, host_weights=True)
    got = run_layer(wl)
    tol = F32_TOL if wl.dtype == "f32" else BF16_TOL
    errs, flips = check_against_oracle(wl, got, tol)
    _say(f"[parity] {cid} flips={flips} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert got["status"] == 0
    if wl.dtype == "f32":
        assert flips == 0


# Raw softmax gates (the chosen entries of the softmax over all E experts, no
# renormalisation): dense dlogits, and the router terms of dx and dWg over
# every expert.
RAW_CASES = [
    ("c1_tiny_fp32_raw", "c1", {}),
    ("c2_mixtral_shape_raw", "c2", dict(S=300, H=256, Hf=384)),
    ("c3_zipf_raw", "c3", dict(S=257, H=256, Hf=256)),
    ("c4_moonep_skewed_raw", "c4", dict(S=640, H=256, Hf=384, beta=4.0)),
    # K = E: the raw gates are the whole softmax (they sum to one)
    ("c2_raw_every_expert", "c2", dict(S=130, H=128, Hf=256, E=4, K=4)),
    # dense logit gradient over the largest expert count, top-16
    ("max_experts_top16_raw", "c4", dict(S=130, H=128, Hf=128, E=1024, K=16, beta=0.0)),
]


@pytest.mark.parametrize("cid,cfg,ov", RAW_CASES, ids=[c[0] for c in RAW_CASES])
def test_layer_parity_raw_gates(cid, cfg, ov):
    _say(f"[parity raw] {cid}: {cfg} {ov}")
    wl = make_workload(cfg, host_weights=True, **ov)
    got = run_layer(wl, flags=0)
    assert got["status"] == 0
    tol = F32_TOL if wl.dtype == "f32" else BF16_TOL
    errs, flips = check_against_oracle(wl, got, tol, renorm=False)
    gsum = got["gates"].sum(axis=1)
    if wl.K == wl.E:
        np.testing.assert_allclose(gsum, 1.0, atol=1e-5)
    else:
        # raw gates do not sum to one; dlogits is non-zero off the chosen experts
        assert np.all(gsum < 1.0 + 1e-6)
        assert np.count_nonzero(got["dlogits"]) > got["topk_idx"].size
    _say(f"[parity raw] {cid}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items())
         + f" flips={flips}")


# Recompute instead of save: the forward keeps no h1/h3 and the backward
# recomputes them into dh1/dh3 and runs the SwiGLU backward in place.  Same
# kernels on the same inputs, so every output must equal the saving mode's
# bit for bit (the saving mode is the one checked against the oracle above).
RECOMPUTE_CASES = [
    ("c1_fp32", "c1", {}),                                            # fp32 kernels
    ("c2_w4", "c2", dict(S=300, H=256, Hf=384)),                      # 256-row tiles
    ("c4_skewed", "c4", dict(S=640, H=256, Hf=384, beta=4.0)),        # ragged, hot expert
    ("c6_few_rows", "c6", dict(S=48, H=512, Hf=256)),                 # 64-row tiles
]


@pytest.mark.parametrize("cid,cfg,ov", RECOMPUTE_CASES, ids=[c[0] for c in RECOMPUTE_CASES])
def test_recompute_matches_saving_mode_bitwise(cid, cfg, ov):
    _say(f"[recompute] {cid}: {cfg} {ov}")
    wl = make_workload(cfg, host_weights=True, **ov)
    saved = run_layer(wl)
    rec = run_layer(wl, flags=L.MOE_F_RENORM | L.MOE_F_RECOMPUTE)
    assert rec["status"] == 0
    assert "h1" not in rec and "h3" not in rec
    for n, v in saved.items():
        if n in ("h1", "h3", "status"):
            continue
        np.testing.assert_array_equal(rec[n], v, err_msg=f"{n} differs under recompute")


@pytest.mark.parametrize("cfg,ov", [("c3", dict(S=257, H=256, Hf=256)),
                                    ("c2", dict(S=2100, H=256, Hf=2048, E=12))],
                         ids=["c3_small", "c2_k_split"])
def test_determinism_bitwise(cfg, ov):
    wl = make_workload(cfg, **ov, host_weights=True)
    a = run_layer(wl)
    b = run_layer(wl)
    for k in a:
        if k == "status":
            continue
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_uniform_logits_tie_break_and_empty_experts():
    # Wg = 0 and no bias: every logit is exactly 0, so every token picks experts 0..K-1.
    wl = make_workload("c2", S=150, H=256, Hf=256, E=8, K=3, host_weights=True)
    wl.Wg[:] = 0.0
    got = run_layer(wl)
    assert (got["topk_idx"] == np.arange(3)[None, :]).all()
    np.testing.assert_array_equal(got["counts"], [150, 150, 150, 0, 0, 0, 0, 0])
    check_against_oracle(wl, got, BF16_TOL)
    assert not np.any(got["dW1"][3:]) and not np.any(got["dW2"][3:])


def test_single_token_and_one_hot_expert():
    wl = make_workload("c2", S=1, H=128, Hf=128, E=4, K=2, host_weights=True)
    got = run_layer(wl)
    check_against_oracle(wl, got, BF16_TOL)
    # every token forced onto expert 5 first: one expert owns S rows (many M tiles)
    wl = make_workload("c3", S=700, H=128, Hf=256, host_weights=True)
    wl.bias = np.zeros(wl.E, np.float32)
    wl.bias[5] = 50.0
    got = run_layer(wl)
    assert (got["topk_idx"][:, 0] == 5).all()
    check_against_oracle(wl, got, BF16_TOL)


def test_single_expert_top1():
    wl = make_workload("c2", S=130, H=128, Hf=256, E=1, K=1, host_weights=True)
    got = run_layer(wl)
    check_against_oracle(wl, got, BF16_TOL)
    np.testing.assert_allclose(got["gates"], 1.0)


def test_nonfinite_logit_sets_status():
    wl = make_workload("c2", S=64, H=128, Hf=128, E=8, K=2, host_weights=True)
    wl.x[3, 7] = np.inf
    got = run_layer(wl, backward=False)
    assert got["status"] & L.MOE_DEV_NONFINITE_LOGIT


def test_dispatch_bad_expert_sets_status_and_skips_pair():
    wl = make_workload("c2", S=64, H=128, Hf=128, E=8, K=2, host_weights=True)
    layer = MoELayer(64, 128, 128, 8, 2, "bf16", backward=False)
    L.moe_clear_status(layer.ws)
    x = to_dev(wl.x, "bf16")
    idx = np.tile(np.array([[1, 3]], np.int32), (64, 1))
    idx[10, 1] = 8   # outside [0, E)
    layer.topk_idx.copy_(torch.from_numpy(idx))
    layer.dispatch(x)
    torch.cuda.synchronize()
    assert layer.status() & L.MOE_DEV_BAD_EXPERT
    row_of = to_host(layer.row_of)
    assert row_of[10 * 2 + 1] == -1
    cu = to_host(layer.cu)
    assert cu[-1] == 64 * 2 - 1 and cu[2] - cu[1] == 64 and cu[4] - cu[3] == 63


def test_zero_tokens():
    layer = MoELayer(0, 128, 128, 8, 2, "bf16")
    W1 = torch.zeros(8, 128, 128, dtype=torch.bfloat16, device="cuda")
    Wg = torch.zeros(128, 8, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(0, 128, dtype=torch.bfloat16, device="cuda")
    layer.dW1.fill_(1.0)
    layer.dWg.fill_(1.0)
    layer.forward(x, Wg, None, W1, W1, W1)
    layer.backward(x, x, Wg, W1, W1, W1)
    torch.cuda.synchronize()
    assert not to_host(layer.counts).any() and not to_host(layer.cu).any()
    assert not to_host(layer.dW1).any() and not to_host(layer.dWg).any()


@pytest.mark.parametrize("cid,cfg,ov,flags", [
    ("c3_zipf_small_accum", "c3", dict(S=257, H=256, Hf=256), L.MOE_F_RENORM),
    ("c2_multi_tile_accum", "c2", dict(S=2100, H=256, Hf=384, E=12), L.MOE_F_RENORM),
    ("c2_raw_gates_recompute_accum", "c2", dict(S=300, H=256, Hf=384), L.MOE_F_RECOMPUTE),
    # the fp32 kernel's accumulating epilogue (64-row weight-gradient tiles)
    ("c1_tiny_fp32_accum", "c1", {}, L.MOE_F_RENORM),
], ids=["c3_zipf_small_accum", "c2_multi_tile_accum", "c2_raw_gates_recompute_accum",
        "c1_tiny_fp32_accum"])
def test_accumulated_weight_gradients(cid, cfg, ov, flags):
    """MOE_F_ACCUM_GRAD adds the step's weight gradients to what the buffers hold.

    The buffers are prefilled with a known pattern P; afterwards dW - P must
    match the oracle's gradient to the bf16 tolerance, and an expert with no
    rows must still hold exactly P.
    """
    _say(f"[accum] {cid} {ov}")
    wl = make_workload(cfg, **ov, host_weights=True)
    # expert E-1 gets no rows: every token's bias for it is very negative
    bias = np.zeros(wl.E, np.float32) if wl.bias is None else wl.bias.copy()
    bias[wl.E - 1] = -1e4
    wl.bias = bias
    dt = wl.dtype
    x, Wg = to_dev(wl.x, dt), to_dev(wl.Wg, dt)
    W1, W3, W2, dout = to_dev(wl.W1, dt), to_dev(wl.W3, dt), to_dev(wl.W2, dt), to_dev(wl.dout, dt)
    b = torch.from_numpy(bias).cuda()
    layer = MoELayer(wl.S, wl.H, wl.Hf, wl.E, wl.K, dt, flags=flags | L.MOE_F_ACCUM_GRAD)
    pats = {}
    for n in ("dW1", "dW3", "dW2", "dWg"):
        g = getattr(layer, n)
        pat = torch.linspace(-0.5, 0.5, g.numel(), dtype=torch.float32, device="cuda").view_as(g)
        g.copy_(pat)
        pats[n] = to_host(pat)
    layer.forward(x, Wg, b, W1, W3, W2)
    layer.backward(dout, x, Wg, W1, W3, W2)
    torch.cuda.synchronize()
    assert layer.status() == 0
    counts = to_host(layer.counts)
    assert counts[wl.E - 1] == 0
    _, bw = oracle_on_gpu_routing(wl.x, wl.Wg, bias, wl.W1, wl.W3, wl.W2, wl.K,
                                  to_host(layer.logits), wl.dout,
                                  renorm=bool(flags & L.MOE_F_RENORM))
    for n in ("dW1", "dW3", "dW2", "dWg"):
        got = to_host(getattr(layer, n)).astype(np.float64) - pats[n]
        assert_close(f"{n} increment", got, bw[n], BF16_TOL)
    if dt == "f32":
        # The fp32 kernels accumulate each output in one fmaf chain and the
        # accumulating epilogue adds that chain's result to the old value
        # once, so dW must be float32(P + G) bit for bit, with G the
        # overwriting run's gradient (the same chain): the fp32 bar without
        # the cancellation of subtracting P.
        over = MoELayer(wl.S, wl.H, wl.Hf, wl.E, wl.K, dt, flags=flags)
        over.forward(x, Wg, b, W1, W3, W2)
        over.backward(dout, x, Wg, W1, W3, W2)
        torch.cuda.synchronize()
        for n in ("dW1", "dW3", "dW2", "dWg"):
            G = to_host(getattr(over, n)).astype(np.float32)
            want = pats[n].astype(np.float32) + G
            np.testing.assert_array_equal(to_host(getattr(layer, n)), want,
                                          err_msg=f"{n}: P + G in fp32, bit for bit")
            assert_close(f"{n} (overwrite)", G, bw[n], F32_TOL)
    for n in ("dW1", "dW3", "dW2"):
        np.testing.assert_array_equal(to_host(getattr(layer, n))[wl.E - 1], pats[n][wl.E - 1],
                                      err_msg=f"{n}: an expert without rows must keep its values")
