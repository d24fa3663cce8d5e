"""GPU parity of the router alone over expert counts that reach every tiling
of the router GEMM (waves along K for fewer than 64 experts, one or two K32
sub-slices per stage, 1 to 16 sixteen-expert column blocks per wavefront).

Through the C ABI against the oracle: logits to 1e-5 normwise (both sides
accumulate exact bf16 products in at least fp32), the top-K bit for bit
against the oracle's selection on the GPU's own fp32 logits (the integer
decision taken in the same precision), gates to 1e-5 and per-expert counts
bit for bit.  S = 100 leaves a ragged last block of 4 tokens.  A second test
runs token counts on both sides of the H-split rule (split up to 1024 tokens);
a third runs the tiled router (bf16, at least 256 experts, a multiple of 8: a
tiled GEMM into fp32 logits, H cut into parts when the tiles are few, then the
top-K launch); a fourth checks the load statistics of routing histograms
(maxvio, load entropy).  From 256 experts up the first two tests take expert
counts that are not multiples of 8, which stay on the fused router.
"""
import sys

import numpy as np
import pytest

import oracle
from synth import make_workload
from tests.moe_testutil import F32_TOL, assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from routing_dispatch_grouped_moe_amd import _lib as L  # noqa: E402

# (E, K): one expert count per fused-router tiling (E padded to 16: 380 -> 384,
# 444 -> 448, 636 -> 640, 1002 -> 1008)
SHAPES = [(8, 2), (24, 4), (40, 6), (64, 8), (100, 8), (160, 8), (224, 8), (380, 8), (444, 16),
          (636, 8), (1002, 16)]


@pytest.mark.parametrize("E,K", SHAPES, ids=[f"E{e}_K{k}" for e, k in SHAPES])
def test_route_shapes(E, K):
    print(f"[route] E={E} K={K}", flush=True)
    sys.stdout.flush()
    wl = make_workload("c3", S=100, H=256, Hf=128, E=E, K=K, host_weights=False)
    S, H = wl.S, wl.H
    d = L.dims(S, H, wl.Hf, E, K, "bf16")
    ws = torch.zeros(L.moe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    x, Wg = to_dev(wl.x, "bf16"), to_dev(wl.Wg, "bf16")
    bias = torch.from_numpy(wl.bias.astype(np.float32)).cuda()
    logits = torch.empty(S, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(S, K, dtype=torch.int32, device="cuda")
    gates = torch.empty(S, K, dtype=torch.float32, device="cuda")
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    L.moe_clear_status(ws)
    L.moe_route(d, x, Wg, bias, logits, idx, gates, counts, ws)
    torch.cuda.synchronize()
    assert L.moe_read_status(ws) == 0

    got_l = to_host(logits)
    assert_close("logits", got_l, oracle.router_logits(wl.x, wl.Wg, wl.bias), F32_TOL)
    want_idx = oracle.topk_experts(got_l, K)
    np.testing.assert_array_equal(to_host(idx), want_idx, err_msg="topk_idx")
    assert_close("gates", to_host(gates), oracle.gate_weights(got_l, want_idx), F32_TOL)
    want_counts, _ = oracle.expert_counts(want_idx, E)
    np.testing.assert_array_equal(to_host(counts), want_counts, err_msg="counts")


# (S, H, E, K): token counts around the router's H-split rule (up to 1024
# tokens, i.e. 32 token groups, split the H reduction over 2 to 16 blocks per
# group; more tokens do not split), at hidden sizes that allow every part count
SPLITS = [(64, 4096, 380, 8), (500, 2048, 380, 8), (1000, 2048, 64, 4), (1024, 1024, 160, 8),
          (1056, 1024, 160, 8)]


@pytest.mark.parametrize("S,H,E,K", SPLITS, ids=[f"S{s}_H{h}_E{e}" for s, h, e, _ in SPLITS])
def test_route_split_boundary(S, H, E, K):
    print(f"[route split] S={S} H={H} E={E} K={K}", flush=True)
    sys.stdout.flush()
    wl = make_workload("c3", S=S, H=H, Hf=128, E=E, K=K, host_weights=False)
    d = L.dims(S, H, wl.Hf, E, K, "bf16")
    ws = torch.zeros(L.moe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    x, Wg = to_dev(wl.x, "bf16"), to_dev(wl.Wg, "bf16")
    bias = torch.from_numpy(wl.bias.astype(np.float32)).cuda()
    logits = torch.empty(S, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(S, K, dtype=torch.int32, device="cuda")
    gates = torch.empty(S, K, dtype=torch.float32, device="cuda")
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    L.moe_clear_status(ws)
    # twice: the per-group tickets must start from zero on every call
    for _ in range(2):
        L.moe_route(d, x, Wg, bias, logits, idx, gates, counts, ws)
    torch.cuda.synchronize()
    assert L.moe_read_status(ws) == 0
    got_l = to_host(logits)
    assert_close("logits", got_l, oracle.router_logits(wl.x, wl.Wg, wl.bias), F32_TOL)
    want_idx = oracle.topk_experts(got_l, K)
    np.testing.assert_array_equal(to_host(idx), want_idx, err_msg="topk_idx")
    assert_close("gates", to_host(gates), oracle.gate_weights(got_l, want_idx), F32_TOL)
    want_counts, _ = oracle.expert_counts(want_idx, E)
    np.testing.assert_array_equal(to_host(counts), want_counts, err_msg="counts")


# (S, H, E, K): the tiled router (at least 256 experts, E a multiple of 8): one
# or several 128-expert tiles, a partial last tile, ragged token tiles, and
# (32768 tokens) three blocks per compute unit; with few tokens the H extent
# is cut into parts: 16 parts of 4 K steps (64 x 4096 x 384), 16 parts of 7
# (decode, 128 x 7168 x 384), 4 parts (300 x 1024 x 1000) and 4 unequal parts
# of 4, 5, 4 and 5 K steps (100 x 1152 x 256)
TILED = [(2048, 256, 256, 8), (2100, 512, 384, 8), (4000, 128, 1000, 16), (8192, 256, 384, 8),
         (2049, 1024, 640, 4), (32768, 128, 384, 8), (64, 4096, 384, 8), (128, 7168, 384, 8),
         (300, 1024, 1000, 8), (100, 1152, 256, 4)]


@pytest.mark.parametrize("S,H,E,K", TILED, ids=[f"S{s}_H{h}_E{e}_K{k}" for s, h, e, k in TILED])
def test_route_tiled(S, H, E, K):
    print(f"[route tiled] S={S} H={H} E={E} K={K}", flush=True)
    sys.stdout.flush()
    wl = make_workload("c3", S=S, H=H, Hf=128, E=E, K=K, host_weights=False)
    d = L.dims(S, H, wl.Hf, E, K, "bf16")
    ws = torch.zeros(L.moe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    x, Wg = to_dev(wl.x, "bf16"), to_dev(wl.Wg, "bf16")
    bias = torch.from_numpy(wl.bias.astype(np.float32)).cuda()
    logits = torch.empty(S, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(S, K, dtype=torch.int32, device="cuda")
    gates = torch.empty(S, K, dtype=torch.float32, device="cuda")
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    L.moe_clear_status(ws)
    L.moe_route(d, x, Wg, bias, logits, idx, gates, counts, ws)
    # and once more with no logits buffer of the caller's (the workspace holds them)
    idx2 = torch.empty_like(idx)
    gates2 = torch.empty_like(gates)
    counts2 = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    L.moe_route(d, x, Wg, bias, None, idx2, gates2, counts2, ws)
    torch.cuda.synchronize()
    assert L.moe_read_status(ws) == 0
    got_l = to_host(logits)
    assert_close("logits", got_l, oracle.router_logits(wl.x, wl.Wg, wl.bias), F32_TOL)
    want_idx = oracle.topk_experts(got_l, K)
    np.testing.assert_array_equal(to_host(idx), want_idx, err_msg="topk_idx")
    assert_close("gates", to_host(gates), oracle.gate_weights(got_l, want_idx), F32_TOL)
    want_counts, _ = oracle.expert_counts(want_idx, E)
    np.testing.assert_array_equal(to_host(counts), want_counts, err_msg="counts")
    assert torch.equal(idx, idx2) and torch.equal(gates, gates2) and torch.equal(counts, counts2)


def test_route_tiled_parts_no_bias():
    """The H split with no bias: the part sum adds none (128 tokens x 384
    experts x H 2048: 8 parts)."""
    S, H, E, K = 128, 2048, 384, 8
    print(f"[route tiled, no bias] S={S} H={H} E={E} K={K}", flush=True)
    sys.stdout.flush()
    wl = make_workload("c3", S=S, H=H, Hf=128, E=E, K=K, host_weights=False)
    d = L.dims(S, H, wl.Hf, E, K, "bf16")
    ws = torch.zeros(L.moe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    x, Wg = to_dev(wl.x, "bf16"), to_dev(wl.Wg, "bf16")
    logits = torch.empty(S, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(S, K, dtype=torch.int32, device="cuda")
    gates = torch.empty(S, K, dtype=torch.float32, device="cuda")
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    L.moe_clear_status(ws)
    L.moe_route(d, x, Wg, None, logits, idx, gates, counts, ws)
    torch.cuda.synchronize()
    assert L.moe_read_status(ws) == 0
    got_l = to_host(logits)
    assert_close("logits", got_l, oracle.router_logits(wl.x, wl.Wg, None), F32_TOL)
    want_idx = oracle.topk_experts(got_l, K)
    np.testing.assert_array_equal(to_host(idx), want_idx, err_msg="topk_idx")
    assert_close("gates", to_host(gates), oracle.gate_weights(got_l, want_idx), F32_TOL)
    want_counts, _ = oracle.expert_counts(want_idx, E)
    np.testing.assert_array_equal(to_host(counts), want_counts, err_msg="counts")


def test_load_stats():
    """maxvio and load entropy of routing histograms through the C ABI against the oracle."""
    rng = np.random.default_rng(5)
    cases = {
        "balanced": np.full(384, 171, np.int32),
        "one_hot": np.eye(1, 64, 17, dtype=np.int32)[0] * 8192,
        "zipf": np.floor(8192 * 4 / np.arange(1, 65) ** 1.1 / np.sum(1 / np.arange(1, 65) ** 1.1))
        .astype(np.int32),
        "random": rng.integers(0, 1000, size=1000).astype(np.int32),
        "single_expert": np.array([5], np.int32),
        "all_zero": np.zeros(16, np.int32),
    }
    for name, c in cases.items():
        print(f"[load stats] {name} E={c.size}", flush=True)
        ct = torch.from_numpy(c).cuda()
        st = torch.full((2,), -1.0, dtype=torch.float32, device="cuda")
        L.moe_load_stats(c.size, ct, st)
        torch.cuda.synchronize()
        got = st.cpu().numpy()
        if c.sum() == 0:
            assert got.tolist() == [0.0, 0.0]
            continue
        np.testing.assert_allclose(got[0], oracle.maxvio(c), rtol=1e-5, atol=1e-6, err_msg=name)
        np.testing.assert_allclose(got[1], oracle.load_entropy(c), rtol=1e-5, atol=1e-6,
                                   err_msg=name)
