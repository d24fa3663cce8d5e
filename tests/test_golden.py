"""Hand-worked examples under tests/golden/ against the oracle (CPU) and the HIP path (GPU).

Each fixture states, next to its numbers, how they were derived by hand from
the definitions and which passage of the pages each definition comes from.
The CPU tests pin the oracle to those numbers; the GPU tests run the same
examples through the C ABI (fp32 storage, the inputs padded to H = 128 with
zeros, so every GPU result is exact or within fp32 rounding).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_fixture(name):
    """key: json-value lines; '#' lines are comments."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = json.loads(v)
    return out


# ------------------------------------------------------------------ CPU --

def test_golden_routing_oracle():
    g = load_fixture("routing_tiny.txt")
    E, K = g["E"], g["K"]
    logits = np.array(g["logits"], np.float32)
    idx = oracle.topk_experts(logits, K)
    assert idx.tolist() == g["topk_idx"]
    np.testing.assert_allclose(oracle.gate_weights(logits, idx), g["gates"], rtol=1e-6, atol=0)
    counts, cu = oracle.expert_counts(idx, E)
    assert counts.tolist() == g["counts"] and cu.tolist() == g["cu_seqlens"]
    row_of, tok_of = oracle.dispatch_permutation(idx, E)
    assert row_of.tolist() == g["row_of"] and tok_of.tolist() == g["tok_of"]
    assert oracle.maxvio(counts) == pytest.approx(g["maxvio"], abs=1e-12)
    gates = np.array(g["gates"])
    y = np.array(g["y"])
    np.testing.assert_allclose(oracle.combine(y, row_of, gates), g["out"], rtol=0, atol=1e-12)
    dy, dg = oracle.combine_backward(np.array(g["dout"]), y, row_of, gates)
    np.testing.assert_allclose(dg, g["dgates"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dy[:, 0], g["dy_first_column"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.gate_backward(dg, logits, idx), g["dlogits"], rtol=0, atol=2e-7)


def test_golden_swiglu_oracle():
    g = load_fixture("swiglu_tiny.txt")
    x = np.array(g["x"], np.float32)
    W = [np.array(g[k], np.float32)[None] for k in ("W1", "W3", "W2")]
    h1, h3, a, y = oracle.expert_ffn(x, np.array([0, 1]), *W)
    for name, got in (("h1", h1), ("h3", h3), ("a", a), ("y", y)):
        np.testing.assert_allclose(got, g[name], rtol=1e-6, atol=1e-12, err_msg=name)


def test_golden_mod_oracle():
    g = load_fixture("mod_keep_tiny.txt")
    r = np.array(g["r"], np.float32)
    keep = oracle.mod_keep(r, g["B"], g["T"], g["C"])
    assert keep.tolist() == g["keep_idx"]
    out = oracle.mod_merge(np.array(g["x"]), r, keep, np.array(g["m"]))
    np.testing.assert_array_equal(out, g["out"])


# ------------------------------------------------------------------ GPU --

def _pad(a, width=128):
    a = np.asarray(a, np.float32)
    out = np.zeros((a.shape[0], width), np.float32)
    out[:, :a.shape[1]] = a
    return out


@pytest.mark.gpu
def test_golden_routing_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from routing_dispatch_grouped_moe_amd import _lib as L
    g = load_fixture("routing_tiny.txt")
    S, E, K, H = g["S"], g["E"], g["K"], 128
    print(f"golden routing: S={S} E={E} K={K} H={H} fp32", flush=True)
    dev = "cuda"
    d = L.dims(S, H, H, E, K, "f32")
    # x[s] carries the logits in its first E entries and Wg is the identity on
    # them, so the router's logits are exactly the fixture's
    x = torch.from_numpy(_pad(g["logits"])).to(dev)
    Wg = torch.zeros(H, E, dtype=torch.float32)
    Wg[:E, :E] = torch.eye(E)
    Wg = Wg.to(dev)
    ws = torch.zeros(L.moe_workspace_bytes(d), dtype=torch.uint8, device=dev)
    logits = torch.empty(S, E, dtype=torch.float32, device=dev)
    idx = torch.empty(S, K, dtype=torch.int32, device=dev)
    gates = torch.empty(S, K, dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    cu = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_of = torch.empty(S * K, dtype=torch.int32, device=dev)
    tok_of = torch.empty(S * K, dtype=torch.int32, device=dev)
    xd = torch.empty(S * K, H, dtype=torch.float32, device=dev)
    out = torch.empty(S, H, dtype=torch.float32, device=dev)
    L.moe_clear_status(ws)
    L.moe_route(d, x, Wg, None, logits, idx, gates, counts, ws)
    L.moe_dispatch(d, x, idx, cu, row_of, tok_of, xd, ws)
    y = torch.from_numpy(_pad(g["y"])).to(dev)
    L.moe_combine(d, y, row_of, gates, out)
    torch.cuda.synchronize()
    assert L.moe_read_status(ws) == 0
    assert idx.cpu().tolist() == g["topk_idx"]
    np.testing.assert_allclose(gates.cpu().numpy(), g["gates"], rtol=1e-6, atol=0)
    assert counts.cpu().tolist() == g["counts"]
    assert cu.cpu().tolist() == g["cu_seqlens"]
    assert row_of.cpu().tolist() == g["row_of"]
    assert tok_of.cpu().tolist() == g["tok_of"]
    np.testing.assert_array_equal(xd.cpu().numpy(), x.cpu().numpy()[g["tok_of"]])
    o = out.cpu().numpy()
    np.testing.assert_allclose(o[:, :2], g["out"], rtol=1e-6, atol=0)
    assert not o[:, 2:].any()


@pytest.mark.gpu
def test_golden_swiglu_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from routing_dispatch_grouped_moe_amd import _lib as L
    g = load_fixture("swiglu_tiny.txt")
    H = Hf = 128
    print(f"golden swiglu: one row, one expert, H=Hf={H} fp32", flush=True)
    dev = "cuda"
    d = L.dims(1, H, Hf, 1, 1, "f32")

    def mat(a):
        m = np.zeros((1, H, Hf), np.float32)
        a = np.asarray(a, np.float32)
        m[0, :a.shape[0], :a.shape[1]] = a
        return torch.from_numpy(m).to(dev)

    xd = torch.from_numpy(_pad(g["x"])).to(dev)
    W1, W3, W2 = mat(g["W1"]), mat(g["W3"]), mat(g["W2"])
    cu = torch.tensor([0, 1], dtype=torch.int32, device=dev)
    ws = torch.zeros(L.moe_workspace_bytes(d), dtype=torch.uint8, device=dev)
    h1, h3, a = (torch.empty(1, Hf, dtype=torch.float32, device=dev) for _ in range(3))
    y = torch.empty(1, H, dtype=torch.float32, device=dev)
    L.moe_grouped_ffn(d, xd, cu, W1, W3, W2, h1, h3, a, y, ws)
    torch.cuda.synchronize()
    for name, t in (("h1", h1), ("h3", h3), ("a", a), ("y", y)):
        v = t.cpu().numpy()
        np.testing.assert_allclose(v[:, :2], g[name], rtol=1e-6, atol=1e-12, err_msg=name)
        assert not v[:, 2:].any(), name


@pytest.mark.gpu
def test_golden_mod_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from routing_dispatch_grouped_moe_amd import _lib as L
    g = load_fixture("mod_keep_tiny.txt")
    B, T, Cn, H = g["B"], g["T"], g["C"], 128
    print(f"golden MoD: B={B} T={T} C={Cn} H={H} fp32", flush=True)
    dev = "cuda"
    # scores r = x_sel . w_r with w_r the first unit vector
    xs = torch.from_numpy(_pad(np.array(g["r"], np.float32)[:, None])).to(dev)
    w_r = torch.zeros(H, dtype=torch.float32, device=dev)
    w_r[0] = 1.0
    r = torch.empty(B * T, dtype=torch.float32, device=dev)
    keep = torch.empty(B * Cn, dtype=torch.int32, device=dev)
    xk = torch.empty(B * Cn, H, dtype=torch.float32, device=dev)
    L.moe_mod_select(B, T, Cn, H, L.MOE_F32, xs, w_r, r, keep, xk)
    x = torch.from_numpy(_pad(g["x"])).to(dev)
    m = torch.from_numpy(_pad(g["m"])).to(dev)
    out = torch.empty(B * T, H, dtype=torch.float32, device=dev)
    r_fix = torch.tensor(g["r"], dtype=torch.float32, device=dev)
    keep_fix = torch.tensor(g["keep_idx"], dtype=torch.int32, device=dev)
    L.moe_mod_merge(B, T, Cn, H, L.MOE_F32, x, r_fix, keep_fix, m, out)
    torch.cuda.synchronize()
    assert keep.cpu().tolist() == g["keep_idx"]
    np.testing.assert_array_equal(xk.cpu().numpy(), xs.cpu().numpy()[g["keep_idx"]])
    o = out.cpu().numpy()
    np.testing.assert_array_equal(o[:, :2], g["out"])
    assert not o[:, 2:].any()
