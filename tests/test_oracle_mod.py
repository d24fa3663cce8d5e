"""Pins of the oracle's Mixture-of-Depths step (CPU only)."""
import numpy as np
import pytest
import torch

import oracle


def _brute_keep(r, B, T, C):
    keep = []
    for b in range(B):
        order = sorted(range(T), key=lambda t: (-float(r[b * T + t]), t))
        keep += sorted(b * T + t for t in order[:C])
    return keep


@pytest.mark.parametrize("B,T,C", [(1, 8, 4), (3, 10, 5), (2, 7, 0), (2, 7, 7), (4, 16, 8)])
def test_keep_set_matches_comparison_sort_with_ties(B, T, C):
    rng = np.random.default_rng(B * 100 + T)
    r = rng.integers(-2, 3, size=B * T).astype(np.float32)   # many ties
    r[(r == 0) & (rng.random(B * T) < 0.5)] = -0.0
    assert oracle.mod_keep(r, B, T, C).tolist() == _brute_keep(r, B, T, C)


def _moe_layer(seed, H, Hf, E, K):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((H, E)) * 0.5, rng.standard_normal((E, H, Hf)) * 0.3,
            rng.standard_normal((E, H, Hf)) * 0.3, rng.standard_normal((E, Hf, H)) * 0.3)


def _mod_moe(x, w_r, B, T, C, Wg, W1, W3, W2, K, dout):
    r = oracle.mod_scores(x, w_r, out_dtype=np.float64)
    keep = oracle.mod_keep(r, B, T, C)
    xk = x[keep]
    fw = oracle.moe_forward(xk, Wg, None, W1, W3, W2, K=K, logits_dtype=np.float64)
    out = oracle.mod_merge(x, r, keep, fw["out"])
    dm, dr, _, _ = oracle.mod_backward(x, w_r, r, keep, fw["out"], dout, None)
    bw = oracle.moe_backward(fw, dm, xk, Wg, W1, W3, W2, K=K)
    _, _, dx, dw_r = oracle.mod_backward(x, w_r, r, keep, fw["out"], dout, bw["dx"])
    return out, dx, dw_r, bw, keep, fw


def test_all_kept_and_none_kept():
    B, T, H, Hf, E, K = 2, 6, 6, 5, 4, 2
    rng = np.random.default_rng(1)
    x = rng.standard_normal((B * T, H)); w_r = rng.standard_normal(H) * 0.5
    dout = rng.standard_normal((B * T, H))
    Wg, W1, W3, W2 = _moe_layer(2, H, Hf, E, K)
    out, dx, dw_r, _, keep, _ = _mod_moe(x, w_r, B, T, 0, Wg, W1, W3, W2, K, dout)
    assert keep.size == 0
    np.testing.assert_array_equal(out, x)
    np.testing.assert_array_equal(dx, dout)
    assert not np.any(dw_r)
    out, _, _, _, keep, _ = _mod_moe(x, w_r, B, T, T, Wg, W1, W3, W2, K, dout)
    assert keep.tolist() == list(range(B * T))
    full = oracle.moe_forward(x, Wg, None, W1, W3, W2, K=K, logits_dtype=np.float64)["out"]
    r = x @ w_r
    np.testing.assert_allclose(out, x + r[:, None] * full, rtol=1e-12, atol=1e-12)


def test_mod_moe_backward_matches_torch_autograd():
    B, T, C, H, Hf, E, K = 2, 8, 4, 6, 5, 4, 2
    rng = np.random.default_rng(3)
    x = rng.standard_normal((B * T, H)); w_r = rng.standard_normal(H) * 0.5
    dout = rng.standard_normal((B * T, H))
    Wg, W1, W3, W2 = _moe_layer(4, H, Hf, E, K)
    out, dx, dw_r, bw, keep, fw = _mod_moe(x, w_r, B, T, C, Wg, W1, W3, W2, K, dout)

    Tn = lambda a: torch.tensor(a, requires_grad=True)
    xt, wrt, Wgt, W1t, W3t, W2t = Tn(x), Tn(w_r), Tn(Wg), Tn(W1), Tn(W3), Tn(W2)
    kt = torch.tensor(keep.astype(np.int64))
    r = xt @ wrt
    xk = xt[kt]
    l = xk @ Wgt
    p = torch.softmax(l, 1)
    mask = torch.zeros_like(p).scatter_(1, torch.tensor(fw["idx"].astype(np.int64)), 1.0)
    G = p * mask
    G = G / G.sum(1, keepdim=True)
    m = torch.zeros_like(xk)
    for e in range(E):
        m = m + G[:, e:e + 1] * ((torch.nn.functional.silu(xk @ W1t[e]) * (xk @ W3t[e])) @ W2t[e])
    ref = xt.clone()
    ref = ref.index_add(0, kt, r[kt, None] * m)
    np.testing.assert_allclose(out, ref.detach().numpy(), rtol=1e-11, atol=1e-12)
    (ref * torch.tensor(dout)).sum().backward()
    tol = dict(rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dx, xt.grad.numpy(), **tol)
    np.testing.assert_allclose(dw_r, wrt.grad.numpy(), **tol)
    np.testing.assert_allclose(bw["dWg"], Wgt.grad.numpy(), **tol)
    np.testing.assert_allclose(bw["dW1"], W1t.grad.numpy(), **tol)
    np.testing.assert_allclose(bw["dW2"], W2t.grad.numpy(), **tol)
