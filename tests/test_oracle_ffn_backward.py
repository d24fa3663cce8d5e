"""Pins of the oracle's expert FFN, combine and backward (CPU only).

The oracle groups rows per expert; these checks compare it with formulations
it does not share: a dense SwiGLU MLP (E=1, K=1) from torch, the dense
"every expert on every token, masked by the gates" form, identity experts,
torch float64 autograd of that dense form, and float64 central finite
differences of the oracle's own forward.
"""
import numpy as np
import pytest
import torch

import oracle


def _case(seed, S, H, Hf, E, K, xs=1.0, ws=0.3, bias=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((S, H)) * xs
    Wg = rng.standard_normal((H, E)) * ws
    W1 = rng.standard_normal((E, H, Hf)) * ws
    W3 = rng.standard_normal((E, H, Hf)) * ws
    W2 = rng.standard_normal((E, Hf, H)) * ws
    b = rng.standard_normal(E) if bias else None
    dout = rng.standard_normal((S, H))
    return x, Wg, b, W1, W3, W2, dout


def _torch_dense(x, Wg, b, W1, W3, W2, idx, renorm):
    """Dense masked MoE in torch float64: every expert on every token, weighted by G[s,e]."""
    l = x @ Wg
    if b is not None:
        l = l + b
    p = torch.softmax(l, dim=1)
    mask = torch.zeros_like(p)
    mask.scatter_(1, idx, 1.0)
    G = p * mask
    if renorm:
        G = G / G.sum(1, keepdim=True)
    out = torch.zeros_like(x)
    for e in range(Wg.shape[1]):
        f = (torch.nn.functional.silu(x @ W1[e]) * (x @ W3[e])) @ W2[e]
        out = out + G[:, e:e + 1] * f
    return out, l


def test_single_expert_is_dense_swiglu_mlp():
    x, Wg, b, W1, W3, W2, _ = _case(0, 9, 16, 24, 1, 1)
    fw = oracle.moe_forward(x, Wg, b, W1, W3, W2, K=1)
    xt = torch.tensor(x)
    ref = (torch.nn.functional.silu(xt @ torch.tensor(W1[0])) * (xt @ torch.tensor(W3[0]))) @ torch.tensor(W2[0])
    np.testing.assert_allclose(fw["out"], ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fw["gates"], 1.0)


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("S,H,Hf,E,K", [(17, 8, 12, 5, 2), (33, 16, 8, 8, 3), (5, 4, 4, 3, 3)])
def test_grouped_equals_dense_masked(S, H, Hf, E, K, renorm):
    x, Wg, b, W1, W3, W2, _ = _case(S + E, S, H, Hf, E, K, bias=True)
    fw = oracle.moe_forward(x, Wg, b, W1, W3, W2, K=K, renorm=renorm, logits_dtype=np.float64)
    T = lambda a: torch.tensor(a)
    ref, _ = _torch_dense(T(x), T(Wg), T(b), T(W1), T(W3), T(W2),
                          torch.tensor(fw["idx"].astype(np.int64)), renorm)
    np.testing.assert_allclose(fw["out"], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_identity_experts_return_gate_weighted_input():
    x, Wg, b, W1, W3, W2, _ = _case(3, 40, 8, 8, 6, 3)
    logits = oracle.router_logits(x, Wg, b)
    idx = oracle.topk_experts(logits, 3)
    g = oracle.gate_weights(logits, idx, renorm=True)
    _, cu = oracle.expert_counts(idx, 6)
    row_of, tok_of = oracle.dispatch_permutation(idx, 6)
    xd = oracle.dispatch_rows(x, tok_of)
    out = oracle.combine(xd, row_of, g)           # y := xd (identity experts)
    np.testing.assert_allclose(out, x, rtol=1e-13, atol=1e-14)
    graw = oracle.gate_weights(logits, idx, renorm=False)
    out = oracle.combine(xd, row_of, graw)
    np.testing.assert_allclose(out, x * graw.sum(1, keepdims=True), rtol=1e-13, atol=1e-14)
    # zero experts give zero output
    z = oracle.combine(np.zeros_like(xd), row_of, g)
    assert not np.any(z)


def test_expert_slices_are_independent_under_expert_relabelling():
    S, H, Hf, E, K = 30, 8, 8, 5, 2
    x, Wg, b, W1, W3, W2, _ = _case(11, S, H, Hf, E, K)
    fw = oracle.moe_forward(x, Wg, b, W1, W3, W2, K=K)
    perm = np.array([3, 0, 4, 1, 2])              # new label of old expert e is perm[e]
    inv = np.argsort(perm)
    fw2 = oracle.moe_forward(x, Wg[:, inv], None if b is None else b[inv], W1[inv], W3[inv], W2[inv], K=K)
    np.testing.assert_array_equal(perm[fw["idx"]], fw2["idx"])
    np.testing.assert_allclose(fw["out"], fw2["out"], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("renorm", [True, False])
def test_backward_matches_torch_autograd_of_dense_form(renorm):
    S, H, Hf, E, K = 21, 12, 10, 6, 2
    x, Wg, b, W1, W3, W2, dout = _case(5, S, H, Hf, E, K, bias=True)
    fw = oracle.moe_forward(x, Wg, b, W1, W3, W2, K=K, renorm=renorm, logits_dtype=np.float64)
    bw = oracle.moe_backward(fw, dout, x, Wg, W1, W3, W2, K=K, renorm=renorm)
    T = lambda a: torch.tensor(a, requires_grad=True)
    xt, Wgt, W1t, W3t, W2t = T(x), T(Wg), T(W1), T(W3), T(W2)
    out, l = _torch_dense(xt, Wgt, torch.tensor(b), W1t, W3t, W2t,
                          torch.tensor(fw["idx"].astype(np.int64)), renorm)
    l.retain_grad()
    (out * torch.tensor(dout)).sum().backward()
    tol = dict(rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bw["dx"], xt.grad.numpy(), **tol)
    np.testing.assert_allclose(bw["dWg"], Wgt.grad.numpy(), **tol)
    np.testing.assert_allclose(bw["dlogits"], l.grad.numpy(), **tol)
    np.testing.assert_allclose(bw["dW1"], W1t.grad.numpy(), **tol)
    np.testing.assert_allclose(bw["dW3"], W3t.grad.numpy(), **tol)
    np.testing.assert_allclose(bw["dW2"], W2t.grad.numpy(), **tol)


def test_backward_matches_central_finite_differences():
    S, H, Hf, E, K = 12, 6, 5, 4, 2
    x, Wg, b, W1, W3, W2, dout = _case(7, S, H, Hf, E, K, xs=1.0, ws=0.5)
    args = dict(x=x, Wg=Wg, W1=W1, W3=W3, W2=W2)

    def loss(a):
        fw = oracle.moe_forward(a["x"], a["Wg"], b, a["W1"], a["W3"], a["W2"], K=K,
                                logits_dtype=np.float64)
        return float((fw["out"] * dout).sum()), fw["idx"]

    fw = oracle.moe_forward(x, Wg, b, W1, W3, W2, K=K, logits_dtype=np.float64)
    bw = oracle.moe_backward(fw, dout, x, Wg, W1, W3, W2, K=K)
    grads = dict(x=bw["dx"], Wg=bw["dWg"], W1=bw["dW1"], W3=bw["dW3"], W2=bw["dW2"])
    rng = np.random.default_rng(0)
    checked = 0
    for name, arr in args.items():
        for _ in range(12):
            i = tuple(int(rng.integers(0, n)) for n in arr.shape)
            h = 1e-5
            a_p = {k: v.copy() for k, v in args.items()}; a_p[name][i] += h
            a_m = {k: v.copy() for k, v in args.items()}; a_m[name][i] -= h
            lp, ip = loss(a_p)
            lm, im = loss(a_m)
            if not (np.array_equal(ip, fw["idx"]) and np.array_equal(im, fw["idx"])):
                continue   # the perturbation changed the routing: no derivative there
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grads[name][i]) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, grads[name][i])
            checked += 1
    assert checked >= 40
    # a random directional derivative through all tensors at once
    dirs = {k: rng.standard_normal(v.shape) for k, v in args.items()}
    h = 1e-6
    lp, _ = loss({k: args[k] + h * dirs[k] for k in args})
    lm, _ = loss({k: args[k] - h * dirs[k] for k in args})
    want = sum(float((grads[k] * dirs[k]).sum()) for k in args)
    assert abs((lp - lm) / (2 * h) - want) <= 1e-6 * max(1.0, abs(want))


def test_backward_invariants():
    S, H, Hf, E, K = 40, 8, 8, 10, 3
    x, Wg, b, W1, W3, W2, dout = _case(9, S, H, Hf, E, K)
    # make expert 7 never chosen
    Wg[:, 7] = 0.0
    b = np.zeros(E); b[7] = -1e3
    fw = oracle.moe_forward(x, Wg, b, W1, W3, W2, K=K)
    assert fw["counts"][7] == 0
    bw = oracle.moe_backward(fw, dout, x, Wg, W1, W3, W2, K=K)
    assert not np.any(bw["dW1"][7]) and not np.any(bw["dW3"][7]) and not np.any(bw["dW2"][7])
    # renormalised gates: dlogits sums to zero per token and vanishes off the chosen experts
    np.testing.assert_allclose(bw["dlogits"].sum(1), 0.0, atol=1e-12)
    off = np.ones((S, E), bool)
    np.put_along_axis(off, fw["idx"].astype(np.int64), False, 1)
    assert not np.any(bw["dlogits"][off])
    # dg = <dout, y[row]>
    for s in range(S):
        for k in range(K):
            r = fw["row_of"][s * K + k]
            assert bw["dg"][s, k] == pytest.approx(float(dout[s] @ fw["y"][r]), rel=1e-12)
    # linear in dout
    bw2 = oracle.moe_backward(fw, 2.5 * dout, x, Wg, W1, W3, W2, K=K)
    for key in ("dx", "dWg", "dW1", "dW3", "dW2"):
        np.testing.assert_allclose(bw2[key], 2.5 * bw[key], rtol=1e-12, atol=1e-14)
