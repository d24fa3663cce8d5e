"""Shared helpers of the test suite: uploads, error norms, oracle runs on GPU routing."""
from __future__ import annotations

import numpy as np

import oracle
from synth import bf16_bits

BF16_TOL = 2e-2   # normwise max relative error, bf16 storage
F32_TOL = 1e-5    # normwise max relative error, fp32 storage


def to_dev(a, dtype, device="cuda"):
    """Upload a float32 array holding exact values as bf16 (bit for bit) or fp32."""
    import torch
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        t = torch.from_numpy(bf16_bits(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a.copy())
    return t.to(device)


def to_host(t):
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy()


def normwise(got, want):
    """||got - want||_inf / ||want||_inf (0 when both are zero)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.abs(want).max() if want.size else 0.0
    num = np.abs(got - want).max() if want.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def assert_close(name, got, want, tol):
    err = normwise(got, want)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= tol, f"{name}: normwise error {err:.3e} > {tol:.1e}"
    return err


def oracle_on_gpu_routing(x, Wg, bias, W1, W3, W2, K, logits_gpu, dout, renorm=True):
    """Oracle forward + backward with the routing decisions taken from the GPU's logits.

    The top-K is recomputed by the oracle from the GPU's own float32 logits
    (the selection must then match bit for bit); everything downstream is the
    oracle's float64 arithmetic on the exact input values.
    """
    idx = oracle.topk_experts(logits_gpu, K)
    fw = oracle.moe_forward(x, Wg, bias, W1, W3, W2, K, renorm=renorm, idx=idx, logits=logits_gpu)
    bw = oracle.moe_backward(fw, dout, x, Wg, W1, W3, W2, K, renorm=renorm)
    return fw, bw
