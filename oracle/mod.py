"""CPU oracle of the Mixture-of-Depths step around the MoE layer (float64).

TEST INFRASTRUCTURE ONLY (see oracle/moe.py for who may call it).

Source: "PyTorch MoE/MoD Training Framework..." (ai-manual.ru), "Comparison
with alternatives" (MoD: a share of the tokens skips the layer entirely, here
50%) and "Who the framework saves" (the MoE+MoD combination).  The pages give
no formula; the reading used:
  * score r[s] = <x[s], w_r>, a raw linear score, rounded to float32;
  * per sequence keep the C tokens of largest score, ties to the lower
    position, listed in ascending position;
  * out[s] = x[s] + r[s] * m[j] for the kept token s at kept slot j (m = MoE
    output of the kept rows), out[s] = x[s] for a skipped token, so the score
    receives a gradient.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def mod_scores(x, w_r, out_dtype=np.float32):
    """r[s] = sum_h x[s,h] w_r[h] in float64, rounded to float32 (``out_dtype`` float64 keeps it)."""
    return (np.asarray(x, F64) @ np.asarray(w_r, F64)).astype(out_dtype)


def mod_keep(r, B, T, C):
    """keep_idx [B*C]: per sequence b, the C positions of largest r (ties: lower position), ascending.

    Indices are global token positions b*T + t.
    """
    r = np.asarray(r).reshape(B, T)
    keep = np.empty((B, C), dtype=np.int64)
    for b in range(B):
        rb = r[b].astype(F64)
        rb = np.where(rb == 0, 0.0, rb)
        order = np.lexsort((np.arange(T), -rb))      # score descending, position ascending
        keep[b] = np.sort(order[:C]) + b * T
    return keep.reshape(-1).astype(np.int32)


def mod_merge(x, r, keep_idx, m):
    """out = x; out[keep_idx[j]] += r[keep_idx[j]] * m[j]."""
    out = np.array(x, dtype=F64, copy=True)
    for j, s in enumerate(np.asarray(keep_idx, dtype=np.int64)):
        out[s] += float(r[s]) * np.asarray(m[j], F64)
    return out


def mod_backward(x, w_r, r, keep_idx, m, dout, dxk):
    """Gradients of the merge and the score, given dxk = d(loss)/d(x[keep]) from the MoE backward.

        dm[j]  = r[s] dout[s]            (s = keep_idx[j])
        dr[j]  = <dout[s], m[j]>         (gradient of the score of kept slot j)
        dx[s]  = dout[s] + [kept] (dxk[j] + dr[j] w_r)
        dw_r   = sum over kept slots of dr[j] x[s]
    Returns dm (the upstream gradient for the MoE layer), dr, dx, dw_r.
    ``dxk`` may be None to obtain dm and dr alone.
    """
    dout = np.asarray(dout, F64)
    keep = np.asarray(keep_idx, dtype=np.int64)
    m = np.asarray(m, F64)
    dm = np.zeros_like(m)
    dr = np.zeros(len(keep))
    for j, s in enumerate(keep):
        dm[j] = float(r[s]) * dout[s]
        dr[j] = dout[s] @ m[j]
    if dxk is None:
        return dm, dr, None, None
    dx = np.array(dout, copy=True)
    wr = np.asarray(w_r, F64)
    dxk = np.asarray(dxk, F64)
    dw_r = np.zeros(x.shape[1])
    for j, s in enumerate(keep):
        dx[s] += dxk[j] + dr[j] * wr
        dw_r += dr[j] * np.asarray(x[s], F64)
    return dm, dr, dx, dw_r
