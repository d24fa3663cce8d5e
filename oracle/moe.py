"""CPU oracle of the MoE layer hot path: plain, slow, obviously correct (float64).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the bench's CPU-baseline leg may import or run this module.  The HIP library
never calls it, and it imports nothing from the HIP library.

Sources (the three pages this method is described on):
  [FW]   "PyTorch MoE/MoD Training Framework: custom CUDA kernels, DeepSpeed
         and a 7x speed-up on T4" (ai-manual.ru).
  [MEP]  "Moonshot AI opened MoonEP: training Mixture of Experts without GPU
         idling" (dzen.guru).
  [T4]   "MoE on T4: how to find and remove the bottlenecks" (ai-manual.ru).

What the layer computes, end to end:
    out[s] = sum_k g[s,k] * FFN_{idx[s,k]}(x[s]),
    FFN_e(v) = (silu(v W1[e]) * (v W3[e])) W2[e]
Routing is a softmax over experts plus a top-K pick ([FW] "What's in the box",
routing/gating item); tokens are moved to contiguous per-expert rows and back
([FW] same section, dispatch/combine item; [MEP] step-by-step guide, dispatch
step and its cu_seqlens offsets); each expert is a three-matrix SwiGLU FFN
([T4] "RMSNorm, RoPE, SwiGLU" table, SwiGLU row; the Mixtral block named in
[FW] "How it looks in practice"); the backward of gating and dispatch is taken
together ([FW] "What's in the box", sparse-backward item) and the weight
gradients go to an fp32 buffer shaped like the weights ([MEP] guide, gradient
buffer step).

Readings where the pages are silent:
  * gates are renormalised over the K chosen experts (drop-in for the Mixtral
    block) unless ``renorm=False``;
  * the top-K order key is (logit descending, expert index ascending) on the
    float32 logits, -0.0 equal to +0.0, NaN ranked last;
  * rows of one expert are in ascending token order (a stable counting sort);
  * cu_seqlens has E+1 entries, cu[0] = 0, cu[E] = S*K;
  * no capacity limit, no token dropping, no biases in the experts;
  * W1, W3 are [E, H, Hf] and W2 is [E, Hf, H], row-major;
  * a constant router bias is added to the logits before selection and gates
    and receives no gradient;
  * Mixture-of-Depths: out = x + r * MoE(x) on the kept tokens, x elsewhere.

All arithmetic is float64 on inputs widened exactly from float32/bf16.  The
router logits are rounded to float32 once (the precision the selection is
taken in on both sides).  Parity status of every function is pinned by the
not-gpu tests in tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(a):
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------- routing --

def router_logits(x, Wg, bias=None, out_dtype=np.float32):
    """logits[s,e] = sum_h x[s,h] Wg[h,e] + bias[e], accumulated in float64, rounded to float32.

    [FW] "What's in the box", routing/gating item (the router scores every
    expert for every token); the bias term is the workloads' per-expert skew.
    ``out_dtype=np.float64`` skips the final rounding (finite-difference checks).
    """
    l = _f64(x) @ _f64(Wg)
    if bias is not None:
        l = l + _f64(bias)[None, :]
    return l.astype(out_dtype)


def topk_experts(logits, K):
    """idx[s, 0..K-1]: the K experts of largest logit, best first, ties to the lower index.

    [FW] "What's in the box", routing/gating item, and "Comparison with
    alternatives" (a top-k selection per token).  Selection compares the logits
    as given (float32 on the hot path); +0.0 and -0.0 compare equal; a NaN
    logit ranks below every number.
    """
    l = np.array(logits, copy=True)
    S, E = l.shape
    l[l == 0] = 0.0                        # -0.0 -> +0.0
    nan = np.isnan(l)
    neg = -l.astype(F64)
    neg[nan] = 0.0
    e_idx = np.broadcast_to(np.arange(E), (S, E))
    idx = np.empty((S, K), dtype=np.int32)
    for s in range(S):
        # primary key: NaN last; then logit descending; then expert ascending
        order = np.lexsort((e_idx[s], neg[s], nan[s]))
        idx[s] = order[:K]
    return idx


def softmax_probs(logits):
    """p[s,e] = exp(l[s,e] - max_e l) / sum_j exp(l[s,j] - max_e l), float64."""
    l = _f64(logits)
    m = l.max(axis=1, keepdims=True)
    z = np.exp(l - m)
    return z / z.sum(axis=1, keepdims=True)


def gate_weights(logits, idx, renorm=True):
    """g[s,k] = p[s, idx[s,k]] (raw) or that value divided by sum_j p[s, idx[s,j]] (renorm).

    [FW] "What's in the box", routing/gating item (softmax over the experts),
    and "How it looks in practice" (a drop-in for the Mixtral block, which
    renormalises the chosen probabilities).
    """
    p = softmax_probs(logits)
    g = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renorm:
        g = g / g.sum(axis=1, keepdims=True)
    return g


# --------------------------------------------------------------- dispatch --

def expert_counts(idx, E):
    """counts[e] = number of (token, k) pairs sent to expert e; cu[0]=0, cu[e+1]=cu[e]+counts[e].

    [MEP] guide, dispatch step (cu_seqlens marks each expert's active rows) and
    the contract step (every (token, k) pair gets a row, S*K in total).
    """
    counts = np.zeros(E, dtype=np.int64)
    for e in idx.reshape(-1):
        counts[int(e)] += 1
    cu = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        cu[e + 1] = cu[e] + counts[e]
    return counts.astype(np.int32), cu.astype(np.int32)


def dispatch_permutation(idx, E):
    """row_of[s*K+k] and tok_of[row]: a stable counting sort of the (token, k) pairs by expert.

    Expert e owns rows cu[e] .. cu[e+1]-1; inside them its tokens appear in
    ascending token order.  [MEP] guide, dispatch step; [FW] "What's in the
    box", dispatch/combine item (tokens written straight into their expert's
    buffer).
    """
    S, K = idx.shape
    _, cu = expert_counts(idx, E)
    row_of = np.full(S * K, -1, dtype=np.int64)
    tok_of = np.full(S * K, -1, dtype=np.int64)
    for e in range(E):
        # np.nonzero walks idx in row-major order: ascending token, then k
        ss, kk = np.nonzero(np.asarray(idx) == e)
        rows = int(cu[e]) + np.arange(ss.size)
        row_of[ss * K + kk] = rows
        tok_of[rows] = ss
    return row_of.astype(np.int32), tok_of.astype(np.int32)


def dispatch_rows(x, tok_of):
    """xd[row] = x[tok_of[row]] (a copy of each token into each of its K rows)."""
    return np.asarray(x)[np.asarray(tok_of, dtype=np.int64)]


# ------------------------------------------------------------ expert FFN --

def silu(z):
    return z / (1.0 + np.exp(-z))


def expert_ffn(xd, cu, W1, W3, W2, experts=None):
    """Per expert e on its rows X: h1 = X W1[e], h3 = X W3[e], a = silu(h1)*h3, y = a W2[e].

    [T4] "RMSNorm, RoPE, SwiGLU" table, SwiGLU row (three matrix products);
    [MEP] guide, weights step (one contiguous tensor per projection, each
    expert addressed by its index).  ``W1/W3/W2`` may be callables e -> array
    (to stream one expert at a time).  Returns float64 h1, h3, a, y.
    """
    xd = _f64(xd)
    R = xd.shape[0]
    E = len(cu) - 1
    get = (lambda W, e: _f64(W(e) if callable(W) else W[e]))
    Hf = get(W1, 0).shape[1] if R else 0
    H = xd.shape[1]
    h1 = np.zeros((R, Hf)); h3 = np.zeros((R, Hf)); a = np.zeros((R, Hf)); y = np.zeros((R, H))
    for e in range(E) if experts is None else experts:
        r0, r1 = int(cu[e]), int(cu[e + 1])
        if r1 == r0:
            continue
        X = xd[r0:r1]
        h1[r0:r1] = X @ get(W1, e)
        h3[r0:r1] = X @ get(W3, e)
        a[r0:r1] = silu(h1[r0:r1]) * h3[r0:r1]
        y[r0:r1] = a[r0:r1] @ get(W2, e)
    return h1, h3, a, y


def combine(y, row_of, gates):
    """out[s] = sum over k (ascending) of g[s,k] * y[row_of[s*K+k]].  [FW] dispatch/combine item."""
    y = _f64(y)
    S, K = gates.shape
    out = np.zeros((S, y.shape[1]))
    for s in range(S):
        for k in range(K):
            out[s] += float(gates[s, k]) * y[int(row_of[s * K + k])]
    return out


# --------------------------------------------------------------- backward --

def combine_backward(dout, y, row_of, gates):
    """dy[row_of[s*K+k]] = g[s,k] dout[s];  dg[s,k] = <dout[s], y[row_of[s*K+k]]>.

    [FW] "What's in the box", sparse-backward item (gating and dispatch
    gradients taken in one pass).
    """
    dout = _f64(dout); y = _f64(y)
    S, K = gates.shape
    dy = np.zeros_like(y)
    dg = np.zeros((S, K))
    for s in range(S):
        for k in range(K):
            r = int(row_of[s * K + k])
            dy[r] = float(gates[s, k]) * dout[s]
            dg[s, k] = dout[s] @ y[r]
    return dy, dg


def gate_backward(dg, logits, idx, renorm=True):
    """dlogits [S,E] from dg through the gate function; the discrete pick has no gradient.

    renorm: g_k = exp(l_k)/sum_j exp(l_j) over the chosen set, so
            dl[idx_k] = g_k (dg_k - sum_j g_j dg_j), zero elsewhere.
    raw:    g_k = p[idx_k] with p the full softmax, so
            dl[e] = p_e (dp_e - sum_k g_k dg_k) with dp_e = dg_k where e = idx_k, else 0.
    """
    S, K = idx.shape
    E = logits.shape[1]
    g = gate_weights(logits, idx, renorm=renorm)
    dl = np.zeros((S, E))
    if renorm:
        inner = (g * dg).sum(axis=1)
        for s in range(S):
            for k in range(K):
                dl[s, int(idx[s, k])] = g[s, k] * (dg[s, k] - inner[s])
    else:
        p = softmax_probs(logits)
        inner = (g * dg).sum(axis=1)
        for s in range(S):
            dp = np.zeros(E)
            for k in range(K):
                dp[int(idx[s, k])] = dg[s, k]
            dl[s] = p[s] * (dp - inner[s])
    return dl


def expert_ffn_backward(dy, xd, cu, W1, W3, W2, h1, h3, a, experts=None, on_dW=None):
    """Per expert, with X its rows:
        da  = dy W2[e]^T
        dW2 = a^T dy
        dh1 = da * h3 * silu'(h1),  silu'(z) = s(z) (1 + z (1 - s(z))), s = sigmoid
        dh3 = da * silu(h1)
        dxd = dh1 W1[e]^T + dh3 W3[e]^T
        dW1 = X^T dh1,  dW3 = X^T dh3
    Experts with no rows get zero gradients ([MEP] guide, fp32 gradient buffer
    mirroring each projection tensor).  With ``on_dW`` given, each expert's
    (dW1, dW3, dW2) is handed to on_dW(e, ...) instead of being stored (for
    shapes whose gradients do not fit in host memory); the returned dW arrays
    are then None.
    """
    dy = _f64(dy); xd = _f64(xd)
    E = len(cu) - 1
    get = (lambda W, e: _f64(W(e) if callable(W) else W[e]))
    H = xd.shape[1]
    Hf = h1.shape[1]
    R = xd.shape[0]
    dxd = np.zeros((R, H)); dh1 = np.zeros((R, Hf)); dh3 = np.zeros((R, Hf))
    ex = list(range(E)) if experts is None else list(experts)
    if on_dW is None:
        dW1 = np.zeros((len(ex), H, Hf)); dW3 = np.zeros((len(ex), H, Hf))
        dW2 = np.zeros((len(ex), Hf, H))
    else:
        dW1 = dW3 = dW2 = None
    for i, e in enumerate(ex):
        r0, r1 = int(cu[e]), int(cu[e + 1])
        if r1 == r0:
            continue
        X = xd[r0:r1]
        z = _f64(h1[r0:r1]); u = _f64(h3[r0:r1]); A = _f64(a[r0:r1]); D = dy[r0:r1]
        da = D @ get(W2, e).T
        g2 = A.T @ D
        sg = 1.0 / (1.0 + np.exp(-z))
        dh1[r0:r1] = da * u * sg * (1.0 + z * (1.0 - sg))
        dh3[r0:r1] = da * (z * sg)
        dxd[r0:r1] = dh1[r0:r1] @ get(W1, e).T + dh3[r0:r1] @ get(W3, e).T
        g1 = X.T @ dh1[r0:r1]
        g3 = X.T @ dh3[r0:r1]
        if on_dW is None:
            dW1[i], dW3[i], dW2[i] = g1, g3, g2
        else:
            on_dW(e, g1, g3, g2)
    return dxd, dh1, dh3, dW1, dW3, dW2


def dispatch_router_backward(dxd, row_of, dlogits, x, Wg, K):
    """dx[s] = sum_k dxd[row_of[s*K+k]] + sum_e dl[s,e] Wg[:,e];  dWg = x^T dl (no bias gradient)."""
    dxd = _f64(dxd); dl = _f64(dlogits)
    S = dl.shape[0]
    dx = dl @ _f64(Wg).T
    for s in range(S):
        for k in range(K):
            dx[s] += dxd[int(row_of[s * K + k])]
    dWg = _f64(x).T @ dl
    return dx, dWg


# ------------------------------------------------------------ composites --

def moe_forward(x, Wg, bias, W1, W3, W2, K, renorm=True, idx=None, logits=None,
                logits_dtype=np.float32):
    """The whole forward; ``idx``/``logits`` may be given to force the routing (stage-wise parity)."""
    E = Wg.shape[1]
    if logits is None:
        logits = router_logits(x, Wg, bias, out_dtype=logits_dtype)
    if idx is None:
        idx = topk_experts(logits, K)
    gates = gate_weights(logits, idx, renorm)
    counts, cu = expert_counts(idx, E)
    row_of, tok_of = dispatch_permutation(idx, E)
    xd = dispatch_rows(x, tok_of)
    h1, h3, a, y = expert_ffn(xd, cu, W1, W3, W2)
    out = combine(y, row_of, gates)
    return dict(logits=logits, idx=idx, gates=gates, counts=counts, cu=cu, row_of=row_of,
                tok_of=tok_of, xd=xd, h1=h1, h3=h3, a=a, y=y, out=out)


def moe_backward(fw, dout, x, Wg, W1, W3, W2, K, renorm=True, on_dW=None):
    """The whole backward from a ``moe_forward`` record (``on_dW``: see expert_ffn_backward)."""
    dy, dg = combine_backward(dout, fw["y"], fw["row_of"], fw["gates"])
    dl = gate_backward(dg, fw["logits"], fw["idx"], renorm)
    dxd, dh1, dh3, dW1, dW3, dW2 = expert_ffn_backward(dy, fw["xd"], fw["cu"], W1, W3, W2,
                                                       fw["h1"], fw["h3"], fw["a"], on_dW=on_dW)
    dx, dWg = dispatch_router_backward(dxd, fw["row_of"], dl, x, Wg, K)
    return dict(dy=dy, dg=dg, dlogits=dl, dxd=dxd, dh1=dh1, dh3=dh3, dW1=dW1, dW3=dW3,
                dW2=dW2, dx=dx, dWg=dWg)


def maxvio(counts):
    """max_e counts[e] / mean(counts) - 1 ([MEP] "Which problem MoonEP solves": 0 is perfect balance)."""
    c = np.asarray(counts, dtype=F64)
    return float(c.max() / c.mean() - 1.0)


def load_entropy(counts):
    """-sum_e f_e ln f_e over the experts with f_e = counts[e] / sum(counts) > 0 (natural log).

    A second load statistic of the routing histogram next to maxvio ([MEP]
    "Which problem MoonEP solves": the per-expert load the dispatch must
    absorb): ln E for a perfectly balanced load, 0 when one expert takes
    every pair.  The pages name no formula; this is the Shannon entropy of
    the load distribution.
    """
    c = np.asarray(counts, dtype=F64)
    tot = c.sum()
    if tot == 0:
        return 0.0
    h = 0.0
    for v in c:
        if v > 0:
            f = v / tot
            h -= f * np.log(f)
    return float(h)
