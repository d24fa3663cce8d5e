"""Buffers and call sequence of one MoE layer over the C ABI.

torch only allocates device memory and supplies the stream; every step is one
of the library's entry points (moe_route, moe_dispatch, moe_ffn_up,
moe_ffn_down, moe_combine, moe_backward, and the moe_mod_* calls).
"""
from __future__ import annotations

import torch

from . import _lib as L


class MoELayer:
    """Owns the activation, intermediate and gradient buffers of one layer shape."""

    def __init__(self, S, H, Hf, E, K, dtype="bf16", device="cuda", flags=L.MOE_F_RENORM,
                 backward=True, write_logits=True):
        self.S, self.H, self.Hf, self.E, self.K = int(S), int(H), int(Hf), int(E), int(K)
        self.bf16 = dtype in ("bf16", torch.bfloat16)
        self.tdt = torch.bfloat16 if self.bf16 else torch.float32
        self.d = L.dims(S, H, Hf, E, K, L.MOE_BF16 if self.bf16 else L.MOE_F32, flags)
        nb = L.moe_workspace_bytes(self.d)
        if nb == 0:
            raise ValueError(f"unsupported layer dims S={S} H={H} Hf={Hf} E={E} K={K}")
        dev = torch.device(device)
        R = self.S * self.K
        self.R = R
        f32, i32, t = torch.float32, torch.int32, self.tdt
        e = lambda *shape, dtype=t: torch.empty(shape, dtype=dtype, device=dev)
        self.ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
        self.logits = e(S, E, dtype=f32) if write_logits else None
        self.topk_idx = e(S, K, dtype=i32)
        self.gates = e(S, K, dtype=f32)
        self.counts = e(E, dtype=i32)
        self.cu = e(E + 1, dtype=i32)
        self.row_of = e(R, dtype=i32)
        self.tok_of = e(R, dtype=i32)
        self.xd = e(R, H)
        # under recompute h1, h3 are not kept between forward and backward
        self.recompute = bool(flags & L.MOE_F_RECOMPUTE)
        self.h1 = None if self.recompute else e(R, Hf)
        self.h3 = None if self.recompute else e(R, Hf)
        self.a = e(R, Hf)
        self.y = e(R, H)
        self.out = e(S, H)
        self.has_bwd = backward
        if backward:
            self.dy = e(R, H)
            self.dh1 = e(R, Hf)
            self.dh3 = e(R, Hf)
            self.dxd = e(R, H)
            self.dgates = e(S, K, dtype=f32)
            self.dlogits = e(S, E, dtype=f32)
            self.dx = e(S, H)
            self.dWg = e(H, E, dtype=f32)
            self.dW1 = e(E, H, Hf, dtype=f32)
            self.dW3 = e(E, H, Hf, dtype=f32)
            self.dW2 = e(E, Hf, H, dtype=f32)

    # forward ----------------------------------------------------------------
    def route(self, x, Wg, bias=None):
        L.moe_route(self.d, x, Wg, bias, self.logits, self.topk_idx, self.gates, self.counts, self.ws)

    def dispatch(self, x):
        L.moe_dispatch(self.d, x, self.topk_idx, self.cu, self.row_of, self.tok_of, self.xd, self.ws)

    def ffn(self, W1, W3, W2):
        L.moe_ffn_up(self.d, self.xd, self.cu, W1, W3, self.h1, self.h3, self.a, self.ws)
        L.moe_ffn_down(self.d, self.a, self.cu, W2, self.y, self.ws)

    def combine(self):
        L.moe_combine(self.d, self.y, self.row_of, self.gates, self.out)

    def forward(self, x, Wg, bias, W1, W3, W2):
        self.route(x, Wg, bias)
        self.dispatch(x)
        self.ffn(W1, W3, W2)
        self.combine()
        return self.out

    # backward ---------------------------------------------------------------
    def backward(self, dout, x, Wg, W1, W3, W2):
        saved = dict(x=x, Wg=Wg, W1=W1, W3=W3, W2=W2, xd=self.xd, h1=self.h1, h3=self.h3, a=self.a,
                     y=self.y, topk_idx=self.topk_idx, gates=self.gates, cu_seqlens=self.cu,
                     row_of=self.row_of, tok_of=self.tok_of, logits=self.logits)
        bufs = dict(dy=self.dy, dh1=self.dh1, dh3=self.dh3, dxd=self.dxd, dgates=self.dgates,
                    dlogits=self.dlogits)
        L.moe_backward(self.d, saved, dout, self.dx, self.dWg, self.dW1, self.dW3, self.dW2, bufs,
                       self.ws)
        return self.dx

    def status(self):
        return L.moe_read_status(self.ws)


class MoDMoELayer:
    """Mixture-of-Depths selection around a MoE layer: B sequences of T tokens, C kept each."""

    def __init__(self, B, T, C, H, Hf, E, K, dtype="bf16", device="cuda", flags=L.MOE_F_RENORM):
        self.B, self.T, self.C, self.H = int(B), int(T), int(C), int(H)
        self.moe = MoELayer(B * C, H, Hf, E, K, dtype, device, flags)
        t, dev = self.moe.tdt, torch.device(device)
        self.dt = L.MOE_BF16 if self.moe.bf16 else L.MOE_F32
        self.flags = flags
        S = B * T
        self.r = torch.empty(S, dtype=torch.float32, device=dev)
        self.keep = torch.empty(max(B * C, 1), dtype=torch.int32, device=dev)
        self.xk = torch.empty(B * C, H, dtype=t, device=dev)
        self.out = torch.empty(S, H, dtype=t, device=dev)
        self.dm = torch.empty(B * C, H, dtype=t, device=dev)
        self.dr = torch.empty(max(B * C, 1), dtype=torch.float32, device=dev)
        self.dx = torch.empty(S, H, dtype=t, device=dev)
        self.dw_r = torch.empty(H, dtype=torch.float32, device=dev)
        self.mws = torch.empty(L.moe_mod_workspace_bytes(H), dtype=torch.uint8, device=dev)

    def forward(self, x, w_r, Wg, bias, W1, W3, W2):
        L.moe_mod_select(self.B, self.T, self.C, self.H, self.dt, x, w_r, self.r, self.keep, self.xk)
        m = self.moe.forward(self.xk, Wg, bias, W1, W3, W2)
        L.moe_mod_merge(self.B, self.T, self.C, self.H, self.dt, x, self.r, self.keep, m, self.out)
        return self.out

    def backward(self, dout, x, w_r, Wg, W1, W3, W2):
        L.moe_mod_backward(self.B, self.T, self.C, self.H, self.dt, self.flags, x, w_r, self.r,
                           self.keep, self.moe.out, dout, None, self.dm, self.dr, None, None, None)
        dxk = self.moe.backward(self.dm, self.xk, Wg, W1, W3, W2)
        L.moe_mod_backward(self.B, self.T, self.C, self.H, self.dt, self.flags, x, w_r, self.r,
                           self.keep, self.moe.out, dout, dxk, self.dm, self.dr, self.dx, self.dw_r,
                           self.mws)
        return self.dx
