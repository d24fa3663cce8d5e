"""ctypes binding of libmoe_amd.so (argument marshalling only).

Every function here has the name of a C entry point declared in
include/moe.h and passes plain device pointers, sizes and the current HIP
stream through; all work runs in the library's kernels.  torch is imported
before the library is loaded so that the library binds to the same HIP
runtime instance as torch (both use the soname libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # noqa: F401  (must be loaded first: one HIP runtime per process)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_amd.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_F_RENORM, MOE_F_ACCUM_GRAD, MOE_F_RECOMPUTE = 1, 2, 8
MOE_DEV_NONFINITE_LOGIT, MOE_DEV_BAD_EXPERT, MOE_DEV_DUP_EXPERT = 1, 2, 4
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_DTYPE",
                4: "MOE_ERR_ALIGN", 5: "MOE_ERR_WORKSPACE", 6: "MOE_ERR_UNSUPPORTED",
                7: "MOE_ERR_HIP"}

# Every entry point include/moe.h declares (checked by the CPU test suite).
EXPORTS = (
    "moe_workspace_bytes", "moe_clear_status", "moe_status_string", "moe_read_status",
    "moe_route", "moe_load_stats", "moe_dispatch", "moe_dispatch_noalloc", "moe_grouped_ffn",
    "moe_ffn_up", "moe_ffn_down", "moe_combine", "moe_backward", "moe_mod_workspace_bytes", "moe_mod_select",
    "moe_mod_merge", "moe_mod_backward", "moe_timer_enable", "moe_timer_reset",
    "moe_timer_read",
)


class Dims(C.Structure):
    _fields_ = [("S", C.c_int64), ("H", C.c_int32), ("Hf", C.c_int32), ("E", C.c_int32),
                ("K", C.c_int32), ("dtype", C.c_int32), ("flags", C.c_uint32)]


class Saved(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "x", "Wg", "W1", "W3", "W2", "xd", "h1", "h3", "a", "y", "topk_idx", "gates",
        "cu_seqlens", "row_of", "tok_of", "logits")]


class BwdBufs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("dy", "dh1", "dh3", "dxd", "dgates", "dlogits")]


class MoeError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {STATUS_NAMES.get(code, code)}")
        self.code = code


_lib = None


def load():
    """Load libmoe_amd.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          f"`python -m routing_dispatch_grouped_moe_amd.build`")
    lib = C.CDLL(LIB_PATH)
    P, S, I32, I64, U32 = C.c_void_p, C.c_size_t, C.c_int32, C.c_int64, C.c_uint32
    D = C.POINTER(Dims)
    sig = {
        "moe_workspace_bytes": (S, [D]),
        "moe_clear_status": (I32, [P, P]),
        "moe_status_string": (C.c_char_p, [I32]),
        "moe_read_status": (I32, [P, C.POINTER(U32), P]),
        "moe_route": (I32, [D, P, P, P, P, P, P, P, P, S, P]),
        "moe_dispatch": (I32, [D, P, P, P, P, P, P, P, S, P]),
        "moe_dispatch_noalloc": (I32, [D, P, P, P, P, P, P, P, P]),
        "moe_load_stats": (I32, [I32, P, P, P]),
        "moe_grouped_ffn": (I32, [D, P, P, P, P, P, P, P, P, P, P, S, P]),
        "moe_ffn_up": (I32, [D, P, P, P, P, P, P, P, P, S, P]),
        "moe_ffn_down": (I32, [D, P, P, P, P, P, S, P]),
        "moe_combine": (I32, [D, P, P, P, P, P]),
        "moe_backward": (I32, [D, C.POINTER(Saved), P, P, P, P, P, P, C.POINTER(BwdBufs), P, S, P]),
        "moe_mod_workspace_bytes": (S, [I32]),
        "moe_mod_select": (I32, [I32, I32, I32, I32, I32, P, P, P, P, P, P]),
        "moe_mod_merge": (I32, [I32, I32, I32, I32, I32, P, P, P, P, P, P]),
        "moe_mod_backward": (I32, [I32, I32, I32, I32, I32, U32, P, P, P, P, P, P, P, P, P, P, P,
                                   P, S, P]),
        "moe_timer_enable": (None, [I32]),
        "moe_timer_reset": (None, []),
        "moe_timer_read": (I32, [C.POINTER(C.c_char_p), C.POINTER(C.c_double),
                                 C.POINTER(I64), I32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, code):
    if code != 0:
        raise MoeError(fn, code)


def dims(S, H, Hf, E, K, dtype, flags=MOE_F_RENORM):
    dt = dtype if isinstance(dtype, int) else (MOE_BF16 if dtype in ("bf16", torch.bfloat16) else MOE_F32)
    return Dims(int(S), int(H), int(Hf), int(E), int(K), dt, int(flags))


def moe_workspace_bytes(d):
    return int(load().moe_workspace_bytes(C.byref(d)))


def moe_clear_status(ws):
    _check("moe_clear_status", load().moe_clear_status(_p(ws), _stream()))


def moe_read_status(ws):
    v = C.c_uint32(0)
    _check("moe_read_status", load().moe_read_status(_p(ws), C.byref(v), _stream()))
    return int(v.value)


def moe_route(d, x, Wg, bias, logits, topk_idx, gates, counts, ws):
    _check("moe_route", load().moe_route(C.byref(d), _p(x), _p(Wg), _p(bias), _p(logits),
                                         _p(topk_idx), _p(gates), _p(counts), _p(ws),
                                         ws.numel() * ws.element_size(), _stream()))


def moe_load_stats(E, counts, stats):
    """stats [2] fp32 (device) <- (maxvio, load entropy) of the counts [E] int32 (device)."""
    _check("moe_load_stats", load().moe_load_stats(int(E), _p(counts), _p(stats), _stream()))


def moe_dispatch(d, x, topk_idx, cu_seqlens, row_of, tok_of, xd, ws):
    _check("moe_dispatch", load().moe_dispatch(C.byref(d), _p(x), _p(topk_idx), _p(cu_seqlens),
                                               _p(row_of), _p(tok_of), _p(xd), _p(ws),
                                               ws.numel() * ws.element_size(), _stream()))


def moe_dispatch_noalloc(d, x, topk_idx, cu_seqlens, row_of, tok_of, xd, status=None):
    """moe_dispatch on the library's own scratch (no workspace); status: optional device uint32."""
    _check("moe_dispatch_noalloc", load().moe_dispatch_noalloc(
        C.byref(d), _p(x), _p(topk_idx), _p(cu_seqlens), _p(row_of), _p(tok_of), _p(xd),
        _p(status), _stream()))


def moe_grouped_ffn(d, xd, cu_seqlens, W1, W3, W2, h1, h3, a, y, ws):
    _check("moe_grouped_ffn", load().moe_grouped_ffn(
        C.byref(d), _p(xd), _p(cu_seqlens), _p(W1), _p(W3), _p(W2), _p(h1), _p(h3), _p(a), _p(y),
        _p(ws), ws.numel() * ws.element_size(), _stream()))


def moe_ffn_up(d, xd, cu_seqlens, W1, W3, h1, h3, a, ws):
    _check("moe_ffn_up", load().moe_ffn_up(C.byref(d), _p(xd), _p(cu_seqlens), _p(W1), _p(W3),
                                           _p(h1), _p(h3), _p(a), _p(ws),
                                           ws.numel() * ws.element_size(), _stream()))


def moe_ffn_down(d, a, cu_seqlens, W2, y, ws):
    _check("moe_ffn_down", load().moe_ffn_down(C.byref(d), _p(a), _p(cu_seqlens), _p(W2), _p(y),
                                               _p(ws), ws.numel() * ws.element_size(), _stream()))


def moe_combine(d, y, row_of, gates, out):
    _check("moe_combine", load().moe_combine(C.byref(d), _p(y), _p(row_of), _p(gates), _p(out),
                                             _stream()))


def moe_backward(d, saved: dict, dout, dx, dWg, dW1, dW3, dW2, bufs: dict, ws):
    sv = Saved(**{k: (saved[k].data_ptr() if saved.get(k) is not None else None)
                  for k, _ in Saved._fields_})
    bb = BwdBufs(**{k: (bufs[k].data_ptr() if bufs.get(k) is not None else None)
                    for k, _ in BwdBufs._fields_})
    _check("moe_backward", load().moe_backward(
        C.byref(d), C.byref(sv), _p(dout), _p(dx), _p(dWg), _p(dW1), _p(dW3), _p(dW2),
        C.byref(bb), _p(ws), ws.numel() * ws.element_size(), _stream()))


def moe_mod_workspace_bytes(H):
    return int(load().moe_mod_workspace_bytes(int(H)))


def moe_mod_select(B, T, Cn, H, dtype, x, w_r, r, keep_idx, xk):
    _check("moe_mod_select", load().moe_mod_select(B, T, Cn, H, dtype, _p(x), _p(w_r), _p(r),
                                                   _p(keep_idx), _p(xk), _stream()))


def moe_mod_merge(B, T, Cn, H, dtype, x, r, keep_idx, m, out):
    _check("moe_mod_merge", load().moe_mod_merge(B, T, Cn, H, dtype, _p(x), _p(r), _p(keep_idx),
                                                 _p(m), _p(out), _stream()))


def moe_mod_backward(B, T, Cn, H, dtype, flags, x, w_r, r, keep_idx, m, dout, dxk, dm, dr, dx,
                     dw_r, ws):
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_mod_backward", load().moe_mod_backward(
        B, T, Cn, H, dtype, flags, _p(x), _p(w_r), _p(r), _p(keep_idx), _p(m), _p(dout),
        _p(dxk), _p(dm), _p(dr), _p(dx), _p(dw_r), _p(ws), nb, _stream()))


def moe_timer_enable(on=True):
    load().moe_timer_enable(1 if on else 0)


def moe_timer_reset():
    load().moe_timer_reset()


def moe_timer_read():
    """{kernel name: (total ms, launches)} since the last reset."""
    lib = load()
    cap = 64
    names = (C.c_char_p * cap)()
    ms = (C.c_double * cap)()
    n = (C.c_int64 * cap)()
    k = lib.moe_timer_read(names, ms, n, cap)
    return {names[i].decode(): (float(ms[i]), int(n[i])) for i in range(min(k, cap))}
