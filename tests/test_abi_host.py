"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, sizes its workspace, and rejects invalid arguments before launching."""
import ctypes as C
import os
import re

import numpy as np

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from routing_dispatch_grouped_moe_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmoe_amd.so not built (python -m routing_dispatch_grouped_moe_amd.build)")
    _lib.load()
    return _lib


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert "moe_route" in names and "moe_backward" in names
    lib = C.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"
    assert set(names) == set(L.EXPORTS)


def test_workspace_bytes_and_invalid_dims(L):
    d = L.dims(8192, 7168, 2048, 384, 8, "bf16")
    nb = L.moe_workspace_bytes(d)
    assert nb > 0 and nb % 256 == 0
    bad = [
        L.dims(8, 100, 128, 8, 2, "bf16"),    # H not a multiple of 128
        L.dims(8, 128, 128, 8, 9, "bf16"),    # K > E
        L.dims(8, 128, 128, 2000, 2, "bf16"),  # E > 1024
        L.dims(8, 128, 128, 64, 17, "bf16"),  # K > 16
        L.dims(-1, 128, 128, 8, 2, "bf16"),
        L.Dims(8, 128, 128, 8, 2, 7, 1),      # bad dtype
        L.dims(1 << 28, 128, 128, 16, 16, "bf16"),  # S*K overflows int32
    ]
    for b in bad:
        assert L.moe_workspace_bytes(b) == 0


def _raw(L):
    return L.load()


FAKE = C.c_void_p(1 << 20)        # aligned, never dereferenced: validation fails first
MISALIGNED = C.c_void_p((1 << 20) + 4)


def test_route_rejects_before_launch(L):
    lib = _raw(L)
    d = L.dims(64, 128, 256, 8, 2, "f32")
    ws_n = L.moe_workspace_bytes(d)
    args = [FAKE] * 7
    # null x
    st = lib.moe_route(C.byref(d), None, *args[1:], FAKE, ws_n, None)
    assert st == 1
    # misaligned topk_idx
    st = lib.moe_route(C.byref(d), FAKE, FAKE, None, None, MISALIGNED, FAKE, FAKE, FAKE, ws_n, None)
    assert st == 4
    # workspace too small
    st = lib.moe_route(C.byref(d), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, ws_n - 256, None)
    assert st == 5
    # K > E
    d2 = L.dims(64, 128, 256, 2, 3, "f32")
    st = lib.moe_route(C.byref(d2), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, ws_n, None)
    assert st == 6
    # bad dtype
    d3 = L.Dims(64, 128, 256, 8, 2, 5, 1)
    st = lib.moe_route(C.byref(d3), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, ws_n, None)
    assert st == 3
    # null dims
    st = lib.moe_route(None, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, ws_n, None)
    assert st == 1


def test_other_entry_points_reject_before_launch(L):
    lib = _raw(L)
    d = L.dims(64, 128, 256, 8, 2, "bf16")
    ws_n = L.moe_workspace_bytes(d)
    assert lib.moe_dispatch(C.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws_n, None) == 1
    assert lib.moe_grouped_ffn(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, 0, None) == 5
    assert lib.moe_ffn_up(C.byref(d), FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE, FAKE, FAKE, ws_n,
                          None) == 4
    assert lib.moe_ffn_down(C.byref(d), FAKE, None, FAKE, FAKE, FAKE, ws_n, None) == 1
    assert lib.moe_combine(C.byref(d), FAKE, FAKE, None, FAKE, None) == 1
    dshape = L.dims(64, 192, 256, 8, 2, "bf16")
    assert lib.moe_combine(C.byref(dshape), FAKE, FAKE, FAKE, FAKE, None) == 6
    # backward: raw (non-renormalised) gates need the saved logits
    sv = L.Saved(*([1 << 20] * 15 + [0]))
    bb = L.BwdBufs(*([1 << 20] * 6))
    draw = L.dims(64, 128, 256, 8, 2, "bf16", flags=0)
    assert lib.moe_backward(C.byref(draw), C.byref(sv), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            C.byref(bb), FAKE, ws_n, None) == 1
    assert lib.moe_backward(C.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, C.byref(bb), FAKE,
                            ws_n, None) == 1
    sv_bad = L.Saved(*([1 << 20] * 14 + [0]))
    assert lib.moe_backward(C.byref(d), C.byref(sv_bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            C.byref(bb), FAKE, ws_n, None) == 1
    # load statistics
    assert lib.moe_load_stats(0, FAKE, FAKE, None) == 2
    assert lib.moe_load_stats(1025, FAKE, FAKE, None) == 2
    assert lib.moe_load_stats(8, None, FAKE, None) == 1
    # MoD
    assert lib.moe_mod_select(4, 2048, 3000, 4096, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 6
    assert lib.moe_mod_select(4, 10000, 10, 4096, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 6
    assert lib.moe_mod_select(4, 2048, 1024, 4000, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 6
    assert lib.moe_mod_merge(0, 2048, 1024, 4096, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert lib.moe_mod_backward(4, 2048, 1024, 4096, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == 5
    assert L.moe_mod_workspace_bytes(4096) > 0


def test_dispatch_noalloc_rejects_before_launch(L):
    """The allocation-free dispatch validates like moe_dispatch and refuses sizes past its scratch."""
    lib = _raw(L)
    f = lib.moe_dispatch_noalloc
    d = L.dims(8192, 7168, 2048, 384, 8, "bf16")
    assert f(C.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert f(C.byref(d), FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE, None, None) == 4
    assert f(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, C.c_void_p((1 << 20) + 2), None) == 4
    assert f(C.byref(L.dims(64, 100, 128, 8, 2, "bf16")), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
             None, None) == 6
    # scratch limit: 256 + 40 * ceil(S / 256) * E bytes (regions rounded to 256) <= 4 MiB;
    # only sizes past it are passed here (a size that fits would go on to launch, which
    # the GPU test covers at the boundary itself)
    for S, E in ((26113, 1024), (69889, 384), (2 ** 22, 64), (2 ** 22, 8)):
        st = f(C.byref(L.dims(S, 128, 128, E, 2, "bf16")), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
               None, None)
        assert st == 5, (S, E, st)


def test_status_strings(L):
    lib = _raw(L)
    for code, name in [(0, b"ok"), (5, b"workspace too small"), (7, b"HIP launch error")]:
        assert lib.moe_status_string(code) == name


def _expected_dims_status(S, H, Hf, E, K, dtype):
    """The size contract stated in include/moe.h, restated: 0 for valid dims, else the error."""
    if dtype not in (0, 1):
        return 3
    if S < 0 or H <= 0 or Hf <= 0 or E <= 0 or K <= 0:
        return 2
    if E > 1024 or K > 16 or K > E:
        return 6
    if H % 128 or Hf % 128 or H > 65536 or Hf > 65536:
        return 6
    if S * K >= 2 ** 31 or S * max(H, Hf) >= 2 ** 30 or H * Hf >= 2 ** 30:
        return 2
    return 0


def test_dims_contract_on_random_sizes(L):
    """Random sizes around every limit: the library accepts exactly the documented ones.

    Valid dims size a workspace (> 0, 256-aligned); invalid dims size none and
    make every entry point return the documented error before anything is
    launched.  Valid dims are only ever passed with NULL tensors, so the calls
    stop at argument validation (MOE_ERR_NULL) and never reach a kernel.
    """
    lib = _raw(L)
    rng = np.random.default_rng(11)
    picks = {
        "S": [0, 1, 63, 8192, 2 ** 20, 2 ** 27, -1],
        "H": [128, 256, 4096, 7168, 65536, 65536 + 128, 100, 0, -128],
        "Hf": [128, 1408, 2048, 14336, 65536, 131072, 200, 0],
        "E": [1, 8, 384, 1024, 1025, 0, -3],
        "K": [1, 2, 8, 16, 17, 0],
        "dtype": [0, 1, 2, -1],
    }
    for _ in range(400):
        v = {k: int(rng.choice(c)) for k, c in picks.items()}
        want = _expected_dims_status(**v)
        d = L.Dims(v["S"], v["H"], v["Hf"], v["E"], v["K"], v["dtype"], 1)
        nb = lib.moe_workspace_bytes(C.byref(d))
        if want == 0:
            assert nb > 0 and nb % 256 == 0, v
            st = lib.moe_route(C.byref(d), None, None, None, None, None, None, None, None, 0, None)
            assert st == 1, (v, st)
        else:
            assert nb == 0, v
            st = lib.moe_route(C.byref(d), None, None, None, None, None, None, None, None, 0, None)
            assert st == want, (v, st, want)
            st = lib.moe_combine(C.byref(d), None, None, None, None, None)
            assert st == want, (v, st, want)
