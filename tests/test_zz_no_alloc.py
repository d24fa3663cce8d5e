"""moe_dispatch_noalloc (the dispatch without a workspace) against moe_dispatch.

Both entry points run the same kernels; the allocation-free one keeps the
per-block bitmaps, counts and bases in the library's own per-GPU scratch.
Two calls in a row on that scratch, the second smaller than the first, must
each give moe_dispatch's outputs bit for bit (integer outputs and the xd
copy), and the oracle's counting sort as well.
"""
import sys

import numpy as np
import pytest

import oracle
from tests.moe_testutil import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from routing_dispatch_grouped_moe_amd import _lib as L  # noqa: E402


def _topk(S, E, K, rng):
    # K distinct experts per token: the first K of a random key order per row
    return np.argsort(rng.random((S, E)), axis=1)[:, :K].astype(np.int32)


def _outputs(S, H, E, K):
    cu = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_of = torch.full((S * K,), -7, dtype=torch.int32, device="cuda")
    tok_of = torch.full((S * K,), -7, dtype=torch.int32, device="cuda")
    xd = torch.zeros(S * K, H, dtype=torch.bfloat16, device="cuda")
    return cu, row_of, tok_of, xd


def _both(S, H, E, K, seed):
    print(f"[noalloc] S={S} H={H} E={E} K={K}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(seed)
    idx = _topk(S, E, K, rng)
    x = to_dev(rng.standard_normal((S, H), dtype=np.float32), "bf16")
    idx_t = torch.from_numpy(idx).cuda()
    d = L.dims(S, H, 128, E, K, "bf16")
    ws = torch.zeros(L.moe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    L.moe_clear_status(ws)
    ref = _outputs(S, H, E, K)
    L.moe_dispatch(d, x, idx_t, *ref, ws)
    got = _outputs(S, H, E, K)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.moe_dispatch_noalloc(d, x, idx_t, *got, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and L.moe_read_status(ws) == 0
    for name, a, b in zip(("cu_seqlens", "row_of", "tok_of"), ref[:3], got[:3]):
        assert torch.equal(a, b), name
    assert torch.equal(ref[3].view(torch.int16), got[3].view(torch.int16)), "xd"
    counts, cu = oracle.expert_counts(idx, E)
    row_of, tok_of = oracle.dispatch_permutation(idx, E)
    np.testing.assert_array_equal(got[0].cpu().numpy(), cu)
    np.testing.assert_array_equal(got[1].cpu().numpy(), row_of)
    np.testing.assert_array_equal(got[2].cpu().numpy(), tok_of)


def test_noalloc_two_calls_second_smaller():
    # the MoonEP shape's dispatch (tokens 8192, 384 experts, top-8), then a
    # smaller, ragged one on the scratch the first call left behind
    _both(8192, 256, 384, 8, seed=1)
    _both(1000, 384, 384, 8, seed=2)


def test_noalloc_largest_accepted_size():
    # ceil(S / 256) * E = 102 * 1024 cells fill the scratch to 4 178 176 bytes
    _both(26112, 128, 1024, 2, seed=3)


def test_noalloc_reports_bad_expert_into_caller_word():
    S, H, E, K = 300, 128, 16, 2
    rng = np.random.default_rng(5)
    idx = _topk(S, E, K, rng)
    idx[7, 1] = E + 3  # outside [0, E)
    x = to_dev(rng.standard_normal((S, H), dtype=np.float32), "bf16")
    d = L.dims(S, H, 128, E, K, "bf16")
    out = _outputs(S, H, E, K)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.moe_dispatch_noalloc(d, x, torch.from_numpy(idx).cuda(), *out, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & L.MOE_DEV_BAD_EXPERT
    assert int(out[1][7 * K + 1].item()) == -1
    # and without a status word the call still completes
    L.moe_dispatch_noalloc(d, x, torch.from_numpy(idx).cuda(), *out)
    torch.cuda.synchronize()
