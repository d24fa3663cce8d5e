"""moe_dispatch alone against the oracle's stable counting sort, bit for bit.

The dispatch permutation has a plain definition (MoonEP page, step-by-step
guide: every (token, k) pair gets a row, experts' rows contiguous, cu_seqlens
the offsets; rows of one expert in ascending token order), so the oracle's
counting sort fixes every integer output and xd is an exact copy.  The cases
cover the count-table scan in both of its forms (the [blocks][experts] table
staged in LDS, in one or more rounds of loads, and the larger tables that
take the per-expert walk through global memory), the LDS budget's boundary,
ragged token counts, empty experts and one expert taking every pair.
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


def random_topk(S, E, K, rng, hot=None):
    """K distinct experts per token (uniform, or with expert `hot` in every token's set)."""
    idx = np.empty((S, K), np.int32)
    for s in range(S):
        if hot is None:
            idx[s] = rng.choice(E, size=K, replace=False)
        else:
            rest = rng.choice(np.setdiff1d(np.arange(E), [hot]), size=K - 1, replace=False)
            idx[s] = np.concatenate([[hot], rest])
    return idx


def run_dispatch(S, H, E, K, idx, x_host, dtype="bf16"):
    d = L.dims(S, H, 128, E, K, dtype)
    ws = torch.zeros(L.moe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    L.moe_clear_status(ws)
    x = to_dev(x_host, dtype)
    idx_t = torch.from_numpy(idx).cuda()
    cu = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_of = torch.empty(S * K, dtype=torch.int32, device="cuda")
    tok_of = torch.empty(S * K, dtype=torch.int32, device="cuda")
    xd = torch.empty(S * K, H, dtype=x.dtype, device="cuda")
    L.moe_dispatch(d, x, idx_t, cu, row_of, tok_of, xd, ws)
    torch.cuda.synchronize()
    assert L.moe_read_status(ws) == 0
    return x, cu, row_of, tok_of, xd


CASES = [
    # (S, H, E, K, hot)      count table nb x E (LDS holds 32768 entries)
    (8192, 128, 384, 8, None),     # 32 x 384: the MoonEP shape's table, LDS
    (1000, 256, 64, 4, None),      # 4 x 64, ragged last block
    (300, 128, 8, 2, 5),           # one expert in every token's set
    (33000, 128, 1024, 2, None),   # 129 x 1024 > 32768: global-memory walk
    (32768, 128, 1024, 1, None),   # 128 x 1024 = 131072: global-memory walk
    (8193, 128, 1024, 4, None),    # 33 x 1024 = 33792: just past the LDS table
    (8192, 128, 1024, 4, None),    # 32 x 1024 = 32768: exactly the LDS table
    (20000, 128, 256, 2, None),    # 79 x 256: LDS, more than one round of loads
    (70, 128, 1000, 16, None),     # most experts empty
]


@pytest.mark.parametrize("S,H,E,K,hot", CASES, ids=[f"S{c[0]}_E{c[2]}_K{c[3]}" for c in CASES])
def test_dispatch_matches_counting_sort(S, H, E, K, hot):
    print(f"[dispatch] S={S} H={H} E={E} K={K} hot={hot}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(S * 31 + E)
    idx = random_topk(S, E, K, rng, hot)
    xh = rng.standard_normal((S, H), dtype=np.float32)
    x, cu, row_of, tok_of, xd = run_dispatch(S, H, E, K, idx, xh)
    counts, cu_o = oracle.expert_counts(idx, E)
    ro, to = oracle.dispatch_permutation(idx, E)
    np.testing.assert_array_equal(cu.cpu().numpy(), cu_o, err_msg="cu_seqlens")
    np.testing.assert_array_equal(row_of.cpu().numpy(), ro, err_msg="row_of")
    np.testing.assert_array_equal(tok_of.cpu().numpy(), to, err_msg="tok_of")
    tok_t = torch.from_numpy(to.astype(np.int64)).cuda()
    assert torch.equal(xd.view(torch.int16), x.view(torch.int16)[tok_t]), "xd"


def test_dispatch_repeatable_bitwise():
    S, H, E, K = 5000, 256, 384, 8
    rng = np.random.default_rng(3)
    idx = random_topk(S, E, K, rng)
    xh = rng.standard_normal((S, H), dtype=np.float32)
    a = run_dispatch(S, H, E, K, idx, xh)
    b = run_dispatch(S, H, E, K, idx, xh)
    for u, v in zip(a[1:], b[1:]):
        assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.uint8) if v.dtype == torch.bfloat16 else v)
