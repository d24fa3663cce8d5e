"""The layer step captured in a HIP graph (through torch.cuda.graph) and replayed.

The library allocates nothing, sets no memory with hipMemsetAsync and does not
synchronise inside a step, so one forward + backward can be captured and
replayed.  Each replay must give the eager step's outputs bit for bit; the
outputs are cleared by eager work between replays, so a replay that skipped
a kernel would show.
"""
import sys

import numpy as np
import pytest

from synth import make_workload
from tests.moe_testutil import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from routing_dispatch_grouped_moe_amd import MoELayer  # noqa: E402
from routing_dispatch_grouped_moe_amd import _lib as L  # noqa: E402

OUTS = ["logits", "topk_idx", "gates", "counts", "cu", "row_of", "tok_of", "xd", "a", "y", "out",
        "dy", "dh1", "dh3", "dxd", "dgates", "dlogits", "dx", "dWg", "dW1", "dW3", "dW2"]


@pytest.mark.parametrize("cfg,ov,flags", [
    ("c2", dict(S=300, H=256, Hf=384), L.MOE_F_RENORM),
    ("c4", dict(S=640, H=256, Hf=384, beta=4.0), L.MOE_F_RENORM | L.MOE_F_RECOMPUTE),
    ("c3", dict(S=257, H=256, Hf=256), 0),
    # 128 tokens x 384 experts: the tiled router cuts H = 2048 into 8 parts
    # (partial logits, then the part sum, then the top-K launch)
    ("c4", dict(S=128, H=2048, Hf=256), L.MOE_F_RENORM),
], ids=["c2_renorm", "c4_skewed_recompute", "c3_raw_gates", "c4_router_parts"])
def test_graph_replay_matches_eager(cfg, ov, flags):
    print(f"[graph] {cfg} {ov} flags={flags}", flush=True)
    sys.stdout.flush()
    wl = make_workload(cfg, host_weights=True, **ov)
    dt = wl.dtype
    x, Wg, dout = to_dev(wl.x, dt), to_dev(wl.Wg, dt), to_dev(wl.dout, dt)
    W1, W3, W2 = to_dev(wl.W1, dt), to_dev(wl.W3, dt), to_dev(wl.W2, dt)
    b = None if wl.bias is None else torch.from_numpy(wl.bias.astype(np.float32)).cuda()
    layer = MoELayer(wl.S, wl.H, wl.Hf, wl.E, wl.K, dt, flags=flags)

    def step():
        layer.forward(x, Wg, b, W1, W3, W2)
        layer.backward(dout, x, Wg, W1, W3, W2)

    step()
    torch.cuda.synchronize()
    ref = {n: getattr(layer, n).clone() for n in OUTS}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for n in OUTS:
            getattr(layer, n).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert layer.status() == 0
        for n in OUTS:
            assert torch.equal(getattr(layer, n), ref[n]), f"replay {rep}: {n} differs from eager"
    print(f"[graph] {cfg}: 3 replays equal to the eager step", flush=True)
