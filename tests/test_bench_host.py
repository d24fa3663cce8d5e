"""bench.py pieces that need no GPU: the one-GPU guard and the per-kernel cost model."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_cost_model_at_the_384_expert_shape():
    # S = 8192, H = 7168, H' = 2048, E = 384, K = 8, bf16, every expert active
    cfg = dict(S=8192, H=7168, Hf=2048, E=384, K=8, dtype="bf16")
    counts = [8192 * 8 // 384] * 384
    R = 8192 * 8
    up_f, up_b = bench.kernel_model("ffn_up", cfg, counts)
    assert up_f == 4 * R * 7168 * 2048                      # 3.85 TFLOP
    wb = 384 * 7168 * 2048 * 2                               # one projection's bf16 weights
    assert up_b == 2 * wb + R * 7168 * 2 + 3 * R * 2048 * 2
    dw_f, dw_b = bench.kernel_model("bwd_dW13", cfg, counts)
    assert dw_f == up_f and dw_b == 2 * 384 * 7168 * 2048 * 4 + R * 7168 * 2 + 2 * R * 2048 * 2
    # dispatch moves each token once in and K times out
    _, disp_b = bench.kernel_model("dispatch_scatter", cfg, counts)
    assert disp_b == 8192 * 7168 * 2 + R * 7168 * 2 + 4 * 8192 * 8 + 8 * R
    # inactive experts' weights are not counted
    counts2 = [R // 192] * 192 + [0] * 192
    _, up_b2 = bench.kernel_model("ffn_up", cfg, counts2)
    assert up_b - up_b2 == 2 * 192 * 7168 * 2048 * 2


def test_roofline_entry_picks_the_binding_peak():
    cfg = dict(S=8192, H=4096, Hf=14336, E=8, K=2, dtype="bf16")
    counts = [2048] * 8
    # an MFMA-bound product and an HBM-bound copy-like kernel
    up = bench.roofline_entry("ffn_up", cfg, counts, 3.6e-3, True)
    assert up["bound"] == "mfma" and up["unit"] == "TFLOP/s" and 0 < up["frac"] < 1
    comb = bench.roofline_entry("combine", cfg, counts, 40e-6, True)
    assert comb["bound"] == "hbm" and comb["unit"] == "GB/s" and 0 < comb["frac"] < 1


def test_whole_call_models_at_the_384_expert_shape():
    # what each C-ABI call as a whole must move (its set-up kernels add no
    # algorithmic bytes)
    cfg = dict(S=8192, H=7168, Hf=2048, E=384, K=8, dtype="bf16")
    counts = [8192 * 8 // 384] * 384
    S, H, E, K, R = 8192, 7168, 384, 8, 8192 * 8
    _, disp = bench.kernel_model("call:moe_dispatch", cfg, counts)
    assert disp == 4 * S * K + S * H * 2 + R * H * 2 + 8 * R + 4 * (E + 1)
    assert abs(disp / 8e12 * 1e6 - 132.2) < 0.5          # about 132 us at 8 TB/s
    _, comb = bench.kernel_model("call:moe_combine", cfg, counts)
    assert comb == R * H * 2 + S * H * 2 + 8 * S * K
    f, rb = bench.kernel_model("call:moe_route", cfg, counts)
    assert f == 2 * S * H * E and rb == S * H * 2 + H * E * 2 + 4 * S * E + 8 * S * K + 4 * E
    # route at this shape is MFMA-bound by its algorithmic figures (on the ridge)
    assert bench.roofline_entry("call:moe_route", cfg, counts, 100e-6, True)["bound"] == "mfma"


def test_median():
    assert bench.median([3.0, 1.0, 2.0]) == 2.0
    assert bench.median([4.0, 1.0, 3.0, 2.0]) == 2.5
    assert bench.median([]) is None
