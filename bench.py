"""MoE layer forward+backward throughput on one MI355X, with per-kernel roofline.

One step = route -> dispatch -> grouped SwiGLU FFN (up, down) -> combine ->
full backward (combine/gate backward, dA, dW2, dxd, dW1/dW3, dispatch and
router backward) on one batch of synthetic tokens already resident in HBM.
Prints ONE JSON line.  Default workload: the Mixtral-style layer
(batch 4 x seq 2048 = 8192 tokens, H=4096, H'=14336, E=8, K=2, bf16).  The
decode-shape workload (--config c6: 128 tokens of the 384-expert layer) is
timed forward only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/sec fwd+bwd; grouped-GEMM % MFMA peak; dispatch % HBM BW"
METRIC_FWD = "MoE layer tokens/sec fwd (decode shape); grouped-GEMM % HBM BW"
PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # FLOP/s dense bf16 MFMA
PEAK_F32_VALU = 157.3e12   # FLOP/s fp32 vector


def kernel_model(name, cfg, counts):
    """Algorithmic (FLOPs, bytes) of one launch of a kernel at this workload."""
    S, H, Hf, E, K = cfg["S"], cfg["H"], cfg["Hf"], cfg["E"], cfg["K"]
    b = 2 if cfg["dtype"] == "bf16" else 4
    R = S * K
    active = sum(1 for c in counts if c > 0)
    Wb = active * H * Hf * b          # one projection's weights of the active experts
    Gb = E * H * Hf * 4               # one projection's fp32 gradient
    m = {
        "route": (2 * S * H * E, S * H * b + H * E * b + 4 * S * E + 8 * S * K),
        "dispatch_scatter": (0, S * H * b + R * H * b + 4 * S * K + 8 * R),
        "ffn_up": (4 * R * H * Hf, 2 * Wb + R * H * b + 3 * R * Hf * b),
        "ffn_down": (2 * R * Hf * H, Wb + R * Hf * b + R * H * b),
        "combine": (2 * R * H, R * H * b + S * H * b + 8 * S * K),
        "combine_bwd": (4 * R * H, S * H * b + 2 * R * H * b + 4 * S * E + 12 * S * K),
        "bwd_dA": (2 * R * Hf * H, Wb + R * H * b + 4 * R * Hf * b),
        "bwd_dW2": (2 * R * Hf * H, Gb + R * H * b + R * Hf * b),
        "bwd_dxd": (4 * R * H * Hf, 2 * Wb + 2 * R * Hf * b + R * H * b),
        "bwd_dW13": (4 * R * H * Hf, 2 * Gb + R * H * b + 2 * R * Hf * b),
        # the K router-weight rows each token gathers come from the small
        # cached [E, H] table: counted once
        "dispatch_bwd_dx": (2 * R * H, R * H * b + S * H * b + E * H * b + 8 * S * K),
        "router_dWg_partial": (2 * R * H, R * H * b + 4 * R),
    }
    if cfg.get("raw"):
        # raw softmax gates: dense dlogits, router terms over all E experts
        m["combine_bwd"] = (4 * R * H + 8 * S * E, S * H * b + 2 * R * H * b + 8 * S * E + 4 * S * K)
        m["dispatch_bwd_dx"] = (2 * S * H * E + R * H, R * H * b + S * H * b + E * H * b + 4 * S * E)
        m["router_dWg_partial"] = (2 * S * H * E, S * H * b + 4 * S * E)
    return m.get(name)


def roofline_entry(name, cfg, counts, avg_s, bf16):
    fb = kernel_model(name, cfg, counts)
    if fb is None or avg_s <= 0:
        return None
    flops, byts = fb
    peak_f = PEAK_BF16 if bf16 else PEAK_F32_VALU
    t_f, t_b = flops / peak_f, byts / PEAK_HBM
    if t_f >= t_b:
        return {"bound": "mfma" if bf16 else "alu", "achieved": flops / avg_s / 1e12,
                "peak": peak_f / 1e12, "unit": "TFLOP/s", "frac": (flops / avg_s) / peak_f,
                "flops": flops, "bytes": byts}
    return {"bound": "hbm", "achieved": byts / avg_s / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": (byts / avg_s) / PEAK_HBM, "flops": flops, "bytes": byts}


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "routing_dispatch_grouped_moe_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    ent = tab.get(f"{kernel}@{workload}")
    if not ent or ent.get("source_hash") != source_hash(ent.get("sources", [])):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(name, maxvio, sample_tokens, forward_only=False):
    """Time the float64 oracle (as it stands) on a bounded token sample of the same workload."""
    import numpy as np
    import oracle
    from synth import make_workload, CONFIGS
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    cfg = CONFIGS[name]
    wl = make_workload(name, maxvio=maxvio, host_weights=False)
    S = min(sample_tokens, wl.S_in)
    x, dout = wl.x[:S], wl.dout[:S]
    E, H, Hf = wl.E, wl.H, wl.Hf
    from synth import host_expert_weights
    cache = {}

    def w(kind):
        def get(e):
            if e not in cache:
                cache[e] = host_expert_weights(wl.cfg, e)
            return cache[e][kind]
        return get

    W1, W3, W2 = w(0), w(1), w(2)
    # the weights of the experts this sample touches are drawn before timing
    logits = oracle.router_logits(x, wl.Wg, wl.bias)
    for e in np.unique(oracle.topk_experts(logits, wl.K)):
        W1(int(e))  # draws all three of expert e's matrices
    t0 = time.perf_counter()
    fw = oracle.moe_forward(x, wl.Wg, wl.bias, W1, W3, W2, wl.K)
    if not forward_only:
        oracle.moe_backward(fw, dout, x, wl.Wg, W1, W3, W2, wl.K,
                            on_dW=lambda e, g1, g3, g2: None)
    t = time.perf_counter() - t0
    del fw
    what = "forward" if forward_only else "forward+backward incl. weight gradients"
    return {"value": S / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} of the {wl.S_in} tokens of {cfg['workload']} (E={E}, H={H}, "
                      f"H'={Hf}), host-drawn weights of the same distribution, float64 "
                      f"{what}, {t:.1f} s",
            "cpu_model": cpu_model()}


def cpu_model():
    """CPU model name of the host, from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5", "c6"])
    ap.add_argument("--maxvio", type=float, default=None, help="c4 load skew level")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None)
    ap.add_argument("--kernels", action="store_true", help="also print the per-kernel table")
    ap.add_argument("--gates", default="renorm", choices=["renorm", "raw"],
                    help="gates renormalised over the K chosen experts (default) or raw softmax")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in one HIP graph (graph_ms_per_step)")
    ap.add_argument("--recompute", action="store_true",
                    help="keep no h1/h3 between forward and backward (the backward recomputes them)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 512 MiB device-to-device copy first (a known-size kernel for "
                         "scaling HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the multi-GPU expert-"
              f"parallel path is not implemented", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from synth import make_workload, device_expert_weights
    from routing_dispatch_grouped_moe_amd import MoELayer, MoDMoELayer
    from routing_dispatch_grouped_moe_amd import _lib as L

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = make_workload(args.config, maxvio=args.maxvio, host_weights=False)
    cfg = wl.cfg
    bf16 = wl.dtype == "bf16"
    fwd_only = bool(cfg.get("forward_only"))

    def up(a):
        from synth import bf16_bits
        a = np.ascontiguousarray(a, np.float32)
        if bf16:
            return torch.from_numpy(bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x, Wg, dout = up(wl.x), up(wl.Wg), up(wl.dout)
    bias = None if wl.bias is None else torch.from_numpy(wl.bias).to(dev)
    W1, W3, W2 = device_expert_weights(cfg, dev)
    mod = "B" in cfg
    flags = (L.MOE_F_RENORM if args.gates == "renorm" else 0) | \
        (L.MOE_F_RECOMPUTE if args.recompute else 0)
    if mod:
        w_r = up(wl.w_r)
        layer = MoDMoELayer(cfg["B"], cfg["T"], cfg["C"], wl.H, wl.Hf, wl.E, wl.K, wl.dtype, dev,
                            flags=flags)
        moe = layer.moe

        def step():
            layer.forward(x, w_r, Wg, bias, W1, W3, W2)
            layer.backward(dout, x, w_r, Wg, W1, W3, W2)
    else:
        layer = MoELayer(wl.S, wl.H, wl.Hf, wl.E, wl.K, wl.dtype, dev, flags=flags)
        moe = layer

        def step():
            layer.forward(x, Wg, bias, W1, W3, W2)
            if not fwd_only:
                layer.backward(dout, x, Wg, W1, W3, W2)

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # one elementwise kernel: 512 MiB read, 512 MiB written
        torch.cuda.synchronize()
        say("calibration kernel (neg): 512 MiB read + 512 MiB written")
        del src, dst
    say(f"{cfg['workload']}: inputs resident; warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    say(f"timing {args.steps} steps")
    L.moe_timer_reset()
    L.moe_timer_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    L.moe_timer_enable(False)
    ktab = L.moe_timer_read()
    L.moe_timer_reset()

    graph_ms = None
    if args.graph:
        # the same step captured once in a HIP graph, replayed K times
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        say(f"timing {args.steps} graph replays")
        tg0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - tg0) / args.steps * 1e3
        del g

    S_in = wl.S_in
    elapsed = t1 - t0
    ms_per_step = elapsed / args.steps * 1e3
    counts = moe.counts.cpu().numpy().tolist()
    # load statistics of the routing histogram, from the library
    stats = torch.empty(2, dtype=torch.float32, device=dev)
    L.moe_load_stats(wl.E, moe.counts, stats)
    maxvio, load_entropy = (float(v) for v in stats.cpu().numpy())
    mcfg = dict(S=moe.S, H=wl.H, Hf=wl.Hf, E=wl.E, K=wl.K, dtype=wl.dtype,
                raw=args.gates == "raw")

    kernels = {}
    for name, (ms, n) in sorted(ktab.items(), key=lambda kv: -kv[1][0]):
        avg = ms / 1e3 / max(n, 1)
        ent = {"avg_us": avg * 1e6, "launches": n, "total_ms_per_step": ms / args.steps}
        rl = roofline_entry(name, mcfg, counts, avg, bf16)
        if rl:
            ent.update({"bound": rl["bound"], "frac": rl["frac"], "achieved": rl["achieved"],
                        "unit": rl["unit"], "flops": rl["flops"], "bytes": rl["bytes"]})
        kernels[name] = ent
    dom = max(kernels, key=lambda k: kernels[k]["total_ms_per_step"])
    dom_avg = kernels[dom]["avg_us"] / 1e6
    rl = roofline_entry(dom, mcfg, counts, dom_avg, bf16) or {}
    roof = {"kernel": dom, "bound": rl.get("bound"), "achieved": rl.get("achieved"),
            "peak": rl.get("peak"), "unit": rl.get("unit"), "frac": rl.get("frac"),
            "traffic": measured_traffic(dom, cfg["workload"]),
            "algorithmic_flops": rl.get("flops"), "algorithmic_bytes": rl.get("bytes")}

    gemm_names = ["ffn_up", "ffn_down", "bwd_dA", "bwd_dW2", "bwd_dxd", "bwd_dW13"]
    gflops = sum(kernel_model(n, mcfg, counts)[0] for n in gemm_names if n in kernels)
    gtime = sum(kernels[n]["avg_us"] * 1e-6 * kernels[n]["launches"] / args.steps
                for n in gemm_names if n in kernels)
    disp = kernels.get("dispatch_scatter", {})

    # device memory the layer holds: all its buffers, and the part the
    # forward leaves for the backward (inputs excluded)
    def nbytes(t):
        return 0 if t is None else t.numel() * t.element_size()
    kept = sum(nbytes(getattr(moe, n, None)) for n in
               ("logits", "topk_idx", "gates", "cu", "row_of", "tok_of", "xd", "h1", "h3", "a", "y"))
    held = sum(nbytes(v) for v in vars(moe).values() if isinstance(v, torch.Tensor))
    out = {
        "metric": METRIC_FWD if fwd_only else METRIC,
        "value": S_in * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded; random-init weights of the named shape)",
        "config": {"workload": cfg["workload"], "tokens": S_in, "moe_tokens": moe.S, "H": wl.H,
                   "H_ffn": wl.Hf, "experts": wl.E, "top_k": wl.K, "router_bias_beta": wl.beta,
                   "maxvio_measured": maxvio, "load_entropy": load_entropy,
                   "parallelism": "single GPU, all experts resident",
                   "step": "forward" if fwd_only else "forward+backward",
                   "gates": "softmax renormalised over the top-K" if args.gates == "renorm"
                   else "raw softmax (no renormalisation)",
                   "activations": "h1, h3 recomputed in the backward" if args.recompute
                   else "h1, h3 saved"},
        "graph_ms_per_step": graph_ms,
        "graph_tokens_per_s": (S_in / (graph_ms / 1e3)) if graph_ms else None,
        "memory": {"layer_buffers_gb": held / 1e9, "kept_forward_to_backward_gb": kept / 1e9,
                   "peak_allocated_gb": torch.cuda.max_memory_allocated(dev) / 1e9},
        "roofline": roof,
        "grouped_gemm_mfma_frac": (gflops / gtime) / PEAK_BF16 if gtime > 0 else None,
        "grouped_gemm_hbm_frac": (
            sum(kernel_model(n, mcfg, counts)[1] for n in gemm_names if n in kernels) / gtime
            / PEAK_HBM if gtime > 0 else None),
        "dispatch_hbm_frac": disp.get("frac") if disp.get("bound") == "hbm" else None,
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in kernels.items()},
        "kernels_frac": {k: round(v["frac"], 4) for k, v in kernels.items() if "frac" in v},
        # both fractions of every modelled kernel: algorithmic FLOPs against the
        # bf16 MFMA peak and algorithmic bytes against the HBM peak
        "kernels_mfma_hbm_frac": {
            k: [round(v["flops"] / (v["avg_us"] * 1e-6) / PEAK_BF16, 4),
                round(v["bytes"] / (v["avg_us"] * 1e-6) / PEAK_HBM, 4)]
            for k, v in kernels.items() if "flops" in v and v["avg_us"] > 0},
    }
    if not args.no_cpu_baseline:
        del x, Wg, dout, W1, W3, W2, layer, moe
        torch.cuda.empty_cache()
        default_sample = {"c1": 64, "c2": 4096, "c3": 1024, "c4": 16, "c5": 512,
                          "c6": 8}[args.config]
        say(f"GPU part done ({ms_per_step:.2f} ms/step); timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(args.config, args.maxvio,
                                           args.cpu_sample or default_sample, fwd_only)
    print(json.dumps(out), flush=True)
    if args.kernels:
        for k, v in kernels.items():
            print(f"  {k:24s} {v['avg_us']:10.1f} us x{v['launches'] // args.steps}"
                  f"  {v.get('bound', ''):5s} {100 * v.get('frac', 0):6.1f}%", file=sys.stderr)


if __name__ == "__main__":
    main()
