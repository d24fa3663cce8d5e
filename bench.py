"""MoE layer forward+backward throughput on one MI355X, with per-kernel roofline.

One step = route -> dispatch -> grouped SwiGLU FFN (up, down) -> combine ->
full backward (combine/gate backward, dA, dW2, dxd, dW1/dW3, dispatch and
router backward) on one batch of synthetic tokens already resident in HBM.
Prints ONE JSON line.

Default workload: the MoonEP-shaped single-GPU share (S=8192 tokens, E=384
experts all resident, H=7168, H'=2048, K=8, bf16; MoonEP page, step-by-step
guide, benchmark step), timed with the unbiased router (the balanced case),
then at the router skews of maxvio 0.2, 1, 10 and 20 in the same process
(MoonEP page, "Which problem MoonEP solves") with their ratio to the balanced
case.  --config c2 gives the Mixtral-style layer (batch 4 x seq 2048, E=8,
K=2, H=4096, H'=14336; MoE/MoD framework page, "How it looks in practice").
The decode-shape workload (--config c6: 128 tokens of the 384-expert layer)
is timed forward only.

Timing: W warm-up steps, then exactly K steps between two device
synchronisations (value = tokens / wall time), with a HIP event between
consecutive steps for the median.  Per-call durations come from a second
pass with HIP events around every C-ABI call, per-kernel durations from a
third with events around every kernel (the library's timer, recorded on the
launch stream), so the headline carries no instrumentation and the call
times none of the kernel timer's.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/sec fwd+bwd; grouped-GEMM % MFMA peak; dispatch % HBM BW"
METRIC_FWD = "MoE layer tokens/sec fwd (decode shape); grouped-GEMM % HBM BW"
PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # FLOP/s dense bf16 MFMA
PEAK_F32_VALU = 157.3e12   # FLOP/s fp32 vector
SKEW_LEVELS = (0.2, 1.0, 10.0, 20.0)  # maxvio levels of the MoonEP benchmark
GEMM_NAMES = ("ffn_up", "ffn_down", "bwd_dA", "bwd_dW2", "bwd_dxd", "bwd_dW13")


def kernel_model(name, cfg, counts):
    """Algorithmic (FLOPs, bytes) of one launch of a kernel (or one C-ABI call) at this workload."""
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
        # each row's values are read from x through tok_of: x counted once
        "router_dWg_partial": (2 * R * H, S * H * b + 8 * R),
        # whole C-ABI calls: what the call as a whole must move (its
        # set-up kernels -- counts fill, router-weight transpose, dispatch
        # bitmaps and scan -- add no algorithmic bytes)
        "call:moe_route": (2 * S * H * E, S * H * b + H * E * b + 4 * S * E + 8 * S * K + 4 * E),
        "call:moe_dispatch": (0, 4 * S * K + S * H * b + R * H * b + 8 * R + 4 * (E + 1)),
        "call:moe_combine": (2 * R * H, R * H * b + S * H * b + 8 * S * K),
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


def median(v):
    v = sorted(v)
    n = len(v)
    if n == 0:
        return None
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def cpu_info():
    """CPU model name (from /proc/cpuinfo) and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline(wl, sample, gpu_sample, forward_only=False):
    """Time the float64 oracle (as it stands) on a bounded token sample of the same workload,
    and compare the GPU's outputs for those tokens with it.

    gpu_sample holds the GPU run's routing and outputs for the first `sample`
    tokens and the device weights of every expert either side routes them to
    (copied to the host, so the oracle sees the GPU's exact inputs).
    """
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    S = min(sample, wl.S_in)
    x, dout = wl.x[:S], wl.dout[:S]
    wts = gpu_sample["weights"]
    W1, W3, W2 = (lambda e: wts[e][0]), (lambda e: wts[e][1]), (lambda e: wts[e][2])
    t0 = time.perf_counter()
    fw = oracle.moe_forward(x, wl.Wg, wl.bias, W1, W3, W2, wl.K)
    bw = None
    if not forward_only:
        bw = oracle.moe_backward(fw, dout, x, wl.Wg, W1, W3, W2, wl.K,
                                 on_dW=lambda e, g1, g3, g2: None)
    t = time.perf_counter() - t0
    model, ncores = cpu_info()
    what = "forward" if forward_only else "forward+backward incl. weight gradients"
    res = {"value": S / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"first {S} of the {wl.S_in} tokens of {wl.cfg['workload']} (E={wl.E}, "
                     f"H={wl.H}, H'={wl.Hf}), the GPU run's expert weights, float64 {what}, "
                     f"{t:.1f} s", "cpu_model": model, "host_cores": ncores}

    # parity of the GPU outputs on the sample (normwise max error per tensor,
    # over the tokens whose top-K both sides agree on)
    def normwise(got, want):
        got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
        den = np.abs(want).max() if want.size else 0.0
        num = np.abs(got - want).max() if want.size else 0.0
        return float(num / den) if den > 0 else float(num)

    g = gpu_sample
    if g.get("topk_idx") is None:
        res["parity"] = None  # the MoD block's sample is timed only
        return res
    same = np.all(fw["idx"] == g["topk_idx"], axis=1)
    par = {"tokens": int(S), "topk_mismatched_tokens": int((~same).sum()),
           "logits": normwise(g["logits"], fw["logits"]) if g.get("logits") is not None else None}
    if same.any():
        par["gates"] = normwise(g["gates"][same], fw["gates"][same])
        par["out"] = normwise(g["out"][same], fw["out"][same])
        if bw is not None and g.get("dx") is not None:
            par["dx"] = normwise(g["dx"][same], bw["dx"][same])
    par["bound"] = 2e-2 if wl.dtype == "bf16" else 1e-5
    par["metric"] = "normwise max error ||gpu - oracle||_inf / ||oracle||_inf per tensor"
    res["parity"] = par
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5", "c6"])
    ap.add_argument("--maxvio", type=float, default=None,
                    help="c4: time this load-skew level as the headline (default: unbiased)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="c4: skip the maxvio 0.2/1/10/20 legs")
    ap.add_argument("--kernel-steps", type=int, default=None,
                    help="steps of the instrumented per-kernel pass (default min(steps, 5))")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None)
    ap.add_argument("--kernels", action="store_true", help="also print the per-kernel table")
    ap.add_argument("--gates", default="renorm", choices=["renorm", "raw"],
                    help="gates renormalised over the K chosen experts (default) or raw softmax")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in one HIP graph (graph_ms_per_step)")
    ap.add_argument("--recompute", action="store_true",
                    help="keep no h1/h3 between forward and backward (the backward recomputes them)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="instead of the layer, time the vendor BLAS (torch.bmm, hipBLASLt) on the "
                         "workload's per-expert products at balanced load, for comparison")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 512 MiB read + 512 MiB write kernel first (a known-size kernel "
                         "for scaling HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the multi-GPU expert-"
              f"parallel path is not implemented", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from synth import make_workload, device_expert_weights, router_bias, bf16_bits
    from routing_dispatch_grouped_moe_amd import MoELayer, MoDMoELayer
    from routing_dispatch_grouped_moe_amd import _lib as L

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.library_gemm:
        library_gemm(args.config)
        return
    wl = make_workload(args.config, maxvio=args.maxvio, host_weights=False)
    cfg = wl.cfg
    bf16 = wl.dtype == "bf16"
    fwd_only = bool(cfg.get("forward_only"))
    sweep = cfg.get("bias") == "maxvio" and args.maxvio is None and not args.no_sweep

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    def up(a):
        a = np.ascontiguousarray(a, np.float32)
        if bf16:
            return torch.from_numpy(bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x, Wg, dout = up(wl.x), up(wl.Wg), up(wl.dout)
    bias = None if wl.bias is None else torch.from_numpy(wl.bias).to(dev)
    say(f"{cfg['workload']}: drawing expert weights on the device")
    W1, W3, W2 = device_expert_weights(cfg, dev)
    mod = "B" in cfg
    flags = (L.MOE_F_RENORM if args.gates == "renorm" else 0) | \
        (L.MOE_F_RECOMPUTE if args.recompute else 0)
    if mod:
        w_r = up(wl.w_r)
        layer = MoDMoELayer(cfg["B"], cfg["T"], cfg["C"], wl.H, wl.Hf, wl.E, wl.K, wl.dtype, dev,
                            flags=flags)
        moe = layer.moe
    else:
        layer = MoELayer(wl.S, wl.H, wl.Hf, wl.E, wl.K, wl.dtype, dev, flags=flags)
        moe = layer
    cur_bias = [bias]

    # the step as its C-ABI calls, in order (name, callable)
    def calls():
        b = cur_bias[0]
        if mod:
            B, T, Cn, H, dt = layer.B, layer.T, layer.C, layer.H, layer.dt
            xk = layer.xk
            c = [("moe_mod_select", lambda: L.moe_mod_select(B, T, Cn, H, dt, x, w_r, layer.r,
                                                             layer.keep, xk))]
            xin = xk
        else:
            c, xin = [], x
        c += [("moe_route", lambda: moe.route(xin, Wg, b)),
              ("moe_dispatch", lambda: moe.dispatch(xin)),
              ("moe_ffn_up", lambda: L.moe_ffn_up(moe.d, moe.xd, moe.cu, W1, W3, moe.h1, moe.h3,
                                                  moe.a, moe.ws)),
              ("moe_ffn_down", lambda: L.moe_ffn_down(moe.d, moe.a, moe.cu, W2, moe.y, moe.ws)),
              ("moe_combine", lambda: moe.combine())]
        if mod:
            c += [("moe_mod_merge", lambda: L.moe_mod_merge(B, T, Cn, H, dt, x, layer.r, layer.keep,
                                                            moe.out, layer.out))]
        if fwd_only:
            return c
        if mod:
            c += [("moe_mod_backward", lambda: L.moe_mod_backward(
                      B, T, Cn, H, dt, layer.flags, x, w_r, layer.r, layer.keep, moe.out, dout,
                      None, layer.dm, layer.dr, None, None, None)),
                  ("moe_backward", lambda: moe.backward(layer.dm, xk, Wg, W1, W3, W2)),
                  ("moe_mod_backward", lambda: L.moe_mod_backward(
                      B, T, Cn, H, dt, layer.flags, x, w_r, layer.r, layer.keep, moe.out, dout,
                      moe.dx, layer.dm, layer.dr, layer.dx, layer.dw_r, layer.mws))]
        else:
            c += [("moe_backward", lambda: moe.backward(dout, x, Wg, W1, W3, W2))]
        return c

    def step():
        for _, f in calls():
            f()

    def timed_steps(n):
        """n steps between two synchronisations; (wall seconds, per-step ms list)."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(n):
            step()
            ev[i + 1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return t1 - t0, [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]

    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # one elementwise kernel: 512 MiB read, 512 MiB written
        torch.cuda.synchronize()
        say("calibration kernel (neg): 512 MiB read + 512 MiB written")
        del src, dst

    # ---- headline: K steps, no instrumentation
    say(f"{cfg['workload']}: inputs resident; warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    say(f"timing {args.steps} steps")
    elapsed, step_ms = timed_steps(args.steps)
    ms_per_step = elapsed / args.steps * 1e3
    say(f"{ms_per_step:.3f} ms/step (median {median(step_ms):.3f})")

    # GPU outputs of the sample tokens (before any other routing overwrites them)
    S_in = wl.S_in
    counts = moe.counts.cpu().numpy().tolist()
    stats = torch.empty(2, dtype=torch.float32, device=dev)
    L.moe_load_stats(wl.E, moe.counts, stats)
    maxvio, load_entropy = (float(v) for v in stats.cpu().numpy())
    # about 10-30 s of oracle work on the host (16 threads)
    sample = args.cpu_sample or {"c1": 64, "c2": 4096, "c3": 1024, "c4": 24, "c5": 512,
                                 "c6": 24}[args.config]
    gpu_sample = None
    if not args.no_cpu_baseline and mod:
        gpu_sample = {}  # weights only: the MoD block's sample is timed, not compared
    elif not args.no_cpu_baseline:
        n = min(sample, S_in)
        f32 = lambda t: t.float().cpu().numpy()  # noqa: E731
        gpu_sample = {"topk_idx": moe.topk_idx[:n].cpu().numpy(), "gates": f32(moe.gates[:n]),
                      "logits": f32(moe.logits[:n]) if moe.logits is not None else None,
                      "out": f32(moe.out[:n]), "dx": None if fwd_only else f32(moe.dx[:n])}

    # ---- instrumented passes: the C-ABI calls between HIP events (nothing
    # else recorded), then every kernel between HIP events (library timer),
    # stepping on while amd-smi samples the clock
    ksteps = args.kernel_steps or min(args.steps, 5)
    say(f"instrumented passes: {ksteps} steps each")
    call_ev = {}
    torch.cuda.synchronize()
    for _ in range(ksteps):
        for name, f in calls():
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            call_ev.setdefault(name, []).append((a, b))
    torch.cuda.synchronize()
    calls_ms = {name: sum(a.elapsed_time(b) for a, b in evs) / ksteps
                for name, evs in call_ev.items()}
    clock = None
    try:
        sampler = subprocess.Popen(["amd-smi", "metric", "-g", "0", "-c", "--json"],
                                   stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except OSError:
        sampler = None
    L.moe_timer_reset()
    L.moe_timer_enable(True)
    t_busy = time.perf_counter()
    done_steps = 0
    while True:
        step()
        done_steps += 1
        if done_steps == ksteps:
            torch.cuda.synchronize()
            L.moe_timer_enable(False)
        if done_steps >= ksteps and (sampler is None or sampler.poll() is not None
                                     or time.perf_counter() - t_busy > 20):
            break
    torch.cuda.synchronize()
    L.moe_timer_enable(False)
    ktab = L.moe_timer_read()
    L.moe_timer_reset()
    if sampler is not None:
        try:
            out_s, _ = sampler.communicate(timeout=20)
            data = json.loads(out_s) if out_s else None
        except (subprocess.SubprocessError, ValueError):
            sampler.kill()
            data = None
        if data is not None:
            clock = parse_clock(data)

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

    # ---- load-skew legs (same weights and tokens, router bias for each level)
    skew = None
    if sweep:
        skew = []
        for lv in SKEW_LEVELS:
            bvec, beta = router_bias(cfg, maxvio=lv)
            cur_bias[0] = torch.from_numpy(bvec).to(dev)
            for _ in range(max(2, args.warmup // 2)):
                step()
            el, sm = timed_steps(args.steps)
            L.moe_load_stats(wl.E, moe.counts, stats)
            mv = float(stats.cpu().numpy()[0])
            ms = el / args.steps * 1e3
            skew.append({"maxvio_target": lv, "maxvio_measured": mv, "router_bias_beta": beta,
                         "ms_per_step": ms, "median_ms_per_step": median(sm),
                         "tokens_per_s": S_in * args.steps / el,
                         "vs_balanced": ms_per_step / ms})
            say(f"maxvio {lv:g} (measured {mv:.3f}): {ms:.3f} ms/step, "
                f"{ms_per_step / ms:.3f} of the balanced rate")
        cur_bias[0] = bias

    mcfg = dict(S=moe.S, H=wl.H, Hf=wl.Hf, E=wl.E, K=wl.K, dtype=wl.dtype,
                raw=args.gates == "raw")
    kernels = {}
    for name, (ms, n) in sorted(ktab.items(), key=lambda kv: -kv[1][0]):
        avg = ms / 1e3 / max(n, 1)
        ent = {"avg_us": avg * 1e6, "launches": n, "total_ms_per_step": ms / ksteps}
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
            "algorithmic_flops": rl.get("flops"), "algorithmic_bytes": rl.get("bytes"),
            "avg_us": dom_avg * 1e6}

    gflops = sum(kernel_model(n, mcfg, counts)[0] for n in GEMM_NAMES if n in kernels)
    gtime = sum(kernels[n]["total_ms_per_step"] * 1e-3 for n in GEMM_NAMES if n in kernels)
    # whole C-ABI calls against the bytes the call must move
    whole = {}
    for cname in ("moe_route", "moe_dispatch", "moe_combine"):
        if cname in calls_ms:
            r = roofline_entry("call:" + cname, mcfg, counts, calls_ms[cname] * 1e-3, bf16)
            whole[cname] = {"us": calls_ms[cname] * 1e3, "bound": r["bound"], "frac": r["frac"],
                            "achieved": r["achieved"], "unit": r["unit"]}

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
        "median_ms_per_step": median(step_ms),
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
        "maxvio_sweep": skew,
        "skew_penalty_at_maxvio20": (skew[-1]["vs_balanced"] if skew else None),
        "graph_ms_per_step": graph_ms,
        "graph_tokens_per_s": (S_in / (graph_ms / 1e3)) if graph_ms else None,
        "gpu_clock": clock,
        "memory": {"layer_buffers_gb": held / 1e9, "kept_forward_to_backward_gb": kept / 1e9,
                   "peak_allocated_gb": torch.cuda.max_memory_allocated(dev) / 1e9},
        "roofline": roof,
        "grouped_gemm_mfma_frac": (gflops / gtime) / PEAK_BF16 if gtime > 0 else None,
        "grouped_gemm_hbm_frac": (
            sum(kernel_model(n, mcfg, counts)[1] for n in GEMM_NAMES if n in kernels) / gtime
            / PEAK_HBM if gtime > 0 else None),
        "whole_call": whole,
        "dispatch_hbm_frac": whole.get("moe_dispatch", {}).get("frac"),
        "calls_us": {k: round(v * 1e3, 2) for k, v in calls_ms.items()},
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
        if gpu_sample is not None:
            # the device weights of every expert either side routes the sample to
            import oracle
            n = min(sample, S_in)
            lg = oracle.router_logits(wl.x[:n], wl.Wg, wl.bias)
            # (expert 0 too: the oracle reads its shape)
            ex = set(np.unique(oracle.topk_experts(lg, wl.K)).tolist()) | {0}
            if gpu_sample.get("topk_idx") is not None:
                ex |= set(np.unique(gpu_sample["topk_idx"]).tolist())
            gpu_sample["weights"] = {int(e): tuple(w[int(e)].float().cpu().numpy()
                                                   for w in (W1, W3, W2)) for e in sorted(ex)}
        del x, Wg, dout, W1, W3, W2, layer, moe
        torch.cuda.empty_cache()
        say(f"GPU part done ({ms_per_step:.2f} ms/step); timing the CPU oracle on a sample")
        if gpu_sample is not None:
            out["cpu_baseline"] = cpu_baseline(wl, sample, gpu_sample, fwd_only)
        else:
            out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    if args.kernels:
        for k, v in kernels.items():
            print(f"  {k:24s} {v['avg_us']:10.1f} us x{v['launches'] // ksteps}"
                  f"  {v.get('bound', ''):5s} {100 * v.get('frac', 0):6.1f}%", file=sys.stderr)
        for k, v in calls_ms.items():
            print(f"  call {k:19s} {v * 1e3:10.1f} us", file=sys.stderr)


def library_gemm(config):
    """Vendor BLAS (torch.bmm, i.e. hipBLASLt) on the workload's expert products.

    Every expert gets the balanced row count S*K/E; one projection each of
    the up and down products and the weight-gradient shape (bf16 output,
    where the layer writes fp32).  Contiguous operands only.  Prints one
    JSON line; a comparison point, not part of the layer.
    """
    import torch
    from synth import CONFIGS
    cfg = CONFIGS[config]
    if cfg.get("dtype") != "bf16":
        print(json.dumps({"library_gemm": None, "reason": "bf16 workloads only"}))
        return
    S, E, K, H, Hf = cfg["S"], cfg["E"], cfg["K"], cfg["H"], cfg["Hf"]
    r = max(1, S * K // E)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    bf = torch.bfloat16

    def rnd(*shape):
        return (torch.randn(*shape, device=dev, generator=g) * 0.05).to(bf)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    res = {}
    flops = 2 * E * r * H * Hf
    for name, (ashape, bshape, oshape) in {
            "up_one_projection": ((E, r, H), (E, H, Hf), (E, r, Hf)),
            "down": ((E, r, Hf), (E, Hf, H), (E, r, H)),
            "weight_grad_shape_bf16_out": ((E, H, r), (E, r, Hf), (E, H, Hf))}.items():
        A, B = rnd(*ashape), rnd(*bshape)
        us = timed(lambda: torch.bmm(A, B), 10)
        byts = 2 * (A.numel() + B.numel() + oshape[0] * oshape[1] * oshape[2])
        res[name] = {"shape": f"bmm {list(ashape)} x {list(bshape)}", "us": round(us, 1),
                     "tflops": round(flops / us / 1e6, 1), "mfma_frac": round(flops / us / 1e6 / 2500, 3),
                     "gb": round(byts / 1e9, 3), "tbs": round(byts / us / 1e6, 2)}
        del A, B
        torch.cuda.empty_cache()
    print(json.dumps({"library_gemm": res, "workload": cfg["workload"], "rows_per_expert": r}),
          flush=True)


def parse_clock(data):
    """Graphics / memory clocks (MHz) from amd-smi's JSON (any nesting of {"clk": {"value"}}).

    Sampled while the instrumented pass keeps the GPU busy, so a throttled
    clock shows (T4 tuning page, checklist before optimising: rule out
    throttling first).
    """
    gfx, mem = [], []

    def walk(o, key=""):
        if isinstance(o, dict):
            for k, v in o.items():
                kk = f"{key}/{k}"
                if k == "clk" and isinstance(v, dict) and isinstance(v.get("value"), (int, float)):
                    if "gfx" in key.lower():
                        gfx.append(float(v["value"]))
                    elif "mem" in key.lower():
                        mem.append(float(v["value"]))
                else:
                    walk(v, kk)
        elif isinstance(o, list):
            for v in o:
                walk(v, key)

    walk(data)
    if not gfx and not mem:
        return {"raw": json.dumps(data)[:300]}
    return {"gfx_mhz_mean": sum(gfx) / len(gfx) if gfx else None,
            "gfx_mhz_min": min(gfx) if gfx else None,
            "mem_mhz": max(mem) if mem else None,
            "source": "amd-smi metric -c, sampled during the instrumented pass"}


if __name__ == "__main__":
    main()
