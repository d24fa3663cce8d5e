"""Seeded input recipes for the five MoE-layer workloads.

Every tensor is drawn from its own NumPy ``SeedSequence([seed, tensor_id,
sub])`` stream, so each one (and each expert's slice of a weight tensor) can
be regenerated on its own.  bf16 tensors are produced by rounding float32
draws to bf16 with round-to-nearest-even; they are carried on the host as the
float32 values they represent (exact) plus their 16-bit patterns for upload.

The expert weights of the large shapes (up to 34 GB of bf16) are generated on
the GPU with torch's device generator, one expert at a time
(``device_expert_weights``); a checker that needs an expert's weights copies
that slice back from the device.

Shapes and distributions follow the workloads on the pages: the Mixtral-like
8-expert layer at batch 4 x seq 2048 (MoE/MoD framework page, "How it looks in
practice"), the MoonEP benchmark defaults S=8192, E=384, H=7168, K=8, H'=2048
with a load skew swept over maxvio 0.2/1/10/20 (MoonEP page, step-by-step
guide, benchmark step), a fine-grained 64-expert layer with a Zipf-skewed
router, and a Mixture-of-Depths block keeping half of each sequence.
"""
from __future__ import annotations

import dataclasses
import json
import os
from typing import Dict, Optional

import numpy as np

# tensor ids for the per-tensor seed streams
T_X, T_WG, T_W1, T_W3, T_W2, T_DOUT, T_PERM, T_WR = 1, 2, 3, 4, 5, 6, 7, 8

CONFIGS: Dict[str, dict] = {
    # tiny fp32 layer; x and all weights ~N(0, 0.02^2)
    "c1": dict(workload="tiny-fp32", S=64, H=128, Hf=256, E=8, K=2, dtype="f32",
               seed=0, x_std=0.02, w_std=0.02, bias="none"),
    # Mixtral-style: batch 4 x seq 2048, 8 experts, top-2, bf16
    "c2": dict(workload="mixtral-8x-top2-bf16", S=8192, H=4096, Hf=14336, E=8, K=2,
               dtype="bf16", seed=1, x_std=1.0, w_std=0.02, bias="none"),
    # fine-grained, router biased per expert by a Zipf(1.1) log-pmf
    "c3": dict(workload="finegrained-64x-top4-zipf-bf16", S=8192, H=2048, Hf=1408, E=64,
               K=4, dtype="bf16", seed=2, x_std=1.0, w_std=0.02, bias="zipf", zipf_s=1.1),
    # MoonEP benchmark shape, one GPU's share with all 384 experts resident
    "c4": dict(workload="moonep-384x-top8-bf16", S=8192, H=7168, Hf=2048, E=384, K=8,
               dtype="bf16", seed=3, x_std=1.0, w_std=0.02, bias="maxvio"),
    # Mixture-of-Depths (keep 1024 of 2048 per sequence) + 16-expert top-2 MoE
    "c5": dict(workload="mod50-moe-16x-top2-bf16", S=4096, B=4, T=2048, C=1024, H=4096,
               Hf=5632, E=16, K=2, dtype="bf16", seed=4, x_std=1.0, w_std=0.02,
               bias="none"),
    # inference (decode) shape of the MoonEP layer: 128 tokens, about 2.7 rows
    # per expert, forward only; the grouped GEMMs stream the expert weights
    "c6": dict(workload="moonep-384x-top8-decode128-bf16", S=128, H=7168, Hf=2048, E=384, K=8,
               dtype="bf16", seed=5, x_std=1.0, w_std=0.02, bias="none", forward_only=True),
}


def _rng(seed: int, tid: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tid), int(sub)]))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return the uint16 patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = u + (((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """The exact float32 value of each bf16 pattern."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array whose values are the bf16 roundings of ``a``."""
    return bf16_bits_to_f32(bf16_bits(a))


def _normal(seed, tid, sub, shape, std, dtype) -> np.ndarray:
    v = _rng(seed, tid, sub).standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return round_bf16(v) if dtype == "bf16" else v


def zipf_bias(E: int, s: float, seed: int) -> np.ndarray:
    """Per-expert router bias -s*ln(1+pi(e)), pi a seeded permutation of the experts.

    Up to a constant this is the log of a Zipf(s) probability mass placed on
    the experts in a random order, which makes a few experts hot.
    """
    perm = _rng(seed, T_PERM).permutation(E)
    return (-float(s) * np.log1p(perm.astype(np.float64))).astype(np.float32)


@dataclasses.dataclass
class Workload:
    """Host-side tensors of one seeded workload (float32 arrays holding exact values)."""
    cfg: dict
    S: int
    H: int
    Hf: int
    E: int
    K: int
    dtype: str            # "f32" or "bf16": storage type of activations and weights
    x: np.ndarray         # [S_in, H]  (S_in = B*T for the MoD config, else S)
    Wg: np.ndarray        # [H, E]
    bias: Optional[np.ndarray]  # [E] float32 or None
    dout: np.ndarray      # [S_in, H]  upstream gradient of the layer output
    W1: Optional[np.ndarray] = None  # [E, H, Hf]  (host-generated configs only)
    W3: Optional[np.ndarray] = None  # [E, H, Hf]
    W2: Optional[np.ndarray] = None  # [E, Hf, H]
    w_r: Optional[np.ndarray] = None  # [H]  MoD scoring vector
    beta: float = 0.0

    @property
    def S_in(self) -> int:
        return self.x.shape[0]


def host_expert_weights(cfg: dict, e: int, dtype: Optional[str] = None, H=None, Hf=None):
    """Expert e's (W1[e], W3[e], W2[e]) drawn on the host from its own seed stream."""
    H = cfg["H"] if H is None else H
    Hf = cfg["Hf"] if Hf is None else Hf
    dt = cfg["dtype"] if dtype is None else dtype
    s = cfg["seed"]
    return (_normal(s, T_W1, e, (H, Hf), cfg["w_std"], dt),
            _normal(s, T_W3, e, (H, Hf), cfg["w_std"], dt),
            _normal(s, T_W2, e, (Hf, H), cfg["w_std"], dt))


def device_expert_weights(cfg: dict, device, E=None, H=None, Hf=None):
    """Allocate and fill W1, W3 [E,H,Hf] and W2 [E,Hf,H] on a torch device.

    Each expert's slice comes from its own torch generator seeded from
    (seed, tensor id, expert), filled in float32 chunks and rounded to bf16
    (torch's conversion rounds to nearest even), so the host never holds the
    whole tensor.
    """
    import torch
    E = cfg["E"] if E is None else E
    H = cfg["H"] if H is None else H
    Hf = cfg["Hf"] if Hf is None else Hf
    tdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    out = []
    for tid, shape in ((T_W1, (H, Hf)), (T_W3, (H, Hf)), (T_W2, (Hf, H))):
        w = torch.empty((E,) + shape, dtype=tdt, device=device)
        g = torch.Generator(device=device)
        for e in range(E):
            g.manual_seed(int(cfg["seed"]) * 1_000_003 + tid * 10_007 + e)
            tmp = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            tmp.mul_(float(cfg["w_std"]))
            w[e].copy_(tmp)
            del tmp
        out.append(w)
    return tuple(out)


_BETA_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "maxvio_beta.json")


def maxvio_beta(target: float) -> float:
    """Router-bias strength beta that gives the MoonEP-shape workload the target maxvio.

    The table is written offline by the oracle's calibration script; a level
    missing from it falls back to beta = 0 (the unbiased, balanced case).
    """
    if not os.path.exists(_BETA_FILE):
        return 0.0
    with open(_BETA_FILE) as f:
        table = json.load(f)
    return float(table.get("beta", {}).get(f"{float(target):g}", 0.0))


def maxvio_bias(target: float) -> Optional[np.ndarray]:
    """Stored per-expert balancing bias for a level below the unbiased router's skew, if any."""
    if not os.path.exists(_BETA_FILE):
        return None
    with open(_BETA_FILE) as f:
        table = json.load(f)
    vec = table.get("bias", {}).get(f"{float(target):g}")
    return None if vec is None else np.asarray(vec, dtype=np.float32)


def router_bias(cfg: dict, *, maxvio: Optional[float] = None, beta: Optional[float] = None):
    """(bias [E] float32 or None, beta) of a workload's router at a load-skew level.

    "zipf": the fixed Zipf(s) skew; "maxvio": the stored balancing bias for a
    level below the unbiased router's own skew, else -beta*ln(1+pi(e)) with
    beta from the stored table (beta = 0, the balanced case, when no level is
    asked for); "none": no bias.
    """
    E, seed = cfg["E"], cfg["seed"]
    if cfg["bias"] == "zipf":
        return zipf_bias(E, cfg["zipf_s"], seed), 0.0
    if cfg["bias"] != "maxvio":
        return None, 0.0
    if beta is None and maxvio is not None and maxvio_bias(maxvio) is not None:
        bias = maxvio_bias(maxvio)
        if bias.shape[0] != E:
            raise ValueError("stored balancing bias does not match E")
        return bias, 0.0
    if beta is None:
        beta = maxvio_beta(maxvio) if maxvio is not None else 0.0
    b = float(beta)
    return (zipf_bias(E, b, seed) if b != 0.0 else np.zeros(E, np.float32)), b


def make_workload(name: str, *, S: Optional[int] = None, beta: Optional[float] = None,
                  maxvio: Optional[float] = None, host_weights: Optional[bool] = None,
                  H: Optional[int] = None, Hf: Optional[int] = None,
                  E: Optional[int] = None, K: Optional[int] = None) -> Workload:
    """Build the seeded host tensors of a named workload.

    ``S``, ``H``, ``Hf``, ``E``, ``K`` override the table (for reduced-size
    parity cases with the same distributions).  Expert weights are generated on
    the host when ``host_weights`` is true (default: when they total at most
    64 M elements); otherwise the caller draws them on the device with
    ``device_expert_weights``.
    """
    cfg = dict(CONFIGS[name])
    for k, v in (("H", H), ("Hf", Hf), ("E", E), ("K", K)):
        if v is not None:
            cfg[k] = int(v)
    seed, dt = cfg["seed"], cfg["dtype"]
    Hd, Hfd, Ed, Kd = cfg["H"], cfg["Hf"], cfg["E"], cfg["K"]
    mod = "B" in cfg
    if S is not None:
        if mod:
            # keep the per-sequence structure: S_in = B*T with C = T/2 kept
            T = int(S) // cfg["B"]
            cfg["T"], cfg["C"] = T, T // 2
        cfg["S"] = int(S) if not mod else cfg["B"] * cfg["C"]
    S_in = cfg["B"] * cfg["T"] if mod else cfg["S"]

    x = _normal(seed, T_X, 0, (S_in, Hd), cfg["x_std"], dt)
    Wg = _normal(seed, T_WG, 0, (Hd, Ed), cfg["w_std"], dt)
    dout = _normal(seed, T_DOUT, 0, (S_in, Hd), 1.0, dt)

    bias, b = router_bias(cfg, maxvio=maxvio, beta=beta)
    w_r = _normal(seed, T_WR, 0, (Hd,), cfg["w_std"], dt) if mod else None

    wl = Workload(cfg=cfg, S=cfg["S"], H=Hd, Hf=Hfd, E=Ed, K=Kd, dtype=dt, x=x, Wg=Wg,
                  bias=bias, dout=dout, w_r=w_r, beta=b)
    if host_weights is None:
        host_weights = 3 * Ed * Hd * Hfd <= 64 * 1024 * 1024
    if host_weights:
        ws = [host_expert_weights(cfg, e) for e in range(Ed)]
        wl.W1 = np.stack([w[0] for w in ws])
        wl.W3 = np.stack([w[1] for w in ws])
        wl.W2 = np.stack([w[2] for w in ws])
    return wl
