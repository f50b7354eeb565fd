"""Seeded synthetic inputs for the W8A8 FP8 MoE layer.

This module only draws random numbers; it holds none of the layer's
arithmetic (no quantisation, routing or expert math).  Both the GPU path and
the CPU oracle receive the tensors it returns.

Every tensor gets its own generator, seeded from (seed, tensor name, expert)
through CRC32, so one tensor can be regenerated without the others.  The
routing inputs (x, W_r, bias, per-token k) are always drawn on the CPU so
that routing is identical whichever device holds the expert weights; the
expert weights are drawn on the device that will use them.

Value distributions (the layer's workload statement): x ~ N(0, 1);
W_r ~ N(0, 1/d); W_gate, W_up ~ N(0, 1/d); W_down ~ N(0, 1/f); all fp32.
"""
from __future__ import annotations

import json
import math
import os
import zlib
from dataclasses import dataclass, field, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int                      # k_max: slots per token
    n_shared: int = 0           # always-on shared experts
    k_choices: tuple = ()       # elastic k: per-token k drawn uniformly from these
    bias: str = "none"          # "none" | "zipf" | "hot" | "equal" (all logits tie)
    bias_param: float = 0.0     # zipf: alpha; hot: beta
    zipf_s: float = 1.1

    def with_(self, **kw) -> "LayerSpec":
        return replace(self, **kw)


# The five layer shapes.  T is the default batch; sweeps override it.
TINY = LayerSpec("tiny", T=16, d=256, f=512, E=8, k=2)
MIXTRAL = LayerSpec("mixtral", T=256, d=4096, f=14336, E=8, k=2)
QWEN3 = LayerSpec("qwen3", T=64, d=2048, f=768, E=128, k=8, bias="zipf")
DEEPSEEK = LayerSpec("deepseek", T=512, d=2048, f=1408, E=64, k=6, n_shared=2, bias="hot")
PRISM = LayerSpec("prism", T=1024, d=2048, f=192, E=512, k=32, k_choices=(4, 8, 16, 32))

SPECS = {s.name: s for s in (TINY, MIXTRAL, QWEN3, DEEPSEEK, PRISM)}

MIXTRAL_DECODE_T = (1, 8, 32, 128, 256)
QWEN3_T = (64, 4096)
QWEN3_D_TARGETS = (16, 32, 64, 96)  # distinct active experts at T=64 (alpha = 0 gives ~126)
DEEPSEEK_T = (32, 512, 8192)

# Router biases calibrated on the CPU oracle's routing (tests/golden/
# make_routing_bias.py writes this file): the DeepSeek-shaped hot expert's
# logit bias per batch size (the hot expert then receives 4x the mean load),
# and the Qwen3-shaped Zipf alpha per target number of distinct experts.
ROUTING_BIAS_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests", "golden",
                                 "routing_bias.json")


def _routing_bias() -> dict:
    with open(ROUTING_BIAS_FILE) as fh:
        return json.load(fh)


def deepseek_spec(T: int) -> "LayerSpec":
    """The DeepSeek-shaped layer at batch T (first T rows of the 8192-token
    draw) with the hot-expert bias calibrated for T."""
    ent = _routing_bias()["deepseek_hot"][str(T)]
    return DEEPSEEK.with_(T=T, bias="hot", bias_param=float(ent["beta"]))


def deepseek_hot_target(T: int) -> int:
    """Tokens the hot expert receives at batch T: 4x the mean load."""
    return int(round(4 * T * DEEPSEEK.k / DEEPSEEK.E))


def qwen3_alpha(D: int) -> float:
    """Zipf alpha that makes the T=64 Qwen3-shaped batch activate D experts."""
    return float(_routing_bias()["qwen3_zipf"][str(D)]["alpha"])


def _seed(seed: int, name: str, idx: int = 0) -> int:
    return zlib.crc32(f"{seed}:{name}:{idx}".encode()) & 0x7FFFFFFF


def _gen(seed: int, name: str, idx: int = 0, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, name, idx))
    return g


def normal(shape, std: float, seed: int, name: str, idx: int = 0, device="cpu") -> torch.Tensor:
    g = _gen(seed, name, idx, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


@dataclass
class RoutingInputs:
    x: torch.Tensor                         # [T, d] fp32 (cpu)
    w_router: torch.Tensor                  # [E, d] fp32 (cpu)
    router_bias: Optional[torch.Tensor]     # [E] fp32 or None (cpu)
    k_per_token: Optional[torch.Tensor]     # [T] int32 or None (cpu)


def routing_inputs(spec: LayerSpec, seed: int = 0) -> RoutingInputs:
    """Hidden states, router weight, router bias and per-token k (CPU)."""
    x = normal((spec.T, spec.d), 1.0, seed, "x")
    wr = normal((spec.E, spec.d), 1.0 / math.sqrt(spec.d), seed, "w_router")
    bias = None
    if spec.bias == "zipf" and spec.bias_param != 0.0:
        bias = zipf_bias(spec, seed)
    elif spec.bias == "hot" and spec.bias_param != 0.0:
        hot = int(torch.randint(spec.E, (1,), generator=_gen(seed, "hot_expert")).item())
        bias = torch.zeros(spec.E, dtype=torch.float32)
        bias[hot] = spec.bias_param
    elif spec.bias == "equal":
        # every logit equal: x . W_r = 0 for all experts (tie stress)
        wr = torch.zeros_like(wr)
    kpt = None
    if spec.k_choices:
        ch = torch.tensor(spec.k_choices, dtype=torch.int32)
        sel = torch.randint(len(spec.k_choices), (spec.T,), generator=_gen(seed, "k_per_token"))
        kpt = ch[sel].contiguous()
    return RoutingInputs(x, wr, bias, kpt)


def zipf_bias(spec: LayerSpec, seed: int = 0) -> Optional[torch.Tensor]:
    """b_e = alpha * ln p_{pi(e)} with p_r proportional to r^-s (s = 1.1) and
    pi a seeded permutation, so the hot experts are not simply the low
    indices; None for alpha = 0."""
    if spec.bias_param == 0.0:
        return None
    perm = torch.randperm(spec.E, generator=_gen(seed, "zipf_perm"))
    ranks = torch.arange(1, spec.E + 1, dtype=torch.float64)
    p = ranks.pow(-spec.zipf_s)
    p = p / p.sum()
    return (spec.bias_param * torch.log(p))[perm].to(torch.float32).contiguous()


def hot_expert_index(spec: LayerSpec, seed: int = 0) -> int:
    return int(torch.randint(spec.E, (1,), generator=_gen(seed, "hot_expert")).item())


@dataclass
class ExpertWeightsF32:
    w_gate: torch.Tensor   # [E, f, d]
    w_up: torch.Tensor     # [E, f, d]
    w_down: torch.Tensor   # [E, d, f]
    ws_gate: Optional[torch.Tensor] = None  # [S, f, d]
    ws_up: Optional[torch.Tensor] = None
    ws_down: Optional[torch.Tensor] = None


def expert_weight(spec: LayerSpec, which: str, e: int, seed: int = 0, device="cpu",
                  shared: bool = False) -> torch.Tensor:
    """One expert's fp32 weight: which in {gate, up, down}."""
    name = ("shared_" if shared else "") + which
    if which == "down":
        return normal((spec.d, spec.f), 1.0 / math.sqrt(spec.f), seed, name, e, device)
    return normal((spec.f, spec.d), 1.0 / math.sqrt(spec.d), seed, name, e, device)


def expert_weights(spec: LayerSpec, seed: int = 0, device="cpu") -> ExpertWeightsF32:
    """All expert weights in fp32 (for small and medium layers; large layers
    should stream expert by expert with expert_weight)."""
    def stack(which, n, shared):
        return torch.stack([expert_weight(spec, which, e, seed, device, shared) for e in range(n)])
    w = ExpertWeightsF32(stack("gate", spec.E, False), stack("up", spec.E, False),
                         stack("down", spec.E, False))
    if spec.n_shared:
        w.ws_gate = stack("gate", spec.n_shared, True)
        w.ws_up = stack("up", spec.n_shared, True)
        w.ws_down = stack("down", spec.n_shared, True)
    return w
