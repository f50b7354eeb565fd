"""Shared set-up for the GPU parity tests: seeded layers on the device (through
the library's own quantiser) and the same layers for the CPU oracle (through
the oracle's quantiser, from the same fp32 draws)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as wl

fp8 = None


def lib():
    global fp8
    if fp8 is None:
        import fp8_moe_layer_amd as m
        fp8 = m
    return fp8


def dev():
    return torch.device("cuda", 0)


class Layer:
    """A layer on the GPU (DeviceWeights) and its oracle twin (QuantWeights)."""

    def __init__(self, spec: wl.LayerSpec, seed: int = 0, want_oracle: bool = True):
        m = lib()
        self.spec = spec
        ri = wl.routing_inputs(spec, seed)
        self.ri = ri
        d = dev()
        self.x = ri.x.to(d)
        self.w_router = ri.w_router.to(d)
        self.bias = None if ri.router_bias is None else ri.router_bias.to(d)
        self.kpt = None if ri.k_per_token is None else ri.k_per_token.to(d)
        S = spec.n_shared
        self.dw = m.DeviceWeights.empty(spec.E, spec.d, spec.f, S, device=d)
        host = {}
        if want_oracle:
            host = dict(w_gate=np.empty((spec.E, spec.f, spec.d), np.float32),
                        w_up=np.empty((spec.E, spec.f, spec.d), np.float32),
                        w_down=np.empty((spec.E, spec.d, spec.f), np.float32))
            if S:
                host.update(ws_gate=np.empty((S, spec.f, spec.d), np.float32),
                            ws_up=np.empty((S, spec.f, spec.d), np.float32),
                            ws_down=np.empty((S, spec.d, spec.f), np.float32))
        for shared, n in ((False, spec.E), (True, S)):
            for e in range(n):
                for which in ("gate", "up", "down"):
                    w32 = wl.expert_weight(spec, which, e, seed, d, shared)
                    self.dw.set_expert(which, e, w32, shared)
                    if want_oracle:
                        host[("ws_" if shared else "w_") + which][e] = w32.cpu().numpy()
                    del w32
        torch.cuda.synchronize()
        self.qw = None
        if want_oracle:
            self.qw = oracle.quantize_weights(host["w_gate"], host["w_up"], host["w_down"],
                                              host.get("ws_gate"), host.get("ws_up"),
                                              host.get("ws_down"))
            del host

    def layer(self, block_m=16, no_requant=False, persistent=False):
        return lib().MoELayer(self.dw, self.w_router, self.spec.k, self.bias, block_m, no_requant,
                              persistent)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()
