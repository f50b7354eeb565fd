"""Benchmark: the fused W8A8 FP8 MoE layer forward on one MI355X.

Headline workload: the Mixtral-8x7B-shaped layer -- d=4096, f=14336, E=8,
top-2, W8A8 e4m3 with per-output-channel weight scales and per-token
activation scales -- at the largest batch of its decode sweep, T=256 tokens,
unbiased router.  `value` is T / (mean ms per layer forward).

The same JSON line carries timed points for the other layer shapes
(`points`): the rest of the Mixtral decode sweep, the Qwen3-30B-A3B shape at
T=64 with 16 / 32 / 64 / 96 / ~126 distinct experts and at T=4096 (prefill),
the DeepSeek-MoE-16B shape (2 shared experts, the hot expert at 4x the mean
load) at T = 32 / 512 / 8192 (prefill), and the MoE-Prism elastic-k shape at
T=1024.  Each point reports its layer time, its fraction of the roofline
that bounds it (HBM for decode-sized batches, dense fp8 MFMA for the two
prefill batches), per-stage times and the oracle's parity on a token sample.

Inputs are seeded synthetic draws (workloads.py); the weights are drawn on
the GPU in fp32 and quantised by the library's own e4m3 quantiser.  When a
step's active weights are smaller than 1 GB, R weight copies rotate so the
256 MB Infinity Cache cannot serve them.

One step = one whole layer forward (quantise + router, top-k, permutation,
gate/up + SiLU*up, requantisation, down projection, combine) with inputs
resident in HBM.  W untimed warm-up steps, then K steps timed with HIP
events on the stream the library launches on.  A second pass records
per-step events (median), a third per-stage events (the library records
them around its launches) for the dominant kernel's roofline figure.  The
CPU oracle is timed on a bounded sample of the headline workload on the
host cores.

Prints ONE JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused FP8 MoE layer tokens/s; % peak HBM BW (decode), % FP8 MFMA peak (prefill)"
PEAK_HBM = 8.0e12        # MI355X HBM3E, bytes/s
PEAK_FP8 = 5.0e15        # MI355X dense fp8 MFMA, FLOP/s
RIDGE = PEAK_FP8 / PEAK_HBM

DEFAULT_T = {"tiny": 16, "mixtral": 256, "qwen3": 64, "deepseek": 512, "prism": 1024}
# batch sizes the pages' layer shapes call prefill-sized (the MFMA target)
PREFILL = {("qwen3", 4096), ("deepseek", 8192)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--config", default="mixtral", choices=sorted(DEFAULT_T))
    p.add_argument("--tokens", type=int, default=0, help="batch size (default per config)")
    p.add_argument("--distinct", type=int, default=0,
                   help="qwen3: Zipf offset calibrated for this many distinct experts at T=64")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle wall time")
    p.add_argument("--points", default="all", choices=["all", "none"],
                   help="also time the other layer shapes (all) or only the selected one (none)")
    p.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                   help="untimed forwards for this long before each timed loop (GPU clocks "
                        "ramp up after idle); 0: none")
    p.add_argument("--point-steps", type=int, default=50)
    p.add_argument("--point-warmup", type=int, default=20)
    p.add_argument("--parity-tokens", type=int, default=64,
                   help="tokens of each point compared with the oracle")
    p.add_argument("--no-requant", action="store_true")
    p.add_argument("--no-persistent", action="store_true",
                   help="skip timing the single persistent launch (profiling runs)")
    p.add_argument("--group", action="store_true",
                   help="qwen3: decode batches of 64 from a pool of 512 tokens, in arrival order "
                        "and grouped by expert affinity (moe_group_tokens)")
    p.add_argument("--tiers", action="store_true",
                   help="prism: the elastic-k pool as one mixed-k batch and as quality-tier "
                        "batches at one k each (moe_k_tiers)")
    p.add_argument("--graph", action="store_true",
                   help="also time the layer captured in a HIP graph (one graph per weight copy)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (for counter calibration)")
    return p.parse_args(argv)


class HipEvents:
    """hipEvent_t handles through the HIP runtime that torch has loaded."""

    def __init__(self, n):
        self.hip = C.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.ev = []
        for _ in range(n):
            h = C.c_void_p()
            rc = self.hip.hipEventCreate(C.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            self.ev.append(h.value)

    def record(self, i, stream):
        rc = self.hip.hipEventRecord(self.ev[i], stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(self.ev[b])
        ms = C.c_float()
        rc = self.hip.hipEventElapsedTime(C.byref(ms), self.ev[a], self.ev[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_peaks(torch, dev) -> dict:
    """The device as measured next to the spec-sheet peaks: compute units, and
    the bytes read + written per second by a plain 1 GiB device copy (a
    STREAM-like probe; the spec peak stays the roofline's denominator)."""
    props = torch.cuda.get_device_properties(dev)
    n = 1 << 28  # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    s = start.elapsed_time(end) * 1e-3 / reps
    del src, dst
    return {"compute_units": props.multi_processor_count, "arch": getattr(props, "gcnArchName", ""),
            "copy_GBps": round(2 * n * 4 / s / 1e9, 1),
            "copy_note": "1 GiB device copy, read + write bytes over time (torch copy kernel)"}


# The sources that make the expert GEMM kernels and their launches: device
# code, launchers and the host planner that picks their shapes.
GEMM_SOURCES = ("abi.hip", "common.hpp", "expert_dev.hpp", "internal.hpp", "kernels_expert.hip")


def kernel_source_hash() -> str:
    """Hash of the expert GEMMs' sources, to tell whether stored counter
    readings of the gate/up kernel still describe the kernel being timed."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_moe_layer_amd", "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3
    counter summary for this workload, or None when missing or stale."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = data.get(workload)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("gate_up_bytes")


# ------------------------------------------------------------------ algorithmic accounting

def accounting(spec, T, ids_np):
    """The roofline accounting of one layer forward (intermediates not counted):
    weights + fp32 scales of the distinct active routed experts and the shared
    experts, the fp32 router weight, the fp32 x read and the fp32 out written;
    FP8 flops 2 * rows * 3 * f * d with rows the (token, slot) pairs plus the
    shared-expert rows.  The gate/up kernel's own algorithmic bytes are its
    weights and scales: 2 * f * (d + 4) per active expert."""
    import numpy as np
    d, f, E, S = spec.d, spec.f, spec.E, spec.n_shared
    D = int(len(np.unique(ids_np[ids_np >= 0])))
    P = int((ids_np >= 0).sum())
    rows = P + S * T
    expert_bytes = 3 * f * d + 8 * f + 4 * d
    return {
        "distinct_experts": D, "pairs": P, "rows": rows,
        "layer_bytes": (D + S) * expert_bytes + E * d * 4 + 2 * T * d * 4,
        "layer_flops": 2 * rows * 3 * f * d,
        "gate_up_bytes": (D + S) * 2 * f * (d + 4),
        "gate_up_flops": 2 * rows * 2 * f * d,
        "down_bytes": (D + S) * d * (f + 4),
        "down_flops": 2 * rows * f * d,
    }


def layer_bound(acc):
    return "mfma" if acc["layer_flops"] / acc["layer_bytes"] > RIDGE else "hbm"


# ------------------------------------------------------------------ the measured layer

class Shape:
    """One layer shape resident on the GPU: seeded routing inputs on the
    device, expert weights drawn on the device and quantised there, and
    (want_host) the fp32 host copies the oracle quantises with its own codec."""

    def __init__(self, torch, fp8, wl, spec, seed, dev, want_host):
        import numpy as np
        self.torch, self.fp8, self.wl = torch, fp8, wl
        self.spec, self.seed, self.dev = spec, seed, dev
        ri = wl.routing_inputs(spec, seed)
        self.ri = ri
        self.x = ri.x.to(dev)
        self.w_router = ri.w_router.to(dev)
        self.kpt = None if ri.k_per_token is None else ri.k_per_token.to(dev)
        S = spec.n_shared
        self.dw = fp8.DeviceWeights.empty(spec.E, spec.d, spec.f, S, device=dev)
        host = {}
        if want_host:
            for sh in ((False, True) if S else (False,)):
                for which in ("gate", "up", "down"):
                    n = S if sh else spec.E
                    shp = (spec.d, spec.f) if which == "down" else (spec.f, spec.d)
                    host[("ws_" if sh else "w_") + which] = np.empty((n,) + shp, np.float32)
        for shared, n in ((False, spec.E), (True, S)):
            for e in range(n):
                for which in ("gate", "up", "down"):
                    w32 = wl.expert_weight(spec, which, e, seed, dev, shared)
                    self.dw.set_expert(which, e, w32, shared)
                    if want_host:
                        host[("ws_" if shared else "w_") + which][e] = w32.cpu().numpy()
                    del w32
        torch.cuda.synchronize()
        self.host32 = host
        self.qw = None
        self._copies = []

    def oracle_weights(self):
        if self.qw is None:
            import oracle
            h = self.host32
            self.qw = oracle.quantize_weights(h["w_gate"], h["w_up"], h["w_down"], h.get("ws_gate"),
                                              h.get("ws_up"), h.get("ws_down"))
            self.host32 = {}
        return self.qw

    def clone(self):
        dw = self.dw
        return self.fp8.DeviceWeights(*[None if t is None else t.clone() for t in
                                        (dw.w_gate, dw.w_up, dw.s_gate, dw.s_up, dw.w_down, dw.s_down,
                                         dw.ws_gate, dw.ws_up, dw.ss_gate, dw.ss_up, dw.ws_down,
                                         dw.ss_down)])

    def layers(self, T, bias, no_requant=False, persistent=False):
        """R rotated weight copies, R x (a step's active weight bytes) >= 1 GB
        (active experts counted from a first forward at this batch)."""
        import numpy as np
        torch, fp8, spec = self.torch, self.fp8, self.spec
        base = fp8.MoELayer(self.dw, self.w_router, spec.k, bias, no_requant=no_requant,
                            persistent=persistent)
        ids0 = torch.empty((T, spec.k), dtype=torch.int32, device=self.dev)
        base.forward(self.x[:T].contiguous(), k_per_token=self.kpt_of(T), topk_ids=ids0)
        i0 = ids0.cpu().numpy()
        active = len(np.unique(i0[i0 >= 0])) + spec.n_shared
        expert_bytes = 3 * spec.f * spec.d + 8 * spec.f + 4 * spec.d
        copies = max(1, min(16, math.ceil(1e9 / (active * expert_bytes))))
        while len(self._copies) < copies - 1:
            self._copies.append(self.clone())
        return [base] + [fp8.MoELayer(c, self.w_router, spec.k, bias, no_requant=no_requant,
                                      persistent=persistent) for c in self._copies[:copies - 1]]

    def kpt_of(self, T):
        return None if self.kpt is None else self.kpt[:T].contiguous()

    def free(self):
        self._copies = []
        self.dw = None


# Untimed work before every timed loop, in ms of wall time (--settle-ms).
# The GPU lowers its clocks within ~50 ms of idling (host-side set-up, the
# oracle's parity checks between points) and takes ~10-20 ms of load to come
# back: measured on the Mixtral-shaped T=256 layer, a loop of 5 + 20 steps
# started after 50 ms, 0.2 s or 1 s of idle ran 290-294 us per step, the next
# such loop 273-274 us and later ones 266-268 us, while a loop started after
# 100 ms of back-to-back forwards ran 266 us.  The timed steps then measure
# the layer at the clocks it runs at under load, whatever the warm-up count.
SETTLE_MS = 100.0


def settle(torch, fn):
    """Calls fn (one untimed forward) in batches of eight, synchronising after
    each batch, until SETTLE_MS of wall time have passed; returns the calls."""
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
        for _ in range(8):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def time_steps(torch, layers, x, kpt, out, ids, steps, warmup, sh):
    """Mean ms per step over `steps` back-to-back forwards (HIP events on the
    library's stream), after the settle phase and `warmup` untimed ones."""
    R = len(layers)
    settle(torch, lambda i: layers[i % R].forward(x, k_per_token=kpt, out=out, topk_ids=ids))
    for i in range(warmup):
        layers[i % R].forward(x, k_per_token=kpt, out=out, topk_ids=ids)
    torch.cuda.synchronize()
    ev = HipEvents(2)
    ev.record(0, sh)
    for i in range(steps):
        layers[i % R].forward(x, k_per_token=kpt, out=out, topk_ids=ids)
    ev.record(1, sh)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / steps
    ev.close()
    return ms


def step_distribution(torch, layers, x, kpt, out, ids, steps, sh):
    """p10 / median / p90 of single-step times (one event between steps)."""
    pev = HipEvents(steps + 1)
    pev.record(0, sh)
    for i in range(steps):
        layers[i % len(layers)].forward(x, k_per_token=kpt, out=out, topk_ids=ids)
        pev.record(i + 1, sh)
    torch.cuda.synchronize()
    per = sorted(pev.elapsed_ms(i, i + 1) * 1e3 for i in range(steps))
    pev.close()
    pct = lambda q: round(per[min(len(per) - 1, int(q * len(per)))], 2)
    return {"p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9)}


def stage_times(torch, fp8, layers, x, kpt, out, ids, steps, sh):
    """Mean µs per stage from events the library records around its launches
    (each event adds a few µs, so the stages sum to a little more than a step)."""
    nst = fp8.N_STAGE_EVENTS
    sev = HipEvents(nst * steps)
    acc = [0.0] * (nst - 1)
    for s in range(steps):
        layers[s % len(layers)].forward(x, k_per_token=kpt, out=out, topk_ids=ids,
                                        stage_events=sev.ev[s * nst:(s + 1) * nst])
    torch.cuda.synchronize()
    for s in range(steps):
        for i in range(nst - 1):
            acc[i] += sev.elapsed_ms(s * nst + i, s * nst + i + 1)
    sev.close()
    return {name: round(v / steps * 1e3, 2) for name, v in zip(fp8.STAGES, acc)}


def parity_sample(shape, T, x, kpt, bias_np, out, ids, n):
    """Oracle (full layer incl. router, on its own weights' quantisation) on
    the first n tokens: global and worst-token rel-L2, ids equality."""
    import numpy as np
    import oracle
    spec = shape.spec
    n = min(n, T)
    ks = None if kpt is None else kpt[:n].cpu().numpy()
    ref, ido, _ = oracle.forward(x[:n].cpu().numpy(), shape.oracle_weights(), spec.k,
                                 w_router=shape.ri.w_router.numpy(), router_bias=bias_np,
                                 k_per_token=ks)
    got = out[:n].cpu().numpy().astype(np.float64)
    per = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    return {"rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
            "max_token_rel_l2": float(per.max()),
            "ids_equal": bool(np.array_equal(ids[:n].cpu().numpy(), ido)), "tokens": n}


def time_persistent(torch, shape, T, bias, x, kpt, steps, warmup, sh):
    """The same steps as one cooperative launch each (MOE_F_PERSISTENT)."""
    spec = shape.spec
    lays = shape.layers(T, bias, persistent=True)
    out = torch.empty((T, spec.d), dtype=torch.float32, device=shape.dev)
    ids = torch.empty((T, spec.k), dtype=torch.int32, device=shape.dev)
    ms = time_steps(torch, lays, x, kpt, out, ids, steps, warmup, sh)
    status = max(lay.status() for lay in lays)
    # phase boundaries of the last launch on the first copy (its own clock)
    lays[0].forward(x, k_per_token=kpt, out=out, topk_ids=ids)
    torch.cuda.synchronize()
    return {"us_mean": round(ms * 1e3, 2), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "status": status, "phase_ends_us": lays[0].persistent_stamps()}


def measure_point(torch, fp8, shape, T, bias, steps, warmup, sh, parity_n, label, persistent=True):
    """Time one layer shape at batch T; roofline fractions of the layer."""
    spec = shape.spec
    layers = shape.layers(T, bias)
    x = shape.x[:T].contiguous()
    kpt = shape.kpt_of(T)
    out = torch.empty((T, spec.d), dtype=torch.float32, device=shape.dev)
    ids = torch.empty((T, spec.k), dtype=torch.int32, device=shape.dev)
    ms = time_steps(torch, layers, x, kpt, out, ids, steps, warmup, sh)
    dist = step_distribution(torch, layers, x, kpt, out, ids, steps, sh)
    stages = stage_times(torch, fp8, layers, x, kpt, out, ids, steps, sh)
    acc = accounting(spec, T, ids.cpu().numpy())
    bound = "mfma" if (spec.name, T) in PREFILL else layer_bound(acc)
    med = dist["median"] * 1e-6
    pt = {"workload": label, "T": T, "us_mean": round(ms * 1e3, 2), "us_median": dist["median"],
          "tokens_per_s": round(T / (ms * 1e-3), 1), "distinct_experts": acc["distinct_experts"],
          "n_shared": spec.n_shared, "weight_copies": len(layers), "bound": bound,
          "alg_bytes": acc["layer_bytes"], "fp8_flops": acc["layer_flops"],
          "hbm_frac": round(acc["layer_bytes"] / (ms * 1e-3) / PEAK_HBM, 4),
          "hbm_frac_median": round(acc["layer_bytes"] / med / PEAK_HBM, 4),
          "mfma_frac": round(acc["layer_flops"] / (ms * 1e-3) / PEAK_FP8, 4),
          "mfma_frac_median": round(acc["layer_flops"] / med / PEAK_FP8, 4),
          "stages_us": stages}
    if stages.get("gate_up"):
        t = stages["gate_up"] * 1e-6
        pt["gate_up"] = {"us": stages["gate_up"],
                         "hbm_frac": round(acc["gate_up_bytes"] / t / PEAK_HBM, 4),
                         "mfma_frac": round(acc["gate_up_flops"] / t / PEAK_FP8, 4)}
    if stages.get("down"):
        t = stages["down"] * 1e-6
        pt["down"] = {"us": stages["down"], "hbm_frac": round(acc["down_bytes"] / t / PEAK_HBM, 4),
                      "mfma_frac": round(acc["down_flops"] / t / PEAK_FP8, 4)}
    if persistent:
        pt["persistent"] = time_persistent(torch, shape, T, bias, x, kpt, steps, warmup, sh)
    if parity_n:
        bias_np = None if bias is None else bias.cpu().numpy()
        pt["parity"] = parity_sample(shape, T, x, kpt, bias_np, out, ids, parity_n)
    log(f"{label}: {pt['us_mean']} us (median {pt['us_median']}), D={acc['distinct_experts']}, "
        f"hbm {pt['hbm_frac']}, mfma {pt['mfma_frac']}, stages {stages}, "
        f"persistent {pt.get('persistent')}, parity {pt.get('parity')}")
    del layers
    return pt, ms, dist, stages, acc, out, ids


def _capture(torch, lay, x, kpt, out, ids):
    cap = torch.cuda.Stream()  # default priority
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        lay.forward(x, k_per_token=kpt, out=out, topk_ids=ids)  # workspace before capture
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay.forward(x, k_per_token=kpt, out=out, topk_ids=ids)
    return g


def _time_replays(torch, gs, steps, warmup):
    settle(torch, lambda i: gs[i % len(gs)].replay())
    for i in range(warmup):
        gs[i % len(gs)].replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        gs[i % len(gs)].replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def graph_timings(torch, fp8, shape, layers, x, kpt, out, ids, eager_ms, T, args, sh):
    """The layer replayed from HIP graphs.  For the elastic-k shape, one graph
    per routing budget k (the MoE-Prism segmented executor's per-k MoE
    segments): each k timed as graph replay, eager launches and the single
    persistent launch over the same batch; otherwise one graph per weight
    copy of the measured batch."""
    spec = shape.spec
    if spec.name != "prism":
        gs = [_capture(torch, lay, x, kpt, out, ids) for lay in layers]
        gms = _time_replays(torch, gs, args.steps, args.warmup)
        del gs
        res = {"us_per_step": round(gms * 1e3, 2), "eager_us_per_step": round(eager_ms * 1e3, 2),
               "tokens_per_s": round(T / (gms * 1e-3), 1), "graphs": len(layers)}
        log(f"graph replay: {res}")
        return res
    per_k = []
    for k in (4, 8, 16, 32):
        lay = fp8.MoELayer(shape.dw, shape.w_router, k)
        ok = torch.empty((T, spec.d), dtype=torch.float32, device=shape.dev)
        ik = torch.empty((T, k), dtype=torch.int32, device=shape.dev)
        g = _capture(torch, lay, x, None, ok, ik)
        gms = _time_replays(torch, [g], args.steps, args.warmup)
        del g
        ems = time_steps(torch, [lay], x, None, ok, ik, args.steps, args.warmup, sh)
        pl = fp8.MoELayer(shape.dw, shape.w_router, k, persistent=True)
        pms = time_steps(torch, [pl], x, None, ok, ik, args.steps, args.warmup, sh)
        ent = {"k": k, "graph_us": round(gms * 1e3, 2), "eager_us": round(ems * 1e3, 2),
               "persistent_us": round(pms * 1e3, 2), "persistent_status": pl.status()}
        per_k.append(ent)
        log(f"graph per k: {ent}")
    return {"per_k": per_k, "T": T, "note": "one captured graph per k, all tokens served at k"}


def bias_for(wl, cfg, T, distinct, seed, dev):
    """Router bias of a layer shape at batch T, on the device (or None)."""
    if cfg == "deepseek":
        return wl.routing_inputs(wl.deepseek_spec(T).with_(T=1), seed).router_bias.to(dev)
    if cfg == "qwen3" and distinct:
        b = wl.zipf_bias(wl.QWEN3.with_(bias_param=wl.qwen3_alpha(distinct)), seed)
        return b.to(dev)
    return None


def shape_spec(wl, cfg, Tmax):
    if cfg == "deepseek":
        return wl.DEEPSEEK.with_(T=Tmax, bias="none")
    if cfg == "qwen3":
        return wl.QWEN3.with_(T=Tmax, bias_param=0.0)
    return wl.SPECS[cfg].with_(T=Tmax)


def main():
    global SETTLE_MS
    args = parse()
    SETTLE_MS = max(0.0, args.settle_ms)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py runs on one GPU only: this build measures the layer on a single MI355X "
              "(no sharding, no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    dev = torch.device("cuda", 0)
    if args.calibrate_copy:
        n = 1 << 28  # 1 GiB of fp32
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 3}))
        return

    import fp8_moe_layer_amd as fp8
    import workloads as wl

    cfg = args.config
    T = args.tokens or DEFAULT_T[cfg]
    want_cpu = not args.no_cpu_baseline
    sh = torch.cuda.current_stream().cuda_stream

    # ---- the selected (headline) workload
    Tmax = max(T, *(wl.MIXTRAL_DECODE_T if cfg == "mixtral" else (T,)))
    if cfg == "deepseek":
        Tmax = max(T, wl.DEEPSEEK_T[-1])
    spec = shape_spec(wl, cfg, Tmax)
    log(f"workload {cfg}-shaped d={spec.d} f={spec.f} E={spec.E}+{spec.n_shared} k={spec.k} T={T}")
    t0 = time.time()
    shape = Shape(torch, fp8, wl, spec, args.seed, dev, want_host=want_cpu or args.points == "all")
    log(f"weights ready in {time.time() - t0:.1f}s")
    bias = bias_for(wl, cfg, T, args.distinct, args.seed, dev)
    layers = shape.layers(T, bias, args.no_requant)
    x = shape.x[:T].contiguous()
    kpt = shape.kpt_of(T)
    out = torch.empty((T, spec.d), dtype=torch.float32, device=dev)
    ids = torch.empty((T, spec.k), dtype=torch.int32, device=dev)
    ms = time_steps(torch, layers, x, kpt, out, ids, args.steps, args.warmup, sh)
    tokens_per_s = T / (ms * 1e-3)
    n_copies = len(layers)
    log(f"T={T}: {ms * 1e3:.1f} us/step, {tokens_per_s:.4g} tokens/s, {len(layers)} weight copies")
    step_us = step_distribution(torch, layers, x, kpt, out, ids, args.steps, sh)
    log(f"per-step us: {step_us}")
    stages_us = stage_times(torch, fp8, layers, x, kpt, out, ids, args.steps, sh)
    log(f"stages (us): {stages_us}")
    acc = accounting(spec, T, ids.cpu().numpy())

    # dominant kernel: the gate/up grouped GEMM, algorithmic bytes = weights +
    # scales of the active experts (2 f (d + 4) per expert), flops 2 rows 2f d
    t_gu = stages_us["gate_up"] * 1e-6
    workload = f"{cfg} T={T}"
    if (cfg, T) in PREFILL:
        roofline = {"bound": "mfma", "achieved": round(acc["gate_up_flops"] / t_gu / 1e12, 1),
                    "peak": PEAK_FP8 / 1e12, "unit": "TFLOP/s",
                    "frac": round(acc["gate_up_flops"] / t_gu / PEAK_FP8, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(acc["gate_up_bytes"] / t_gu / 1e9, 1),
                    "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                    "frac": round(acc["gate_up_bytes"] / t_gu / PEAK_HBM, 4)}
    roofline.update({
        "traffic": stored_traffic(workload), "kernel": "gate/up grouped GEMM (SiLU*up epilogue)",
        "alg_bytes_per_launch": acc["gate_up_bytes"],
        "alg_bytes_note": "e4m3 weights + fp32 scales of the distinct active experts, "
                          "2*f*(d+4) bytes each; intermediates not counted",
        "fp8_flops_per_launch": acc["gate_up_flops"], "avg_launch_us": stages_us["gate_up"],
        "timing": "hipEvents recorded by the library on its stream around the launch",
        "measured": measured_peaks(torch, dev)})
    med = step_us["median"] * 1e-6
    layer = {"alg_bytes": acc["layer_bytes"], "fp8_flops": acc["layer_flops"],
             "bound": "mfma" if (cfg, T) in PREFILL else layer_bound(acc),
             "hbm_frac": round(acc["layer_bytes"] / (ms * 1e-3) / PEAK_HBM, 4),
             "hbm_frac_median": round(acc["layer_bytes"] / med / PEAK_HBM, 4),
             "mfma_frac": round(acc["layer_flops"] / (ms * 1e-3) / PEAK_FP8, 5),
             "mfma_frac_median": round(acc["layer_flops"] / med / PEAK_FP8, 5),
             "alg_bytes_note": "weights + scales of the distinct active and shared experts, "
                               "fp32 router weight, x read and out written (fp32)"}

    # ---- the same steps as one persistent cooperative launch each
    persistent = None
    if not args.no_requant and not args.no_persistent:
        persistent = time_persistent(torch, shape, T, bias, x, kpt, args.steps, args.warmup, sh)
        persistent["staged_us_mean"] = round(ms * 1e3, 2)
        log(f"persistent single launch: {persistent}")

    # ---- the same steps replayed from HIP graphs (launch overhead removed)
    graph = None
    if args.graph:
        graph = graph_timings(torch, fp8, shape, layers, x, kpt, out, ids, ms, T, args, sh)

    # ---- decode batches from a token pool: arrival order vs grouped by expert affinity
    grouping = None
    if args.group and cfg == "qwen3":
        grouping = []
        pool, gb = 512, 64
        for alpha in (0.0, 1.0, 1.5):
            gs_ = wl.QWEN3.with_(T=pool, bias_param=alpha)
            gri = wl.routing_inputs(gs_, args.seed)
            gbias = None if gri.router_bias is None else gri.router_bias.to(dev)
            glay = fp8.MoELayer(shape.dw, gri.w_router.to(dev), gs_.k, gbias)
            gx = gri.x.to(dev)
            gid = torch.empty((pool, gs_.k), dtype=torch.int32, device=dev)
            glay.forward(gx, topk_ids=gid)
            gi = gid.cpu().numpy()
            t0 = time.time()
            order = fp8.group_tokens(gi, spec.E, gb)
            host_ms = (time.time() - t0) * 1e3
            entry = {"alpha": alpha, "pool": pool, "batch": gb, "group_host_ms": round(host_ms, 2)}
            for mode, idx in (("arrival", np.arange(pool)), ("grouped", order)):
                bx = [gx[torch.as_tensor(idx[b:b + gb], device=dev, dtype=torch.long)].contiguous()
                      for b in range(0, pool, gb)]
                Ds = [int(len(np.unique(gi[idx[b:b + gb]][gi[idx[b:b + gb]] >= 0])))
                      for b in range(0, pool, gb)]
                bout = torch.empty((gb, spec.d), dtype=torch.float32, device=dev)
                settle(torch, lambda i: glay.forward(bx[i % len(bx)], out=bout))
                for i in range(args.warmup):
                    glay.forward(bx[i % len(bx)], out=bout)
                ev = HipEvents(2)
                torch.cuda.synchronize()
                rounds = max(1, args.steps // len(bx))
                ev.record(0, sh)
                for r in range(rounds):
                    for xb in bx:
                        glay.forward(xb, out=bout)
                ev.record(1, sh)
                torch.cuda.synchronize()
                bms = ev.elapsed_ms(0, 1) / (rounds * len(bx))
                ev.close()
                entry[mode] = {"mean_distinct_experts": round(float(np.mean(Ds)), 1),
                               "us_per_batch": round(bms * 1e3, 1)}
            grouping.append(entry)
            log(f"grouping alpha={alpha}: {entry}")

    # ---- elastic-k pool: one mixed-k batch vs quality-tier batches at one k each
    tiers = None
    if args.tiers and cfg == "prism":
        tiers = []
        kp = shape.kpt[:T].cpu().numpy()
        tlays = {}

        def tlay(k):
            if k not in tlays:
                tlays[k] = fp8.MoELayer(shape.dw, shape.w_router, k, None)
            return tlays[k]

        def time_runs(runs):
            settle(torch, lambda i: runs[i % len(runs)][0].forward(
                runs[i % len(runs)][1], k_per_token=runs[i % len(runs)][2], out=runs[i % len(runs)][3]))
            for i in range(max(1, args.warmup // len(runs))):
                for lay_, xb, kb, ob in runs:
                    lay_.forward(xb, k_per_token=kb, out=ob)
            rounds = max(1, args.steps // len(runs))
            ev = HipEvents(2)
            torch.cuda.synchronize()
            ev.record(0, sh)
            for r in range(rounds):
                for lay_, xb, kb, ob in runs:
                    lay_.forward(xb, k_per_token=kb, out=ob)
            ev.record(1, sh)
            torch.cuda.synchronize()
            ms_ = ev.elapsed_ms(0, 1) / rounds
            ev.close()
            return ms_

        mixed_ms = time_runs([(tlay(spec.k), x, kpt,
                               torch.empty((T, spec.d), dtype=torch.float32, device=dev))])
        budget_pairs = int(kp.sum())
        for tb, ov in ((256, 0), (256, 4096), (128, 0), (128, 4096)):
            order, start, bk = fp8.k_tiers(kp, tb, ov)
            runs = []
            for b in range(len(bk)):
                idx = torch.as_tensor(order[start[b]:start[b + 1]], device=dev, dtype=torch.long)
                runs.append((tlay(int(bk[b])), shape.x[idx].contiguous(), None,
                             torch.empty((len(idx), spec.d), dtype=torch.float32, device=dev)))
            served = int(sum(int(bk[b]) * int(start[b + 1] - start[b]) for b in range(len(bk))))
            tms = time_runs(runs)
            entry = {"pool": T, "batch": tb, "overhead_pairs": ov, "n_batches": len(bk),
                     "over_service": round(served / budget_pairs, 4),
                     "us_per_pool_tiered": round(tms * 1e3, 1),
                     "us_per_pool_mixed": round(mixed_ms * 1e3, 1)}
            tiers.append(entry)
            log(f"tiers: {entry}")

    # ---- CPU oracle on a bounded sample of the headline workload, plus parity
    cpu = None
    parity = None
    if want_cpu:
        import oracle
        t0 = time.time()
        qw = shape.oracle_weights()
        log(f"oracle weights quantised in {time.time() - t0:.1f}s")
        cores = len(os.sched_getaffinity(0))
        xs_all = x.cpu().numpy()
        ks_all = None if kpt is None else kpt.cpu().numpy()
        bias_np = None if bias is None else bias.cpu().numpy()

        def run_oracle(n, nthreads=cores):
            ks = None if ks_all is None else ks_all[:n]
            return oracle.forward(xs_all[:n], qw, spec.k, w_router=shape.ri.w_router.numpy(),
                                  router_bias=bias_np, k_per_token=ks, nthreads=nthreads)

        # size the sample for ~cpu_seconds of oracle work: probe, then scale
        n = min(T, max(1, 4 * cores // max(1, spec.k)))
        t0 = time.time()
        ref, ido, _ = run_oracle(n)
        probe = time.time() - t0
        reps = 1
        if probe < args.cpu_seconds:
            if n < T:
                n2 = min(T, int(n * args.cpu_seconds / max(probe, 1e-3)))
                if n2 > n:
                    n = n2
                    t0 = time.time()
                    ref, ido, _ = run_oracle(n)
                    probe = time.time() - t0
            reps = max(1, min(20, int(args.cpu_seconds / max(probe, 1e-3))))
        t0 = time.time()
        for _ in range(reps):
            ref, ido, _ = run_oracle(n)
        wall = time.time() - t0
        # the same oracle on one thread, over a 1/cores share of the sample
        n1 = max(1, n // cores)
        t0 = time.time()
        run_oracle(n1, 1)
        wall1 = time.time() - t0
        cpu = {"value": round(n * reps / wall, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"first {n} of the {T} tokens, full layer incl. router, repeated {reps}x "
                         f"(the oracle quantises its own weights beforehand, untimed)",
               "seconds": round(wall, 2), "cpu_model": cpu_model(),
               "single_thread": {"value": round(n1 / wall1, 3), "unit": "tokens/s",
                                 "sample": f"first {n1} tokens", "seconds": round(wall1, 2)}}
        got = out[:n].cpu().numpy().astype(np.float64)
        per = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
        parity = {"rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
                  "max_token_rel_l2": float(per.max()),
                  "ids_equal": bool(np.array_equal(ids[:n].cpu().numpy(), ido)), "tokens": n}
        log(f"oracle: {n} tokens x{reps} in {wall:.1f}s on {cores} cores; parity {parity}")
    del layers

    # ---- the other layer shapes (points), same JSON line
    points = None
    if args.points == "all":
        points = []
        psteps, pwarm, pn = args.point_steps, args.point_warmup, args.parity_tokens
        if cfg == "mixtral":
            for Tn in wl.MIXTRAL_DECODE_T:
                if Tn != T:
                    points.append(measure_point(torch, fp8, shape, Tn, None, psteps, pwarm, sh, pn,
                                                f"mixtral-shaped decode T={Tn}")[0])
        shape.free()
        del shape
        torch.cuda.empty_cache()
        for pcfg in ("qwen3", "deepseek", "prism"):
            if pcfg == cfg:
                continue
            Tm = {"qwen3": wl.QWEN3_T[-1], "deepseek": wl.DEEPSEEK_T[-1], "prism": wl.PRISM.T}[pcfg]
            ps = Shape(torch, fp8, wl, shape_spec(wl, pcfg, Tm), args.seed, dev, want_host=pn > 0)
            if pcfg == "qwen3":
                for D in (*wl.QWEN3_D_TARGETS, 0):
                    b = bias_for(wl, pcfg, 64, D, args.seed, dev)
                    lab = f"qwen3-shaped decode T=64, Zipf offset for {D} distinct experts" if D \
                        else "qwen3-shaped decode T=64, no offset"
                    points.append(measure_point(torch, fp8, ps, 64, b, psteps, pwarm, sh, pn, lab)[0])
                points.append(measure_point(torch, fp8, ps, 4096, None, psteps, pwarm, sh, pn,
                                            "qwen3-shaped prefill T=4096")[0])
            elif pcfg == "deepseek":
                for Tn in wl.DEEPSEEK_T:
                    b = bias_for(wl, pcfg, Tn, 0, args.seed, dev)
                    kind = "prefill" if (pcfg, Tn) in PREFILL else "decode"
                    lab = f"deepseek-shaped {kind} T={Tn}, 2 shared experts, hot expert at 4x the mean load"
                    pt = measure_point(torch, fp8, ps, Tn, b, psteps, pwarm, sh, pn, lab)[0]
                    points.append(pt)
            else:
                points.append(measure_point(torch, fp8, ps, wl.PRISM.T, None, psteps, pwarm, sh, pn,
                                            "prism-shaped elastic-k T=1024, k in {4,8,16,32}")[0])
            ps.free()
            del ps
            torch.cuda.empty_cache()

    cfg_out = {"workload": f"{cfg}-shaped W8A8 FP8 MoE layer forward, batch T={T}", "T": T,
               "d": spec.d, "f": spec.f, "E": spec.E, "n_shared": spec.n_shared, "k": spec.k,
               "block_m": 16, "requant": not args.no_requant,
               "distinct_experts": acc["distinct_experts"],
               "router_bias": "none" if bias is None else spec.bias if cfg != "qwen3" else "zipf",
               "weight_copies": n_copies}
    if cfg == "deepseek":
        hot = wl.hot_expert_index(spec, args.seed)
        cnt = int((ids.cpu().numpy() == hot).sum())
        cfg_out["hot_expert_load_vs_mean"] = round(cnt / (T * spec.k / spec.E), 3)
    res = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": SETTLE_MS,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" + ("" if not args.no_requant else "+fp32_intermediate"),
        "data": "synthetic",
        "config": cfg_out,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layer": layer,
        "step_us": step_us,
        "stages_us": stages_us,
        **({"graph": graph} if graph else {}),
        **({"persistent": persistent} if persistent else {}),
        "parity": parity,
    }
    if points is not None:
        res["points"] = points
    if grouping is not None:
        res["grouping"] = grouping
    if tiers is not None:
        res["tiers"] = tiers
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
