"""Benchmark: the fused W8A8 FP8 MoE layer forward on one MI355X.

Default workload: the Mixtral-8x7B-shaped layer -- d=4096, f=14336, E=8,
top-2, W8A8 e4m3 with per-output-channel weight scales and per-token
activation scales -- at the largest batch of its decode sweep, T=256 tokens,
unbiased router.  `--config` selects the other layer shapes (Qwen3-,
DeepSeek-MoE- and MoE-Prism-shaped) for their own measurements.  Inputs are
seeded synthetic draws (workloads.py); the weights are drawn on the GPU in
fp32 and quantised by the library's own e4m3 quantiser.  When the active
weights of a step are smaller than 1 GB, R weight copies are rotated so the
256 MB Infinity Cache cannot serve them.

One step = one whole layer forward (quantise + router, top-k, permutation,
gate/up + SiLU*up, requantisation, down projection, combine) with inputs
already resident in HBM.  W untimed warm-up steps, then K steps timed with
HIP events on the stream the library launches on.  A second pass of K steps
records per-stage events (moe_debug_stage_events) to time the dominant
kernel (gate/up grouped GEMM) for the roofline figure.  The CPU oracle is
timed on a bounded sample of the same workload on the host cores.

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
DEFAULT_BIAS = {"qwen3": 0.0, "deepseek": 2.0}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--config", default="mixtral", choices=sorted(DEFAULT_T))
    p.add_argument("--tokens", type=int, default=0, help="batch size (default per config)")
    p.add_argument("--bias-param", type=float, default=None,
                   help="Zipf alpha (qwen3) or hot-expert logit bias (deepseek)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle wall time")
    p.add_argument("--sweep", action="store_true", help="also time the config's batch sweep")
    p.add_argument("--no-requant", action="store_true")
    p.add_argument("--zipf-sweep", action="store_true",
                   help="qwen3: also time T=64 at several Zipf router biases (distinct experts 16..128)")
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
    return p.parse_args()


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


def main():
    args = parse()
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
    sweep_T = {"mixtral": wl.MIXTRAL_DECODE_T, "qwen3": wl.QWEN3_T,
               "deepseek": wl.DEEPSEEK_T}.get(cfg, (T,)) if args.sweep else ()
    Tmax = max([T, *sweep_T])
    spec = wl.SPECS[cfg].with_(T=Tmax)
    if cfg in DEFAULT_BIAS:
        spec = spec.with_(bias_param=DEFAULT_BIAS[cfg] if args.bias_param is None else args.bias_param)
    S = spec.n_shared
    want_cpu = not args.no_cpu_baseline
    log(f"workload {cfg}-shaped d={spec.d} f={spec.f} E={spec.E}+{S} k={spec.k} T={T}")

    # ---- inputs: routing on the CPU generator, expert weights drawn on the GPU
    ri = wl.routing_inputs(spec, args.seed)
    x_all = ri.x.to(dev)
    w_router = ri.w_router.to(dev)
    bias = None if ri.router_bias is None else ri.router_bias.to(dev)
    kpt_all = None if ri.k_per_token is None else ri.k_per_token.to(dev)
    dw = fp8.DeviceWeights.empty(spec.E, spec.d, spec.f, S, device=dev)
    host32 = {}
    if want_cpu:
        host32 = {("w_" if not sh else "ws_") + which: np.empty(
            ((S if sh else spec.E),) + ((spec.d, spec.f) if which == "down" else (spec.f, spec.d)),
            np.float32) for sh in ((False, True) if S else (False,)) for which in ("gate", "up", "down")}
    t0 = time.time()
    for shared, n in ((False, spec.E), (True, S)):
        for e in range(n):
            for which in ("gate", "up", "down"):
                w32 = wl.expert_weight(spec, which, e, args.seed, dev, shared)
                dw.set_expert(which, e, w32, shared)
                if want_cpu:
                    host32[("ws_" if shared else "w_") + which][e] = w32.cpu().numpy()
                del w32
    torch.cuda.synchronize()
    log(f"weights ready in {time.time() - t0:.1f}s")
    d, f, E = spec.d, spec.f, spec.E
    expert_bytes = 3 * f * d + 8 * f + 4 * d

    def clone_weights():
        return fp8.DeviceWeights(*[None if t is None else t.clone() for t in
                                   (dw.w_gate, dw.w_up, dw.s_gate, dw.s_up, dw.w_down, dw.s_down,
                                    dw.ws_gate, dw.ws_up, dw.ss_gate, dw.ss_up, dw.ws_down, dw.ss_down)])

    def layers_for(Tn):
        """Rotated weight copies so that one step's active weights x copies >= 1 GB
        (the active experts counted from a first forward at this batch)."""
        base = fp8.MoELayer(dw, w_router, spec.k, bias, no_requant=args.no_requant)
        ids0 = torch.empty((Tn, spec.k), dtype=torch.int32, device=dev)
        base.forward(x_all[:Tn].contiguous(), k_per_token=None if kpt_all is None else
                     kpt_all[:Tn].contiguous(), topk_ids=ids0)
        i0 = ids0.cpu().numpy()
        active = len(np.unique(i0[i0 >= 0])) + S
        copies = max(1, min(16, math.ceil(1e9 / (active * expert_bytes))))
        out = [base]
        for _ in range(copies - 1):
            out.append(fp8.MoELayer(clone_weights(), w_router, spec.k, bias, no_requant=args.no_requant))
        return out

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def time_layer(Tn, steps, warmup, layers):
        x = x_all[:Tn].contiguous()
        kpt = None if kpt_all is None else kpt_all[:Tn].contiguous()
        out = torch.empty((Tn, d), dtype=torch.float32, device=dev)
        ids = torch.empty((Tn, spec.k), dtype=torch.int32, device=dev)
        R = len(layers)
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
        return ms, x, kpt, out, ids

    def accounting(Tn, ids_np):
        D = int(len(np.unique(ids_np[ids_np >= 0])))
        P = int((ids_np >= 0).sum())
        rows = P + S * Tn
        gu_bytes = (D + S) * 2 * f * (d + 4) + Tn * (d + 4) + rows * f * 4
        gu_flops = 2 * rows * 2 * f * d
        layer_bytes = (D + S) * expert_bytes + E * d * 4 + 2 * Tn * d * 4
        flops = 2 * rows * 3 * f * d
        return D, P, gu_bytes, gu_flops, layer_bytes, flops

    # ---- headline timing
    layers = layers_for(T)
    ms, x, kpt, out, ids = time_layer(T, args.steps, args.warmup, layers)
    tokens_per_s = T / (ms * 1e-3)
    log(f"T={T}: {ms * 1e3:.1f} us/step, {tokens_per_s:.4g} tokens/s, {len(layers)} weight copies")

    # ---- per-step distribution (events around each step only)
    pev = HipEvents(args.steps + 1)
    pev.record(0, sh)
    for i in range(args.steps):
        layers[i % len(layers)].forward(x, k_per_token=kpt, out=out, topk_ids=ids)
        pev.record(i + 1, sh)
    torch.cuda.synchronize()
    per_step = sorted(pev.elapsed_ms(i, i + 1) * 1e3 for i in range(args.steps))
    pev.close()
    pct = lambda q: round(per_step[min(len(per_step) - 1, int(q * len(per_step)))], 2)
    step_us = {"p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9)}
    log(f"per-step us: {step_us}")

    # ---- per-stage timing (second pass, same inputs)
    nst = fp8.N_STAGE_EVENTS
    sev = HipEvents(nst * args.steps)
    stage_sum = [0.0] * (nst - 1)
    keep = []
    for s in range(args.steps):
        keep.append(fp8.set_stage_events(sev.ev[s * nst:(s + 1) * nst]))
        layers[s % len(layers)].forward(x, k_per_token=kpt, out=out, topk_ids=ids)
    fp8.set_stage_events(None)
    torch.cuda.synchronize()
    for s in range(args.steps):
        for i in range(nst - 1):
            stage_sum[i] += sev.elapsed_ms(s * nst + i, s * nst + i + 1)
    sev.close()
    stages_us = {name: round(v / args.steps * 1e3, 2) for name, v in zip(fp8.STAGES, stage_sum)}
    log(f"stages (us): {stages_us}")

    ids_np = ids.cpu().numpy()
    D, P, gu_bytes, gu_flops, layer_bytes, flops = accounting(T, ids_np)
    t_gu = stages_us["gate_up"] * 1e-6
    workload = f"{cfg} T={T}"
    if gu_flops / gu_bytes > RIDGE:
        roofline = {"bound": "mfma", "achieved": round(gu_flops / t_gu / 1e12, 1),
                    "peak": PEAK_FP8 / 1e12, "unit": "TFLOP/s", "frac": round(gu_flops / t_gu / PEAK_FP8, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(gu_bytes / t_gu / 1e9, 1), "peak": PEAK_HBM / 1e9,
                    "unit": "GB/s", "frac": round(gu_bytes / t_gu / PEAK_HBM, 4)}
    roofline.update({"traffic": stored_traffic(workload), "kernel": "wsgemm_kernel (gate/up)",
                     "alg_bytes_per_launch": gu_bytes, "fp8_flops_per_launch": gu_flops,
                     "avg_launch_us": stages_us["gate_up"], "timing": "hipEvents around the launch, "
                     "recorded by the library on its stream",
                     "measured": measured_peaks(torch, dev)})

    # ---- the same steps replayed from HIP graphs (launch overhead removed)
    graph = None
    if args.graph:
        gs = []
        cap = torch.cuda.Stream()  # default priority
        for lay in layers:
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):
                lay.forward(x, k_per_token=kpt, out=out, topk_ids=ids)
            torch.cuda.current_stream().wait_stream(cap)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                lay.forward(x, k_per_token=kpt, out=out, topk_ids=ids)
            gs.append(g)
        for i in range(args.warmup):
            gs[i % len(gs)].replay()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(args.steps):
            gs[i % len(gs)].replay()
        end.record()
        torch.cuda.synchronize()
        gms = start.elapsed_time(end) / args.steps
        graph = {"us_per_step": round(gms * 1e3, 2), "eager_us_per_step": round(ms * 1e3, 2),
                 "tokens_per_s": round(T / (gms * 1e-3), 1), "graphs": len(gs)}
        log(f"graph replay: {graph}")
        del gs

    # ---- batch sweep (same weights)
    sweep = None
    if sweep_T:
        sweep = {}
        for Tn in sweep_T:
            lay = layers_for(Tn)
            mst, _, _, _, idt = time_layer(Tn, args.steps, args.warmup, lay)
            Dn, _, _, _, lb, fl = accounting(Tn, idt.cpu().numpy())
            sweep[str(Tn)] = {"us": round(mst * 1e3, 1), "tokens_per_s": round(Tn / (mst * 1e-3), 1),
                              "distinct_experts": Dn, "hbm_frac": round(lb / (mst * 1e-3) / PEAK_HBM, 4),
                              "mfma_frac": round(fl / (mst * 1e-3) / PEAK_FP8, 4), "weight_copies": len(lay)}
            log(f"sweep T={Tn}: {sweep[str(Tn)]}")
            del lay

    # ---- Qwen3-shaped decode at several router biases (distinct active experts)
    zipf = None
    # ---- decode batches from a token pool: arrival order vs grouped by expert affinity
    grouping = None
    if args.group and cfg == "qwen3":
        grouping = []
        pool, gb = 512, 64
        for alpha in (0.0, 1.0, 1.5):
            gs_ = wl.SPECS[cfg].with_(T=pool, bias_param=alpha)
            gri = wl.routing_inputs(gs_, args.seed)
            gbias = None if gri.router_bias is None else gri.router_bias.to(dev)
            glay = fp8.MoELayer(dw, gri.w_router.to(dev), gs_.k, gbias)
            gx = gri.x.to(dev)
            gid = torch.empty((pool, gs_.k), dtype=torch.int32, device=dev)
            glay.forward(gx, topk_ids=gid)
            gi = gid.cpu().numpy()
            t0 = time.time()
            order = fp8.group_tokens(gi, E, gb)
            host_ms = (time.time() - t0) * 1e3
            entry = {"alpha": alpha, "pool": pool, "batch": gb, "group_host_ms": round(host_ms, 2)}
            for mode, idx in (("arrival", np.arange(pool)), ("grouped", order)):
                bx = [gx[torch.as_tensor(idx[b:b + gb], device=dev, dtype=torch.long)].contiguous()
                      for b in range(0, pool, gb)]
                Ds = [int(len(np.unique(gi[idx[b:b + gb]][gi[idx[b:b + gb]] >= 0]))) for b in range(0, pool, gb)]
                bout = torch.empty((gb, d), dtype=torch.float32, device=dev)
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
        kp = kpt_all[:T].cpu().numpy()
        tlays = {}

        def tlay(k):
            if k not in tlays:
                tlays[k] = fp8.MoELayer(dw, w_router, k, bias)
            return tlays[k]

        def time_runs(runs):
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

        xm = x_all[:T].contiguous()
        mixed_ms = time_runs([(tlay(spec.k), xm, kpt_all[:T].contiguous(),
                               torch.empty((T, d), dtype=torch.float32, device=dev))])
        budget_pairs = int(kp.sum())
        for tb, ov in ((256, 0), (256, 4096), (128, 0), (128, 4096)):
            order, start, bk = fp8.k_tiers(kp, tb, ov)
            runs = []
            for b in range(len(bk)):
                idx = torch.as_tensor(order[start[b]:start[b + 1]], device=dev, dtype=torch.long)
                runs.append((tlay(int(bk[b])), x_all[idx].contiguous(), None,
                             torch.empty((len(idx), d), dtype=torch.float32, device=dev)))
            served_pairs = int(sum(int(bk[b]) * int(start[b + 1] - start[b]) for b in range(len(bk))))
            tms = time_runs(runs)
            entry = {"pool": T, "batch": tb, "overhead_pairs": ov, "n_batches": len(bk),
                     "over_service": round(served_pairs / budget_pairs, 4),
                     "us_per_pool_tiered": round(tms * 1e3, 1),
                     "us_per_pool_mixed": round(mixed_ms * 1e3, 1)}
            tiers.append(entry)
            log(f"tiers: {entry}")

    if args.zipf_sweep and cfg == "qwen3":
        zipf = []
        zcopies = []
        for alpha in (0.0, 1.0, 1.5, 2.0, 3.0, 4.0):
            zs = wl.SPECS[cfg].with_(T=64, bias_param=alpha)
            zri = wl.routing_inputs(zs, args.seed)
            zb = None if zri.router_bias is None else zri.router_bias.to(dev)
            zx = zri.x.to(dev)
            base = fp8.MoELayer(dw, zri.w_router.to(dev), zs.k, zb)
            zid = torch.empty((64, zs.k), dtype=torch.int32, device=dev)
            base.forward(zx, topk_ids=zid)
            zi = zid.cpu().numpy()
            Dz = int(len(np.unique(zi[zi >= 0])))
            copies = max(1, min(16, math.ceil(1e9 / (Dz * expert_bytes))))
            while len(zcopies) < copies - 1:
                zcopies.append(clone_weights())
            lays = [base] + [fp8.MoELayer(c, zri.w_router.to(dev), zs.k, zb) for c in zcopies[:copies - 1]]
            zout = torch.empty((64, d), dtype=torch.float32, device=dev)
            for i in range(args.warmup):
                lays[i % len(lays)].forward(zx, out=zout, topk_ids=zid)
            ev = HipEvents(2)
            torch.cuda.synchronize()
            ev.record(0, sh)
            for i in range(args.steps):
                lays[i % len(lays)].forward(zx, out=zout, topk_ids=zid)
            ev.record(1, sh)
            torch.cuda.synchronize()
            zms = ev.elapsed_ms(0, 1) / args.steps
            ev.close()
            zbytes = Dz * expert_bytes + E * d * 4 + 2 * 64 * d * 4
            zipf.append({"alpha": alpha, "distinct_experts": Dz, "us": round(zms * 1e3, 1),
                         "hbm_frac": round(zbytes / (zms * 1e-3) / PEAK_HBM, 4), "weight_copies": len(lays)})
            log(f"zipf alpha={alpha}: {zipf[-1]}")

    # ---- CPU oracle on a bounded sample (same inputs), plus a parity check
    cpu = None
    parity = None
    if want_cpu:
        import oracle
        t0 = time.time()
        qw = oracle.quantize_weights(host32["w_gate"], host32["w_up"], host32["w_down"],
                                     host32.get("ws_gate"), host32.get("ws_up"), host32.get("ws_down"))
        del host32
        log(f"oracle weights quantised in {time.time() - t0:.1f}s")
        cores = len(os.sched_getaffinity(0))
        xs_all = x.cpu().numpy()
        ks_all = None if kpt is None else kpt.cpu().numpy()
        bias_np = None if ri.router_bias is None else ri.router_bias.numpy()

        def run_oracle(n, nthreads=cores):
            ks = None if ks_all is None else ks_all[:n]
            return oracle.forward(xs_all[:n], qw, spec.k, w_router=ri.w_router.numpy(),
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
        parity = {"rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
                  "ids_equal": bool(np.array_equal(ids_np[:n], ido)), "tokens": n}
        log(f"oracle: {n} tokens x{reps} in {wall:.1f}s on {cores} cores; parity {parity}")

    res = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" + ("" if not args.no_requant else "+fp32_intermediate"),
        "data": "synthetic",
        "config": {"workload": f"{cfg}-shaped W8A8 FP8 MoE layer forward, batch T={T}", "T": T,
                   "d": d, "f": f, "E": E, "n_shared": S, "k": spec.k, "block_m": 16,
                   "requant": not args.no_requant, "distinct_experts": D,
                   "router_bias": spec.bias if spec.bias_param else "none",
                   "bias_param": spec.bias_param, "weight_copies": len(layers)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layer": {"alg_bytes": layer_bytes, "hbm_frac": round(layer_bytes / (ms * 1e-3) / PEAK_HBM, 4),
                  "fp8_flops": flops, "mfma_frac": round(flops / (ms * 1e-3) / PEAK_FP8, 5)},
        "step_us": step_us,
        "stages_us": stages_us,
        **({"graph": graph} if graph else {}),
        "parity": parity,
    }
    if sweep:
        res["sweep"] = sweep
    if zipf:
        res["zipf_sweep"] = zipf
    if grouping is not None:
        res["grouping"] = grouping
    if tiers is not None:
        res["tiers"] = tiers
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
