"""Benchmark: the fused W8A8 FP8 MoE layer forward on one MI355X.

Workload (default): the Mixtral-8x7B-shaped layer -- d=4096, f=14336, E=8,
top-2, W8A8 e4m3 with per-output-channel weight scales and per-token
activation scales -- at the largest batch of its decode sweep, T=256 tokens,
unbiased router (near-uniform expert load).  Inputs are seeded synthetic
draws (workloads.py); the weights are drawn on the GPU in fp32 and quantised
by the library's own e4m3 quantiser.

One step = one whole layer forward (quantise, router, top-k, permutation,
gate/up + SiLU*up, requantisation, down projection, combine) with inputs
already resident in HBM.  W untimed warm-up steps, then K steps timed with
HIP events on the stream the library launches on.  A second pass of K steps
records per-stage events (moe_debug_stage_events) to time the dominant
kernel (gate/up grouped GEMM) for the roofline figure.  The CPU oracle is
timed on a bounded sample of the same workload on the host cores.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes as C
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--tokens", type=int, default=256)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=48, help="tokens the oracle recomputes")
    p.add_argument("--sweep", action="store_true", help="also time T in 1,8,32,128,256")
    p.add_argument("--no-requant", action="store_true")
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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py runs on one GPU only: this build measures the layer on a single MI355X "
              "(no sharding, no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_moe_layer_amd as fp8
    import workloads as wl

    dev = torch.device("cuda", 0)
    spec = wl.MIXTRAL.with_(T=max(args.tokens, 256 if args.sweep else args.tokens))
    T = args.tokens
    want_cpu = not args.no_cpu_baseline
    log(f"workload mixtral-shaped d={spec.d} f={spec.f} E={spec.E} k={spec.k} T={T}")

    # ---- inputs: routing on the CPU generator, expert weights drawn on the GPU
    ri = wl.routing_inputs(spec, args.seed)
    x_all = ri.x.to(dev)
    w_router = ri.w_router.to(dev)
    dw = fp8.DeviceWeights.empty(spec.E, spec.d, spec.f, 0, device=dev)
    host32 = {}
    if want_cpu:
        host32 = {k: np.empty(s, np.float32) for k, s in
                  (("gate", (spec.E, spec.f, spec.d)), ("up", (spec.E, spec.f, spec.d)),
                   ("down", (spec.E, spec.d, spec.f)))}
    t0 = time.time()
    for e in range(spec.E):
        for which in ("gate", "up", "down"):
            w32 = wl.expert_weight(spec, which, e, args.seed, dev)
            dw.set_expert(which, e, w32)
            if want_cpu:
                host32[which][e] = w32.cpu().numpy()
            del w32
    torch.cuda.synchronize()
    log(f"weights ready in {time.time() - t0:.1f}s")

    layer = fp8.MoELayer(dw, w_router, spec.k, no_requant=args.no_requant)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def time_layer(Tn, steps, warmup):
        x = x_all[:Tn].contiguous()
        out = torch.empty((Tn, spec.d), dtype=torch.float32, device=dev)
        ids = torch.empty((Tn, spec.k), dtype=torch.int32, device=dev)
        for _ in range(warmup):
            layer.forward(x, out=out, topk_ids=ids)
        torch.cuda.synchronize()
        ev = HipEvents(2)
        ev.record(0, sh)
        for _ in range(steps):
            layer.forward(x, out=out, topk_ids=ids)
        ev.record(1, sh)
        torch.cuda.synchronize()
        ms = ev.elapsed_ms(0, 1) / steps
        ev.close()
        return ms, x, out, ids

    # ---- headline timing
    ms, x, out, ids = time_layer(T, args.steps, args.warmup)
    tokens_per_s = T / (ms * 1e-3)
    log(f"T={T}: {ms * 1e3:.1f} us/step, {tokens_per_s:.4g} tokens/s")

    # ---- per-stage timing (second pass, same inputs)
    nst = fp8.N_STAGE_EVENTS
    sev = HipEvents(nst * args.steps)
    stage_sum = [0.0] * (nst - 1)
    keep = []
    for s in range(args.steps):
        keep.append(fp8.set_stage_events(sev.ev[s * nst:(s + 1) * nst]))
        layer.forward(x, out=out, topk_ids=ids)
    fp8.set_stage_events(None)
    torch.cuda.synchronize()
    for s in range(args.steps):
        for i in range(nst - 1):
            stage_sum[i] += sev.elapsed_ms(s * nst + i, s * nst + i + 1)
    sev.close()
    stages_us = {name: round(v / args.steps * 1e3, 2) for name, v in zip(fp8.STAGES, stage_sum)}
    log(f"stages (us): {stages_us}")

    # ---- algorithmic bytes / flops (distinct active experts from this step's routing)
    ids_np = ids.cpu().numpy()
    D = int(len(np.unique(ids_np[ids_np >= 0])))
    P = int((ids_np >= 0).sum())
    d, f, E = spec.d, spec.f, spec.E
    gate_up_bytes = D * 2 * f * (d + 4) + T * (d + 4) + P * f * 4
    layer_bytes = D * (3 * f * d + 8 * f + 4 * d) + E * d * 4 + 2 * T * d * 4
    flops = 2 * P * 3 * f * d
    t_gu = stages_us["gate_up"] * 1e-6
    gu_achieved = gate_up_bytes / t_gu
    roofline = {"bound": "hbm", "achieved": round(gu_achieved / 1e9, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(gu_achieved / PEAK_HBM, 4), "traffic": None,
                "kernel": "gate_up_kernel", "alg_bytes_per_launch": gate_up_bytes,
                "avg_launch_us": stages_us["gate_up"]}
    layer_hbm = layer_bytes / (ms * 1e-3)

    # ---- sweep over the decode batch sizes (same weights)
    sweep = None
    if args.sweep:
        sweep = {}
        for Tn in wl.MIXTRAL_DECODE_T:
            mst, _, _, idt = time_layer(Tn, args.steps, args.warmup)
            it = idt.cpu().numpy()
            Dn = int(len(np.unique(it[it >= 0])))
            lb = Dn * (3 * f * d + 8 * f + 4 * d) + E * d * 4 + 2 * Tn * d * 4
            sweep[str(Tn)] = {"us": round(mst * 1e3, 1), "tokens_per_s": round(Tn / (mst * 1e-3), 1),
                              "distinct_experts": Dn, "hbm_frac": round(lb / (mst * 1e-3) / PEAK_HBM, 4)}
            log(f"sweep T={Tn}: {sweep[str(Tn)]}")

    # ---- CPU oracle on a bounded sample (same inputs), plus a parity check
    cpu = None
    parity = None
    if want_cpu:
        import oracle
        t0 = time.time()
        qw = oracle.quantize_weights(host32["gate"], host32["up"], host32["down"])
        del host32
        log(f"oracle weights quantised in {time.time() - t0:.1f}s")
        S = min(args.cpu_sample, T)
        xs = x[:S].cpu().numpy()
        cores = len(os.sched_getaffinity(0))
        t0 = time.time()
        ref, ido, _ = oracle.forward(xs, qw, spec.k, w_router=ri.w_router.numpy(), nthreads=cores)
        wall = time.time() - t0
        cpu = {"value": round(S / wall, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"first {S} of the {T} tokens, full layer incl. router (oracle quantises "
                         f"its own weights beforehand, untimed)", "seconds": round(wall, 2)}
        got = out[:S].cpu().numpy().astype(np.float64)
        parity = {"rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
                  "ids_equal": bool(np.array_equal(ids_np[:S], ido)), "tokens": S}
        log(f"oracle: {S} tokens in {wall:.1f}s on {cores} cores; parity {parity}")

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
        "config": {"workload": f"mixtral-8x7b-shaped MoE layer, decode batch T={T}", "T": T,
                   "d": d, "f": f, "E": E, "k": spec.k, "block_m": 16,
                   "requant": not args.no_requant, "distinct_experts": D},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layer": {"alg_bytes": layer_bytes, "hbm_frac": round(layer_hbm / PEAK_HBM, 4),
                  "fp8_flops": flops, "mfma_frac": round(flops / (ms * 1e-3) / PEAK_FP8, 5)},
        "stages_us": stages_us,
        "parity": parity,
    }
    if sweep:
        res["sweep"] = sweep
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
