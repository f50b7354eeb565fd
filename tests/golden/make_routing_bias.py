"""Calibrate the router biases that shape the synthetic expert load.

Writes tests/golden/routing_bias.json, which workloads.py reads.  Only the
CPU oracle's router and top-k compute the routing here; the inputs are the
seeded draws of workloads.py.

- DeepSeek-MoE-16B-shaped layer (d=2048, E=64, k=6): one seeded hot expert
  e* gets a logit bias beta, chosen per batch size T so that e* receives
  exactly round(4 * T * k / E) tokens -- four times the mean load of an
  expert (12 / 192 / 3072 tokens at T = 32 / 512 / 8192).  A batch of T
  tokens is the first T rows of the 8192-token draw.  count(beta) is a
  non-decreasing step function, so bisection finds the interval of beta
  with the target count and beta is placed at its middle (robust to a few
  ulps of difference in the logits).
- Qwen3-30B-A3B-shaped layer (d=2048, E=128, k=8, T=64 of the 4096-token
  draw): the Zipf(s=1.1) offset b_e = alpha * ln p_pi(e) with alpha bisected
  so that the batch activates D distinct experts, D in {16, 32, 64, 96}
  (alpha = 0 gives about 126).  D(alpha) is non-increasing up to rare
  steps, so bisection keeps the alpha nearest the target.

Run: python tests/golden/make_routing_bias.py
"""
from __future__ import annotations

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as wl  # noqa: E402

OUT = os.path.join(HERE, "routing_bias.json")
SEED = 0


def hot_count(x, wr, hot, E, k, beta):
    b = np.zeros(E, np.float32)
    b[hot] = beta
    ids, _ = oracle.route_topk(oracle.router_logits(x, wr, b), k)
    return int((ids == hot).sum())


def calibrate_hot(T, target):
    spec = wl.DEEPSEEK.with_(T=wl.DEEPSEEK_T[-1], bias="none")
    ri = wl.routing_inputs(spec, SEED)
    x = ri.x[:T].numpy()
    wr = ri.w_router.numpy()
    hot = wl.hot_expert_index(spec, SEED)
    count = lambda beta: hot_count(x, wr, hot, spec.E, spec.k, beta)
    lo_b, hi_b = 0.0, 16.0
    assert count(lo_b) <= target <= count(hi_b)

    def first_reaching(c):  # smallest beta (to 1e-6) with count >= c
        lo, hi = lo_b, hi_b
        while hi - lo > 1e-6:
            mid = 0.5 * (lo + hi)
            if count(mid) >= c:
                hi = mid
            else:
                lo = mid
        return hi

    a = first_reaching(target)
    b = first_reaching(target + 1) if target < T else hi_b
    beta = float(np.float32(0.5 * (a + b)))
    got = count(beta)
    assert got == target, (T, target, got)
    return {"hot_expert": hot, "beta": beta, "hot_tokens": got, "target": target,
            "beta_interval": [a, b]}


def distinct(x, wr, E, k, alpha):
    spec = wl.QWEN3.with_(T=x.shape[0], bias_param=alpha)
    b = wl.zipf_bias(spec, SEED)
    ids, _ = oracle.route_topk(oracle.router_logits(x, wr, None if b is None else b.numpy()), k)
    return int(len(np.unique(ids[ids >= 0])))


def calibrate_zipf(T, target):
    spec = wl.QWEN3.with_(T=wl.QWEN3_T[-1])
    ri = wl.routing_inputs(spec.with_(bias_param=0.0), SEED)
    x = ri.x[:T].numpy()
    wr = ri.w_router.numpy()
    D = lambda a: distinct(x, wr, spec.E, spec.k, a)
    lo, hi = 0.0, 8.0
    best = (abs(D(lo) - target), lo)
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        dm = D(mid)
        best = min(best, (abs(dm - target), mid))
        if dm == target:
            break
        if dm > target:
            lo = mid
        else:
            hi = mid
    alpha = float(np.float32(best[1]))
    return {"alpha": alpha, "distinct_experts": D(alpha), "target": target}


def main():
    spec = wl.DEEPSEEK
    res = {"seed": SEED, "deepseek_hot": {}, "qwen3_zipf": {}}
    for T in wl.DEEPSEEK_T:
        target = int(round(4 * T * spec.k / spec.E))
        res["deepseek_hot"][str(T)] = calibrate_hot(T, target)
        print("deepseek", T, res["deepseek_hot"][str(T)], flush=True)
    for D in wl.QWEN3_D_TARGETS:
        res["qwen3_zipf"][str(D)] = calibrate_zipf(wl.QWEN3_T[0], D)
        print("qwen3", D, res["qwen3_zipf"][str(D)], flush=True)
    with open(OUT, "w") as fh:
        json.dump(res, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
