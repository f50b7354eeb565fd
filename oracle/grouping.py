"""Decode batching by expert affinity -- oracle, TEST INFRASTRUCTURE ONLY.

"ELDR : Microsoft et KAIST accélèrent le décodage des MoE": a decode step
loads the weights of every distinct expert its batch activates, so batches
whose tokens share experts cost less, and regrouping tokens changes no
token's output.  The grouping rule this package follows (its plain greedy
reading of that idea): each batch starts from the lowest-numbered unplaced
token, then repeatedly takes the unplaced token that adds the fewest experts
not yet in the batch, the lowest number winning ties.

Plain Python sets and loops, for pools of a few thousand tokens at most.
Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may use it; it shares no code with the library.
"""
from __future__ import annotations

import numpy as np


def token_experts(ids) -> list:
    """The set of experts of each token (empty slots are -1)."""
    return [set(int(e) for e in row if e >= 0) for row in np.asarray(ids)]


def group_tokens(ids, batch: int) -> np.ndarray:
    """Order of the tokens: batch b is order[b*batch:(b+1)*batch]."""
    experts = token_experts(ids)
    n = len(experts)
    placed = [False] * n
    order = []
    while len(order) < n:
        seed = next(t for t in range(n) if not placed[t])
        placed[seed] = True
        order.append(seed)
        have = set(experts[seed])
        filled = 1
        while filled < batch and len(order) < n:
            best, best_new = -1, None
            for t in range(n):
                if placed[t]:
                    continue
                new = len(experts[t] - have)
                if best_new is None or new < best_new:
                    best, best_new = t, new
            placed[best] = True
            order.append(best)
            have |= experts[best]
            filled += 1
    return np.asarray(order, dtype=np.int32)


def distinct_per_batch(ids, order, batch: int) -> list:
    """Distinct experts activated by each batch of an order."""
    experts = token_experts(ids)
    return [len(set().union(*(experts[t] for t in order[b:b + batch])))
            for b in range(0, len(order), batch)]


def k_tiers(k_per_token, batch: int, overhead: int):
    """Quality-tier batches by routing budget -- "MoE-Prism: Disentangling
    Monolithic Experts …", section Méthodologie B (offline, throughput-
    oriented mode): sort the requests by k, group them into tiers, and either
    dispatch a tier's residual batch at once or merge it into the next tier,
    which serves it at that tier's larger k.

    The package's reading of the pages' local throughput rule: r residual
    tokens of tier k cost one batch overhead plus r*k pairs when dispatched
    alone, and r*k_next pairs when merged; merging wins only when strictly
    cheaper.  Returns a list of (k, [tokens]) batches in dispatch order."""
    kpt = [int(v) for v in np.asarray(k_per_token).reshape(-1)]
    levels = sorted(set(kpt))
    batches = []
    carried = []
    for i, k in enumerate(levels):
        pool = carried + [t for t in range(len(kpt)) if kpt[t] == k]
        while len(pool) >= batch:
            batches.append((k, pool[:batch]))
            pool = pool[batch:]
        carried = []
        if not pool:
            continue
        r = len(pool)
        if i + 1 < len(levels) and r * levels[i + 1] < overhead + r * k:
            carried = pool
        else:
            batches.append((k, pool))
    return batches
