"""Quality-tier batching by routing budget (moe_k_tiers): the oracle pinned to
a worked example and to closed forms at the rule's extremes, and the library's
host implementation equal to the oracle's plan.  Host code only (no GPU)."""
import math

import numpy as np
import pytest

from oracle import grouping as og


def _lib():
    return pytest.importorskip("fp8_moe_layer_amd")


def _budgets(n, choices, seed):
    rng = np.random.default_rng(seed)
    return rng.choice(np.asarray(choices, np.int32), size=n).astype(np.int32)


def _check_plan(kpt, batch, plan):
    """Every token once; none served below its budget; batches at most
    `batch` long, each at one k, in ascending k."""
    toks = [t for _, b in plan for t in b]
    assert sorted(toks) == list(range(len(kpt)))
    ks = [k for k, _ in plan]
    assert ks == sorted(ks)
    for k, b in plan:
        assert 1 <= len(b) <= batch
        assert all(kpt[t] <= k for t in b)


# ---------------------------------------------------------------- oracle pins

def test_oracle_worked_example():
    # budgets 4,4,4,8,8,16 in batches of 2.  Overhead 10: tier 4 leaves token 2
    # (alone 10+4 = 14 pairs, merged 8) -> merged; tier 8's pool {2,3,4}
    # leaves token 4 (alone 18, merged 16) -> merged; tier 16 runs {4,5}.
    kpt = [4, 4, 4, 8, 8, 16]
    assert og.k_tiers(kpt, 2, 10) == [(4, [0, 1]), (8, [2, 3]), (16, [4, 5])]
    # overhead 3: token 2 alone costs 7 < 8 -> dispatched short; tier 8 is
    # {3,4}; token 5 is the last tier's residual
    assert og.k_tiers(kpt, 2, 3) == [(4, [0, 1]), (4, [2]), (8, [3, 4]), (16, [5])]
    # overhead 4: alone 8 == merged 8 -> a tie is dispatched (no over-service)
    assert og.k_tiers(kpt, 2, 4) == [(4, [0, 1]), (4, [2]), (8, [3, 4]), (16, [5])]


def test_oracle_single_budget_is_arrival_batches():
    kpt = [8] * 11
    assert og.k_tiers(kpt, 4, 1000) == [(8, [0, 1, 2, 3]), (8, [4, 5, 6, 7]), (8, [8, 9, 10])]


def test_oracle_zero_overhead_never_over_serves():
    kpt = _budgets(301, (4, 8, 16, 32), 0)
    plan = og.k_tiers(kpt, 64, 0)
    _check_plan(kpt, 64, plan)
    assert all(kpt[t] == k for k, b in plan for t in b)
    sizes = np.bincount(kpt)
    assert len(plan) == sum(math.ceil(c / 64) for c in sizes if c)


def test_oracle_large_overhead_fills_every_batch_but_the_last():
    kpt = _budgets(301, (4, 8, 16, 32), 1)
    plan = og.k_tiers(kpt, 64, 10 ** 9)
    _check_plan(kpt, 64, plan)
    assert len(plan) == math.ceil(301 / 64)
    assert all(len(b) == 64 for _, b in plan[:-1])
    # over-service comes from carried residuals only: fewer than one batch per tier step
    over = sum(1 for k, b in plan for t in b if kpt[t] < k)
    assert 0 < over < 64 * 3


def test_oracle_tier_sizes_multiple_of_batch_need_no_merge():
    kpt = np.repeat(np.array([2, 4, 32], np.int32), [32, 16, 48])
    plan = og.k_tiers(np.random.default_rng(2).permutation(kpt), 16, 10 ** 6)
    assert [k for k, _ in plan] == [2, 2, 4, 32, 32, 32]
    assert all(len(b) == 16 for _, b in plan)


# ---------------------------------------------------------------- library vs oracle (host code)

def _plan_of(m, kpt, batch, overhead):
    order, start, bk = m.k_tiers(kpt, batch, overhead)
    return [(int(bk[b]), order[start[b]:start[b + 1]].tolist()) for b in range(len(bk))]


@pytest.mark.parametrize("n,choices,batch,overhead", [
    (1024, (4, 8, 16, 32), 256, 1024), (1024, (4, 8, 16, 32), 128, 0),
    (1000, (4, 8, 16, 32), 64, 10 ** 9), (97, (1, 2, 3, 5, 7, 32), 8, 20),
    (5, (1, 32), 16, 100), (64, (6,), 16, 5)])
def test_library_matches_oracle(n, choices, batch, overhead):
    m = _lib()
    kpt = _budgets(n, choices, n + batch)
    plan = _plan_of(m, kpt, batch, overhead)
    assert plan == og.k_tiers(kpt, batch, overhead)
    _check_plan(kpt, batch, plan)


def test_library_worked_example_and_empty_pool():
    m = _lib()
    assert _plan_of(m, np.array([4, 4, 4, 8, 8, 16], np.int32), 2, 10) == \
        [(4, [0, 1]), (8, [2, 3]), (16, [4, 5])]
    order, start, bk = m.k_tiers(np.zeros(0, np.int32), 4, 0)
    assert order.size == 0 and start.tolist() == [0] and bk.size == 0


def test_library_rejects_bad_arguments():
    m = _lib()
    ok = np.array([4, 8], np.int32)
    for kpt, batch, overhead in ((ok, 0, 0), (ok, 4, -1), (np.array([0, 4], np.int32), 4, 0),
                                 (np.array([33], np.int32), 4, 0)):
        with pytest.raises(m.MoEError):
            m.k_tiers(kpt, batch, overhead)
