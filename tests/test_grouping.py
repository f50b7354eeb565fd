"""Decode batching by expert affinity (moe_group_tokens): the oracle pinned to
cases whose answer is fixed without it, and the library's host
implementation bit-exact against the oracle.  Host code only (no GPU)."""
import itertools

import numpy as np
import pytest

from oracle import grouping as og


def _lib():
    return pytest.importorskip("fp8_moe_layer_amd")


def _zipf_pool(n, k, E, alpha, seed):
    """Routing of a pool: each token draws k distinct experts with
    probabilities proportional to rank^-alpha over a seeded expert order."""
    rng = np.random.default_rng(seed)
    p = np.arange(1, E + 1, dtype=np.float64) ** -alpha
    p = p[rng.permutation(E)]
    p /= p.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(n)]).astype(np.int32)


# ---------------------------------------------------------------- oracle pins

def test_oracle_order_is_a_permutation_in_batches():
    ids = _zipf_pool(70, 4, 32, 1.0, 0)
    order = og.group_tokens(ids, 16)
    assert sorted(order.tolist()) == list(range(70))
    assert og.distinct_per_batch(ids, order, 16)[-1] <= 24  # the last batch holds 6 tokens


def test_oracle_separates_disjoint_clusters():
    # token t uses the expert pair {0,1}, {5,6}, {2,3} or {7,4} by t % 4, the
    # four pairs interleaved in arrival order: arrival batches of 8 see all 8
    # experts; the optimum (8 tokens of one pair per batch) sees 2
    ids = np.array([[(t % 2) * 4 + j for j in (t % 4, (t + 1) % 4)] for t in range(32)], np.int32)
    order = og.group_tokens(ids, 8)
    assert og.distinct_per_batch(ids, np.arange(32), 8) == [8, 8, 8, 8]
    assert og.distinct_per_batch(ids, order, 8) == [2, 2, 2, 2]
    for b in range(4):
        assert len({int(t) % 4 for t in order[b * 8:(b + 1) * 8]}) == 1


def test_oracle_single_batch_and_identical_tokens():
    ids = _zipf_pool(20, 3, 16, 0.0, 1)
    assert og.group_tokens(ids, 20).tolist()[0] == 0  # one batch starts at token 0
    same = np.tile(np.array([[3, 5]], np.int32), (9, 1))
    assert og.group_tokens(same, 4).tolist() == list(range(9))  # all ties: arrival order


def test_oracle_invariant_under_expert_relabelling():
    ids = _zipf_pool(60, 4, 24, 1.2, 2)
    perm = np.random.default_rng(3).permutation(24).astype(np.int32)
    assert np.array_equal(og.group_tokens(ids, 8), og.group_tokens(perm[ids], 8))


def test_oracle_greedy_against_exhaustive_on_tiny_pools():
    # every partition of 6 tokens into 2 batches of 3: the greedy's total is
    # never below the optimum and reaches it where one partition is clearly
    # best (two clusters)
    rng = np.random.default_rng(4)
    for trial in range(20):
        ids = rng.integers(0, 6, size=(6, 2)).astype(np.int32)
        order = og.group_tokens(ids, 3)
        greedy = sum(og.distinct_per_batch(ids, order, 3))
        best = min(sum(og.distinct_per_batch(ids, np.array(list(a) + [t for t in range(6) if t not in a]), 3))
                   for a in itertools.combinations(range(6), 3))
        assert best <= greedy <= best + 2
    clusters = np.array([[0, 1], [2, 3], [0, 1], [2, 3], [1, 0], [3, 2]], np.int32)
    order = og.group_tokens(clusters, 3)
    assert sum(og.distinct_per_batch(clusters, order, 3)) == 4


def test_oracle_never_worse_than_arrival_on_skewed_pools():
    for seed, alpha in ((5, 0.8), (6, 1.5)):
        ids = _zipf_pool(256, 8, 128, alpha, seed)
        order = og.group_tokens(ids, 64)
        assert sum(og.distinct_per_batch(ids, order, 64)) < sum(og.distinct_per_batch(ids, np.arange(256), 64))


# ---------------------------------------------------------------- library vs oracle (host code)

@pytest.mark.parametrize("n,k,E,alpha,batch", [(64, 8, 128, 0.0, 16), (200, 8, 128, 1.5, 64),
                                               (97, 6, 64, 1.0, 32), (33, 2, 8, 0.0, 5),
                                               (130, 4, 512, 1.1, 64)])
def test_library_matches_oracle(n, k, E, alpha, batch):
    m = _lib()
    ids = _zipf_pool(n, k, E, alpha, n + k)
    assert np.array_equal(m.group_tokens(ids, E, batch), og.group_tokens(ids, batch))


def test_library_matches_oracle_with_empty_slots_and_repeats():
    m = _lib()
    rng = np.random.default_rng(9)
    ids = rng.integers(-1, 16, size=(80, 6)).astype(np.int32)  # -1 slots, repeated ids
    ids[5] = -1  # a token with no experts
    for batch in (1, 7, 80, 200):
        assert np.array_equal(m.group_tokens(ids, 16, batch), og.group_tokens(ids, batch))


def test_library_rejects_bad_arguments():
    m = _lib()
    ids = np.zeros((4, 2), np.int32)
    with pytest.raises(m.MoEError):
        m.group_tokens(ids, 8, 0)
    with pytest.raises(m.MoEError):
        m.group_tokens(np.full((4, 2), 8, np.int32), 8, 2)  # id outside [-1, E)
    assert m.group_tokens(np.zeros((0, 2), np.int32), 8, 4).size == 0
