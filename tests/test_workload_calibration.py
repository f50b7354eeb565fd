"""The synthetic expert loads are the ones the layer shapes state.

- DeepSeek-MoE-16B shape: the hottest expert receives 4x the mean token
  count, i.e. round(4*T*k/E) = 12 / 192 / 3072 tokens at T = 32 / 512 / 8192,
  with the calibrated hot-expert bias of tests/golden/routing_bias.json, and
  no other expert receives more.
- Qwen3-30B-A3B shape at T=64: the calibrated Zipf offsets make the batch
  activate 16 / 32 / 64 / 96 distinct experts; with no offset about 126.

The routing here is the CPU oracle's (router logits, then top-k).
"""
import numpy as np
import pytest

import oracle
import workloads as wl


def _ids(spec, T):
    ri = wl.routing_inputs(spec.with_(T=max(T, spec.T)), 0)
    b = None if ri.router_bias is None else ri.router_bias.numpy()
    lg = oracle.router_logits(ri.x[:T].numpy(), ri.w_router.numpy(), b)
    ids, _ = oracle.route_topk(lg, spec.k)
    return ids


@pytest.mark.parametrize("T", wl.DEEPSEEK_T)
def test_deepseek_hot_expert_is_four_times_the_mean(T):
    spec = wl.deepseek_spec(T)
    ids = _ids(spec.with_(T=wl.DEEPSEEK_T[-1]), T)
    counts = np.bincount(ids[ids >= 0], minlength=spec.E)
    hot = wl.hot_expert_index(spec, 0)
    target = wl.deepseek_hot_target(T)
    assert target == {32: 12, 512: 192, 8192: 3072}[T]
    assert counts[hot] == target
    assert counts.sum() == T * spec.k
    assert counts[hot] == counts.max()
    # 4x the mean load of an expert
    assert abs(counts[hot] / (T * spec.k / spec.E) - 4.0) < 0.1


@pytest.mark.parametrize("D", wl.QWEN3_D_TARGETS)
def test_qwen3_zipf_distinct_experts(D):
    spec = wl.QWEN3.with_(T=wl.QWEN3_T[-1], bias_param=wl.qwen3_alpha(D))
    ids = _ids(spec, wl.QWEN3_T[0])
    assert len(np.unique(ids[ids >= 0])) == D


def test_qwen3_unbiased_activates_most_experts():
    ids = _ids(wl.QWEN3.with_(T=wl.QWEN3_T[-1], bias_param=0.0), wl.QWEN3_T[0])
    assert len(np.unique(ids[ids >= 0])) >= 120
