"""Quality-tier batches by routing budget (moe_k_tiers) run through the fused
layer: each batch at its one k, tokens of merged residuals served at the next
tier's k.  Every token's output must match the oracle's layer at the k the
plan serves it at (on the same logits), and the plan must be the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_common import Layer, dev, lib, rel_l2, to_np
from oracle import grouping as og

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_REQUANT = 2e-2


@pytest.mark.parametrize("batch,overhead", [(16, 48), (16, 0), (32, 10 ** 6)])
def test_tiered_batches_match_oracle_at_served_k(batch, overhead):
    spec = wl.TINY.with_(T=96, d=256, f=192, E=64, k=8, k_choices=(1, 2, 4, 8))
    L = Layer(spec)
    m = lib()
    kpt = to_np(L.kpt)
    order, start, bk = m.k_tiers(kpt, batch, overhead)
    plan = [(int(bk[b]), order[start[b]:start[b + 1]].tolist()) for b in range(len(bk))]
    assert plan == og.k_tiers(kpt, batch, overhead)
    served = np.empty(spec.T, np.int32)
    logits = np.empty((spec.T, spec.E), np.float32)
    out = torch.empty((spec.T, spec.d), dtype=torch.float32, device=dev())
    layers = {}
    for k, toks in plan:
        if k not in layers:
            layers[k] = m.MoELayer(L.dw, L.w_router, k, L.bias)
        sel = torch.as_tensor(toks, device=dev(), dtype=torch.long)
        xb = L.x[sel].contiguous()
        lg = m.router_logits(xb, L.w_router, L.bias)
        out[sel] = layers[k].forward(xb, logits_override=lg)
        served[toks] = k
        logits[toks] = to_np(lg)
    torch.cuda.synchronize()
    assert np.all(served >= kpt)
    if overhead == 0:
        assert np.array_equal(served, kpt)
    elif overhead >= 48:
        assert np.any(served > kpt)  # some residuals were merged upward
    ref, _, _ = oracle.forward(to_np(L.x), L.qw, spec.k, logits_override=logits, k_per_token=served)
    err = rel_l2(to_np(out), ref)
    assert err <= TOL_REQUANT, f"rel-L2 {err:.3e} > {TOL_REQUANT}"
