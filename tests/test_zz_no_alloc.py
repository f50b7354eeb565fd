"""moe_fused_forward_noalloc (workspace in the library's static device array)
against moe_fused_forward (caller workspace): two calls in a row, the second
with a smaller batch, must give the same outputs and routing, bit for bit
(the same kernels run on the same plan; only the workspace's address
differs), and stay within the oracle's bar."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_common import Layer, dev, lib, rel_l2, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = {
    "tiny-shared": (wl.TINY.with_(T=40, d=256, f=192, E=8, k=2, n_shared=2), (40, 17)),
    "tiny-elastic": (wl.TINY.with_(T=77, d=256, f=192, E=64, k=32, k_choices=(4, 8, 16, 32)),
                     (77, 9)),
    "mixtral-decode": (wl.MIXTRAL, (256, 8)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_caller_workspace(name):
    spec, batches = CASES[name]
    L = Layer(spec, want_oracle=name != "mixtral-decode")
    layer = L.layer()
    for T in batches:
        x = L.x[:T].contiguous()
        kpt = None if L.kpt is None else L.kpt[:T].contiguous()
        ids_a = torch.empty((T, spec.k), dtype=torch.int32, device=dev())
        ids_b = torch.full_like(ids_a, -7)
        w_a = torch.empty((T, spec.k), dtype=torch.float32, device=dev())
        w_b = torch.full_like(w_a, -7.0)
        a = layer.forward(x, k_per_token=kpt, topk_ids=ids_a, topk_w=w_a)
        b = torch.full_like(a, float("nan"))
        layer.forward_noalloc(x, b, k_per_token=kpt, topk_ids=ids_b, topk_w=w_b)
        torch.cuda.synchronize()
        assert torch.equal(ids_a, ids_b) and torch.equal(w_a, w_b)
        assert torch.equal(a, b), f"{name} T={T}: max diff {(a - b).abs().max().item()}"
        if L.qw is not None:
            lo = to_np(lib().router_logits(x, L.w_router, L.bias))
            ref, ido, _ = oracle.forward(to_np(x), L.qw, spec.k, logits_override=lo,
                                         k_per_token=None if kpt is None else to_np(kpt))
            np.testing.assert_array_equal(to_np(ids_b), ido)
            assert rel_l2(to_np(b), ref) <= 2e-2
        print(f"{name} T={T}: no-alloc == caller workspace")


def test_noalloc_refuses_dims_beyond_the_static_array():
    spec = wl.TINY.with_(T=40, d=256, f=192, E=8, k=2)
    L = Layer(spec, want_oracle=False)
    layer = L.layer()
    # a batch whose workspace exceeds the array: refused, nothing enqueued
    T = 1
    while lib().workspace_bytes(layer.dims(T)) <= lib().STATIC_WORKSPACE_BYTES:
        T *= 2
    x = torch.zeros((T, spec.d), dtype=torch.float32, device=dev())
    out = torch.full((T, spec.d), 3.0, dtype=torch.float32, device=dev())
    with pytest.raises(lib().MoEError) as ei:
        layer.forward_noalloc(x, out)
    assert "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
