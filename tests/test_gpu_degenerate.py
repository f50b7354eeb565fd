"""Degenerate layers through the fused forward, every token against the
oracle, routing bit for bit (as in test_gpu_layer):

- one expert (E = k = 1): the softmax over one pick is 1, so the layer is a
  dense SiLU-gated FFN, with and without a shared expert;
- every expert (k = E), with a shared expert;
- tokens whose activations are all zero: their |x| maximum is 0, so the
  activation quantiser and the requantisation of h take their unit-scale
  branch, the router's logits are all equal (picks 0 .. k-1, weights 1/k),
  and the token's output is exactly 0; every other token, then the whole
  batch.
"""
import pytest
import torch

import workloads as wl
from gpu_common import Layer
from test_gpu_layer import _check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEGENERATE = {
    "one-expert": wl.TINY.with_(T=33, d=256, f=192, E=1, k=1),
    "one-expert-shared": wl.TINY.with_(T=33, d=256, f=192, E=1, k=1, n_shared=1),
    "every-expert": wl.TINY.with_(T=50, d=256, f=192, E=8, k=8, n_shared=1),
}


@pytest.fixture(scope="module", params=list(DEGENERATE))
def deg(request):
    return Layer(DEGENERATE[request.param])


@pytest.mark.parametrize("no_requant", [False, True])
def test_degenerate_layer_every_token(deg, no_requant):
    err, worst = _check(deg, no_requant=no_requant)
    print(f"{deg.spec.name} E={deg.spec.E} k={deg.spec.k}: rel-L2 {err:.3e}, worst {worst:.3e}")


@pytest.mark.parametrize("rows", ["every-other", "all"])
@pytest.mark.parametrize("no_requant", [False, True])
def test_zero_tokens(deg, rows, no_requant):
    x0 = deg.x.clone()
    zero = slice(None, None, 2) if rows == "every-other" else slice(None)
    try:
        deg.x[zero] = 0.0
        _check(deg, no_requant=no_requant)
        out = deg.layer(no_requant=no_requant).forward(deg.x)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out[zero]).item() == 0
        if rows == "every-other":
            assert torch.count_nonzero(out[1::2]).item() > 0
    finally:
        deg.x.copy_(x0)
