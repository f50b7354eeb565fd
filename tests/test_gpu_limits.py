"""The fused layer at the limits the boundary accepts (include/fp8moe.h):
the widest layer (d = MOE_MAX_HIDDEN = f = MOE_MAX_FFN = 16384, with a shared
expert), and the most experts and slots per token (E = MOE_MAX_EXPERTS = 512,
k = MOE_MAX_K = 32, per-token k) at a decode-sized and at a tiled-router batch.
Every token against the oracle, routing bit for bit, as in test_gpu_layer."""
import pytest
import torch

import workloads as wl
from gpu_common import Layer
from test_gpu_layer import _check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LIMITS = {
    # one wave per (expert, 2048-float part) of the decode router: 2 experts x 8 parts
    "max-width": wl.TINY.with_(T=5, d=16384, f=16384, E=2, k=2, n_shared=1),
    "max-experts-decode": wl.TINY.with_(T=3, d=256, f=192, E=512, k=32, k_choices=(4, 8, 16, 32)),
    # 300 x 512 (token, expert) pairs: the tiled router over four blocks of 128 experts
    "max-experts-tiled": wl.TINY.with_(T=300, d=256, f=128, E=512, k=32, k_choices=(1, 7, 32)),
}


@pytest.fixture(scope="module", params=list(LIMITS))
def limit_layer(request):
    return Layer(LIMITS[request.param])


@pytest.mark.parametrize("no_requant", [False, True])
def test_layer_at_the_boundary_limits(limit_layer, no_requant):
    err, worst = _check(limit_layer, no_requant=no_requant)
    print(f"{limit_layer.spec.name} d={limit_layer.spec.d} f={limit_layer.spec.f} "
          f"E={limit_layer.spec.E} k={limit_layer.spec.k}: rel-L2 {err:.3e}, worst token {worst:.3e}")
