"""The device-checked debug build (libfp8moe_debug.so, FP8MOE_DEBUG) on the GPU.

On valid inputs it must give exactly the release library's outputs (the checks
only observe) and report no failed check.  On inputs outside the layer's
preconditions -- a k_per_token entry outside [1, k_max], a non-finite
activation, a top-k id outside [-1, E) -- it must return MOE_ERR_DEVICE_CHECK
naming the check.  Every such input is one the kernels turn into a safe value
(a clamped k, a dropped id, a saturated e4m3 code), so none of these runs reads
or writes out of bounds; they run on the debug build only."""
import pytest
import torch

import workloads as wl
from gpu_common import Layer, dev, lib

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ERR_DEVICE_CHECK = 7

SPECS = {
    "tiny-shared-elastic": wl.TINY.with_(T=48, d=256, f=192, E=16, k=4, n_shared=2,
                                         k_choices=(1, 2, 4)),
    "mid-routing": wl.TINY.with_(T=301, d=256, f=128, E=70, k=6, k_choices=(2, 4, 6)),
    "prefill-routing": wl.TINY.with_(T=1100, d=256, f=128, E=64, k=6, n_shared=1),
    "prism-small": wl.PRISM.with_(T=96, d=256, E=64),
}


def _debug():
    m = lib()
    if not m.DEBUG_LIB_PATH.exists():
        pytest.fail("libfp8moe_debug.so is not built (fp8_moe_layer_amd/build.py --debug)")
    return m.DebugLibrary()


@pytest.mark.parametrize("persistent", [False, True])
@pytest.mark.parametrize("name", list(SPECS))
def test_debug_build_matches_release(name, persistent):
    dbg = _debug()
    assert dbg.checks == 1
    L = Layer(SPECS[name], want_oracle=False)
    m = lib()
    layer = m.MoELayer(L.dw, L.w_router, L.spec.k, router_bias=L.bias, persistent=persistent)
    T = L.spec.T
    ids_r = torch.empty((T, L.spec.k), dtype=torch.int32, device=dev())
    ids_d = torch.empty_like(ids_r)
    ref = layer.forward(L.x, k_per_token=L.kpt, topk_ids=ids_r)
    torch.cuda.synchronize()
    rc, text, out = dbg.forward(layer, L.x, k_per_token=L.kpt, topk_ids=ids_d)
    torch.cuda.synchronize()
    assert rc == 0, text
    assert torch.equal(ids_d, ids_r)
    assert torch.equal(out, ref), "the debug build's output differs from the release library's"
    print(f"{name} persistent={persistent}: debug == release, no device check failed")


def test_debug_build_reports_k_per_token_out_of_range():
    dbg = _debug()
    spec = SPECS["tiny-shared-elastic"]
    L = Layer(spec, want_oracle=False)
    layer = lib().MoELayer(L.dw, L.w_router, spec.k)
    kpt = L.kpt.clone()
    kpt[3] = 0
    kpt[10] = spec.k + 1
    rc, text, _ = dbg.forward(layer, L.x, k_per_token=kpt)
    assert rc == ERR_DEVICE_CHECK, (rc, text)
    assert "k_per_token" in text
    # the word was cleared: the valid input passes again
    rc, text, _ = dbg.forward(layer, L.x, k_per_token=L.kpt)
    assert rc == 0, text


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_debug_build_reports_non_finite_input(bad):
    dbg = _debug()
    spec = SPECS["mid-routing"]
    L = Layer(spec, want_oracle=False)
    layer = lib().MoELayer(L.dw, L.w_router, spec.k)
    x = L.x.clone()
    x[17, 5] = bad
    rc, text, _ = dbg.forward(layer, x, k_per_token=L.kpt)
    assert rc == ERR_DEVICE_CHECK, (rc, text)
    assert "non-finite" in text


def test_debug_build_reports_bad_topk_ids_in_the_permutation():
    dbg = _debug()
    T, E, k = 40, 16, 4
    g = torch.Generator(device="cpu").manual_seed(3)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    ids[5, 3] = -1  # an empty slot is valid
    rc, text = dbg.permute(ids.to(dev()), E)
    assert rc == 0, text
    bad = ids.clone()
    bad[2, 1] = E + 3
    bad[7, 0] = -5
    rc, text = dbg.permute(bad.to(dev()), E)
    assert rc == ERR_DEVICE_CHECK, (rc, text)
    assert "top-k id" in text


def test_debug_build_reports_bad_k_in_the_topk_step():
    dbg = _debug()
    T, E, k = 64, 32, 4
    logits = torch.randn((T, E), generator=torch.Generator().manual_seed(5)).to(dev())
    kpt = torch.full((T,), 2, dtype=torch.int32, device=dev())
    rc, text, ids, _ = dbg.route_topk(logits, k, k_per_token=kpt)
    assert rc == 0, text
    assert (ids[:, 2:] == -1).all() and (ids[:, :2] >= 0).all()
    kpt[0] = -1
    rc, text, _, _ = dbg.route_topk(logits, k, k_per_token=kpt)
    assert rc == ERR_DEVICE_CHECK and "k_per_token" in text, (rc, text)
