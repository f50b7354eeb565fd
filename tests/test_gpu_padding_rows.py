"""Expert-segment padding rows are never read.

Each expert's rows are padded to a multiple of block_m ("Routage MoE entre
GPU": the tokens an expert receives are gathered into one contiguous
segment; the padding is this library's tile granularity).  The GEMM
epilogues store h, hq / hsc and y for the rows that hold a (token, slot) pair
only, so no later stage may read the padding rows' intermediates.  Filling
the whole workspace with 0xFF bytes before a forward puts NaN in every fp32,
fp16 and e4m3 slot and -1 in every index slot; a stage reading anything the
forward did not write itself would change the output (NaN times a zero scale
is still NaN).  The output must equal the one on a fresh workspace bit for
bit, on the row-pass, A-resident, prefill and fused-requantisation tiles,
with shared experts, per-token k, a ragged d, coarse padding (block_m 64) and
the no-requant accuracy mode.
"""
import pytest
import torch

import workloads as wl
from gpu_common import Layer, lib

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SPECS = {
    # row-pass tiles, separate requantisation
    "decode": wl.TINY.with_(T=37, d=512, f=512, E=8, k=2),
    # shared experts (rows past the routed capacity)
    "shared": wl.TINY.with_(T=40, d=512, f=256, E=8, k=2, n_shared=2),
    # fused requantisation (f <= 192), per-token k, A-resident down projection
    "rq-elastic": wl.TINY.with_(T=77, d=256, f=192, E=64, k=32, k_choices=(4, 8, 16, 32)),
    # 256-row passes (prefill tile)
    "prefill": wl.TINY.with_(T=2048, d=256, f=256, E=8, k=2),
    # ragged d (a 64-byte K tail), a shared expert
    "ragged-d": wl.TINY.with_(T=33, d=320, f=512, E=16, k=6, n_shared=1),
}


@pytest.fixture(scope="module", params=list(SPECS))
def layer(request):
    return Layer(SPECS[request.param], want_oracle=False)


@pytest.mark.parametrize("block_m", [16, 64])
@pytest.mark.parametrize("no_requant", [False, True])
def test_padding_rows_never_read(layer, block_m, no_requant):
    spec = layer.spec
    m = lib().MoELayer(layer.dw, layer.w_router, spec.k, layer.bias, block_m, no_requant, False)
    kpt = layer.kpt
    ref = m.forward(layer.x, k_per_token=kpt).clone()
    ws = m.workspace(spec.T, layer.x.device)
    ws.fill_(0xFF)
    out = m.forward(layer.x, k_per_token=kpt)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    assert torch.equal(out, ref), f"max |diff| {(out - ref).abs().max().item():.3e}"
