"""moe_forward_noalloc: the whole chain with its intermediates in the
library's fixed device scratch, for callers that cannot allocate.  Through the
C ABI it must give moe_forward's result bit for bit (same kernels), on two
calls in a row on the same scratch, the second with a smaller input, for
bf16 and block-FP8 weights; and it must refuse a shape past the scratch."""
import pytest
import torch

import workloads
from gpu_helpers import log

import expert_layer_amd as moe
from expert_layer_amd.chain import Layer

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _layer(d, fp8):
    return Layer.from_weights(d["w1"], d["w3"], d["w2"], d["sw1"], d["sw3"], d["sw2"], fp8=fp8)


def _run(fn, layer, wl, d, T, ydt, ws=None):
    x = d["x"][:T].contiguous()
    logits = d["logits"][:T].contiguous()
    out = torch.full((T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
    kw = dict(logits=logits, bias=d["bias"], y_dtype=ydt, topk_ids=ids)
    if ws is None:
        fn(layer.experts, x, wl.k, out, **kw)
    else:
        fn(layer.experts, x, wl.k, out, ws, **kw)
    return out, ids


@pytest.mark.parametrize("wtype", ["bf16", "fp8"])
def test_noalloc_matches_forward(wtype):
    wl = W(f"noalloc-{wtype}", T=64, H=1024, E=64, k=8, I=512, shared=1, wtype=wtype, bias="all", seed=95)
    log(f"noalloc {wl.name}: T={wl.T} then 23, H={wl.H} E={wl.E} k={wl.k} I={wl.I}")
    d = workloads.make_inputs(wl, device="cuda")
    layer = _layer(d, wtype == "fp8")
    for T, ydt in ((wl.T, moe.MOE_DTYPE_F32), (23, moe.MOE_DTYPE_BF16)):
        nbytes = moe.moe_forward_workspace_bytes(layer.experts, T, wl.k, ydt)
        assert 0 < nbytes <= moe.MOE_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        want, want_ids = _run(moe.moe_forward, layer, wl, d, T, ydt, ws)
        got, got_ids = _run(moe.moe_forward_noalloc, layer, wl, d, T, ydt)
        torch.cuda.synchronize()
        assert torch.equal(got_ids, want_ids), f"T={T}: routing ids differ"
        assert torch.equal(got, want), f"T={T}: output differs from moe_forward"


def test_noalloc_refuses_past_its_scratch():
    wl = W("noalloc-big", T=8192, H=1024, E=8, k=2, I=512, shared=1, seed=96)
    d = workloads.make_inputs(wl, device="cuda")
    layer = _layer(d, False)
    assert moe.moe_forward_workspace_bytes(layer.experts, wl.T, wl.k) > moe.MOE_NOALLOC_SCRATCH_BYTES
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as exc:
        moe.moe_forward_noalloc(layer.experts, d["x"], wl.k, out, logits=d["logits"])
    assert exc.value.status == moe.MOE_EUNSUPPORTED
