"""mok_moe_forward_noalloc (the forward with the library's own device workspace) against
mok_moe_forward with a caller workspace: y and the saved activations bit-identical, on
two calls in a row, the second with a smaller batch (the shared array keeps the first
call's contents); bf16, MXFP8 and MXFP4; a descriptor whose workspace exceeds the
array is refused with MOK_ERR_WORKSPACE before anything is enqueued."""
import pytest
import torch

from harness import Case
from mixture_experts_layer_stable_amd import inputs

pytestmark = pytest.mark.gpu


def _forward_both(w, case, gemm):
    from mixture_experts_layer_stable_amd import mok
    dev = "cuda"
    mx = gemm != "bf16"
    d = mok.Desc(w.T, w.H, w.E, w.k, w.I, act=mok.BF16, gemm=mok.DTYPES[gemm] if mx else None)
    assert mok.workspace_query(d)["fwd_ws"] <= mok.NOALLOC_WS_BYTES
    buf = mok.Buffers(d, dev, backward=False)
    x, wr = case.x.to(dev), case.wr.to(dev)
    bias = None if case.bias is None else case.bias.to(dev)
    w1, w2, q = case.w1.to(dev), case.w2.to(dev), None
    if mx:
        q = mok.MxWeights(d, dev)
        mok.weights_quantize(d, w1, w2, q)
        w1 = w2 = None
    mok.route(d, x, wr, bias, buf.idx, buf.gate)
    mok.schedule_build(d, buf.idx, buf.sched)
    mok.moe_forward(d, buf.sched, x, buf.gate, w1, w2, buf.y, buf.saved, buf.fwd_ws, mxw=q)
    y_ref, saved_ref = buf.y.clone(), buf.saved.clone()
    buf.y.fill_(0)
    buf.saved.fill_(0)
    mok.moe_forward_noalloc(d, buf.sched, x, buf.gate, w1, w2, buf.y, buf.saved, mxw=q)
    torch.cuda.synchronize()
    mok.check_schedule(d, buf.sched)
    assert torch.equal(buf.y.view(torch.int16), y_ref.view(torch.int16))
    assert torch.equal(buf.saved, saved_ref)


@pytest.mark.parametrize("gemm", ["bf16", "mxfp8", "mxfp4"])
def test_noalloc_forward_matches_caller_workspace(gemm):
    big = inputs.replace(inputs.WORKLOADS["small_bf16"], gemm=gemm)
    small = inputs.replace(big, T=300, E=12, k=3)
    for w in (big, small):
        print("case noalloc T=%d E=%d k=%d gemm=%s" % (w.T, w.E, w.k, gemm), flush=True)
        _forward_both(w, Case(w), gemm)


def test_noalloc_refuses_oversized_workspace():
    from mixture_experts_layer_stable_amd import mok
    w = inputs.WORKLOADS["kimi_k2_bf16"]
    d = mok.Desc(w.T, w.H, w.E, w.k, w.I, act=mok.BF16)
    assert mok.workspace_query(d)["fwd_ws"] > mok.NOALLOC_WS_BYTES
    t = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(mok.MokError) as ei:
        mok.moe_forward_noalloc(d, t, t, t, t, t, t, t)
    assert ei.value.status == mok.ERR_WORKSPACE
