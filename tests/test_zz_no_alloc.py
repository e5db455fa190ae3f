"""moe_forward_noalloc (static per-GPU scratch) against moe_forward (the
caller's workspace), through the C ABI: two calls in a row on each expert
path, the second with fewer tokens; outputs, indices and weights must be
bit-identical, since both run the same kernels in the same order."""
import pytest
import torch

import synth
from mixture_experts_ffn_06_amd._lib import NOALLOC_SCRATCH_BYTES
from tests.test_gpu_parity import RAGGED_BF16, RAGGED_FP8, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(layer, inp, m):
    x = inp["x"][:m]
    ref = layer(x)
    H, k = layer.hidden, layer.topk
    out = torch.full((m, H), 3.0, dtype=layer.act_dtype, device=DEV)
    idx = torch.full((m, k), -1, dtype=torch.int32, device=DEV)
    w = torch.full((m, k), -1.0, dtype=torch.float32, device=DEV)
    layer.plan.forward_noalloc(x, layer.w["router_w"], layer.w["w13"], layer.w["w2"], out, idx, w,
                               shared=layer.shared, bias=layer.w.get("bias"),
                               w13_scale=layer.w.get("w13_scale"), w2_scale=layer.w.get("w2_scale"))
    torch.cuda.synchronize()
    return ref, (out, idx, w)


@pytest.mark.parametrize("wl,path,ms", [
    (RAGGED_FP8, "grouped", (300, 77)),
    (RAGGED_BF16, "grouped", (200, 31)),
    (synth.WORKLOADS["decode_bf16"], "small_m", (16, 5)),
    (synth.WORKLOADS["prefill_bf16"], "grouped", (1024, 256)),
], ids=["fp8_grouped", "bf16_grouped", "decode_small_m", "prefill_grouped"])
def test_noalloc_equals_the_workspace_entry_point(wl, path, ms):
    print(f"case noalloc {wl.name} {path} m={ms}", flush=True)
    inp = synth.make_inputs(wl, device=DEV)
    layer = make_layer(wl, inp, path, max_tokens=ms[0])
    assert layer.plan.workspace_bytes(ms[0]) <= NOALLOC_SCRATCH_BYTES
    for m in ms:
        (o1, i1, w1), (o2, i2, w2) = _both(layer, inp, m)
        assert torch.equal(i1, i2) and torch.equal(w1, w2)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_noalloc_rejects_a_call_beyond_the_scratch():
    from mixture_experts_ffn_06_amd import MoeError, MoePlan
    wl = synth.WORKLOADS["large_fp8"]
    plan = MoePlan(wl.hidden, wl.experts, wl.inter, wl.topk, 4096, shared_inter=wl.shared_inter,
                   gating=wl.gating, routed_scale=wl.routed_scale, weight_dtype="fp8")
    assert plan.workspace_bytes(4096) > NOALLOC_SCRATCH_BYTES
    z = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(MoeError) as ei:
        plan.forward_noalloc(z, z, z, z, z, z, z, shared={"w13": z, "w2": z, "w13_scale": z,
                                                           "w2_scale": z}, m=4096)
    assert ei.value.status == 3 and "scratch" in str(ei.value)
