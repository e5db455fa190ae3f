"""HIP graph capture of the layer forward: every replay must equal the eager
call bit for bit (the forward records no memset and allocates nothing, so it
can be captured).  Replays are interleaved with eager work on other buffers
and host synchronisations."""
import pytest
import torch

import synth
from tests.test_gpu_parity import MX_SMALL, RAGGED_FP8, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("wl,m,path", [
    (synth.WORKLOADS["decode_bf16"], 16, "small_m"),
    (MX_SMALL, 13, "small_m"),
    (RAGGED_FP8, None, "grouped"),
], ids=["decode_bf16", "mxfp4", "ragged_fp8"])
def test_graph_replays_equal_the_eager_forward(wl, m, path):
    print(f"case graph {wl.name} m={m} path={path}", flush=True)
    inp = synth.make_inputs(wl, device=DEV, m=m)
    layer = make_layer(wl, inp, path)
    x = inp["x"]
    mm = x.shape[0]
    o_ref, i_ref, w_ref = [t.clone() for t in layer(x)]
    torch.cuda.synchronize()
    out = torch.empty_like(o_ref)
    idx = torch.empty_like(i_ref)
    tw = torch.empty_like(w_ref)
    layer(x, out=out, topk_idx=idx, topk_w=tw)       # warm-up, eager
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x, out=out, topk_idx=idx, topk_w=tw)
    other = torch.randn((mm, wl.hidden), device=DEV)
    for r in range(4):
        out.fill_(0)
        idx.fill_(-1)
        layer.workspace.fill_(0x5A)                 # a dirty workspace before each replay
        _ = (other * 2.0).sum()                     # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, i_ref), f"replay {r}: indices differ"
        assert torch.equal(tw, w_ref), f"replay {r}: weights differ"
        assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16)), f"replay {r}: output differs"
