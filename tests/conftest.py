import os
import sys

import numpy as np
import pytest

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def to_np(t):
    """torch tensor -> numpy array in the oracle's input encoding.

    bf16 tensors become uint16 bit patterns, fp8 codes stay uint8, fp32 stays
    fp32.  None passes through.
    """
    import torch
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


class LazyExperts:
    """Per-expert numpy view of a stacked ``[E, ...]`` torch tensor.

    The oracle indexes weights per expert; this copies one expert at a time
    to the host, so large device tensors never need a full host copy.
    """

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return to_np(self.t[e])

    def __len__(self):
        return self.t.shape[0]


def oracle_inputs(wl, inp, lazy=False):
    """Map ``synth.make_inputs`` tensors onto ``oracle.layer.forward`` args."""
    from oracle.layer import LayerSpec
    spec = LayerSpec(hidden=wl.hidden, experts=wl.experts, topk=wl.topk,
                     inter=wl.inter, shared_inter=wl.shared_inter,
                     dtype=wl.dtype, gating=wl.gating,
                     routed_scale=wl.routed_scale, renormalize=wl.renormalize,
                     block=wl.block)
    wrap = LazyExperts if lazy else to_np
    kw = dict(x=to_np(inp["x"]), router_w=to_np(inp["router_w"]),
              w13=wrap(inp["w13"]), w2=wrap(inp["w2"]),
              w13_scale=None if inp["w13_scale"] is None else wrap(inp["w13_scale"]),
              w2_scale=None if inp["w2_scale"] is None else wrap(inp["w2_scale"]),
              bias=to_np(inp["bias"]))
    if wl.shared_inter > 0:
        kw["shared"] = {"w13": to_np(inp["shared_w13"]),
                        "w2": to_np(inp["shared_w2"]),
                        "w13_scale": to_np(inp["shared_w13_scale"]),
                        "w2_scale": to_np(inp["shared_w2_scale"]),
                        "gate": to_np(inp.get("shared_gate"))}
    return spec, kw


@pytest.fixture
def np_rng():
    return np.random.default_rng(1234)
