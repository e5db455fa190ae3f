"""Convenience wrapper: one MoE layer's weights, its plan and a workspace.

torch allocates the device buffers; ``libmoe`` does all of the compute.
"""
from __future__ import annotations

import torch

from ._lib import MoePlan


class MoeLayer:
    """Holds weights (device tensors), a ``MoePlan`` and a reusable workspace.

    ``weights`` keys: ``router_w [E,H]``, ``w13 [E,2I,H]``, ``w2 [E,H,I]``,
    optional ``w13_scale``, ``w2_scale`` (fp8), ``shared_w13``,
    ``shared_w2`` (+ ``shared_w13_scale``, ``shared_w2_scale``, and
    ``shared_gate [H]`` for the sigmoid-gated blend), ``bias``.
    """

    def __init__(self, weights: dict, *, hidden: int, num_experts: int,
                 inter: int, topk: int, max_tokens: int, shared_inter: int = 0,
                 gating: str = "softmax", renormalize: bool = True,
                 routed_scale: float = 1.0, weight_dtype: str = "bf16",
                 path: str = "auto"):
        self.w = weights
        self.plan = MoePlan(hidden, num_experts, inter, topk, max_tokens,
                            shared_inter=shared_inter, gating=gating,
                            renormalize=renormalize, routed_scale=routed_scale,
                            weight_dtype=weight_dtype, path=path)
        self.hidden, self.topk = hidden, topk
        self.act_dtype = torch.float32 if weight_dtype == "f32" else torch.bfloat16
        self.device = weights["w13"].device
        nbytes = self.plan.workspace_bytes(max_tokens)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        self.shared = None
        if shared_inter > 0:
            self.shared = {"w13": weights["shared_w13"], "w2": weights["shared_w2"],
                           "w13_scale": weights.get("shared_w13_scale"),
                           "w2_scale": weights.get("shared_w2_scale"),
                           "gate": weights.get("shared_gate")}

    def __call__(self, x: torch.Tensor, out=None, topk_idx=None, topk_w=None,
                 stream=None, debug=None):
        m = x.shape[0]
        if out is None:
            out = torch.empty((m, self.hidden), dtype=self.act_dtype, device=self.device)
        if topk_idx is None:
            topk_idx = torch.empty((m, self.topk), dtype=torch.int32, device=self.device)
        if topk_w is None:
            topk_w = torch.empty((m, self.topk), dtype=torch.float32, device=self.device)
        self.plan.forward(x, self.w["router_w"], self.w["w13"], self.w["w2"], out,
                          topk_idx, topk_w, self.workspace, shared=self.shared,
                          bias=self.w.get("bias"), w13_scale=self.w.get("w13_scale"),
                          w2_scale=self.w.get("w2_scale"), stream=stream,
                          debug=debug, m=m)
        return out, topk_idx, topk_w
