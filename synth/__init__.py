"""Seeded synthetic inputs for one Mixture-of-Experts FFN layer.

This module draws random numbers and stores them in the layer's input
formats: fp32, bf16, or OCP e4m3 codes with one fp32 scale per 128x128 weight
block.  It holds none of the layer's arithmetic -- no router product, gating,
routing, expert GEMM or activation quantisation.  The fp64 oracle and the HIP
library's tests both take their inputs from here, and from nowhere else.

The workloads mirror the layer that forward_prefill.rs (page 3,
``MoeLayer::forward_prefill``) runs: a router over E experts, top-k gating,
SwiGLU experts (w1/w3 ``[E, I, H]`` stacked as ``w13 [E, 2I, H]``, w2
``[E, H, I]``) and an optional shared expert.  There are no trained weights:
every tensor is drawn from a seeded generator.

Draw recipe (all seeds are fixed integers):

* ``x``      ~ N(0, 1), numpy ``default_rng([seed, 3])``, fp32, then stored
  in the activation dtype (bf16 by round-to-nearest-even through torch's cast).
* router     ~ N(0, 0.02), ``default_rng([seed, 0, router_subseed])``.
* expert e   ~ N(0, 0.02), torch generator seeded from ``(seed, 1, e)``; drawn
  one expert at a time on the device that will hold it.
* shared     ~ N(0, 0.02), torch generator seeded from ``(seed, 2, 0)``.
* shared gate (workloads with a gated shared-expert blend): a ``[H]`` vector
  ~ N(0, 0.02), ``default_rng([seed, 5])``, stored like x.
* selection bias (skewed workload only): a seeded permutation assigns each
  expert a popularity rank r in 1..E; ``b_1 = 0`` and, for r >= 2,
  ``b_r = -head - alpha * s * ln r``, i.e. ``alpha * ln(p_r / p_1)`` for
  Zipf(s) popularity ``p_r ~ r**-s`` plus a gap ``head`` that lets the most
  popular expert take more than 10 % of all assignments.  (A one-parameter
  Zipf bias cannot give both that share and only ~20 idle experts when
  each token picks 8 of 256.)

fp8 weights are stored blockwise: for each 128x128 block, scale =
amax / 448 (fp32) and codes = torch's float8_e4m3fn cast of the clamped
quotient.  MXFP4 weights (OCP Microscaling, FP4 E2M1 elements with an E8M0
scale per 32 consecutive elements of a row, along K): shared exponent
``X = floor(log2(amax)) - 2`` (2 = the element format's largest exponent),
scale byte ``X + 127``, elements rounded to the nearest of 0, 0.5, 1, 1.5,
2, 3, 4, 6 (ties to the even code) after division by ``2**X``, saturating
at 6; two elements per byte, the even one in the low nibble.  MXFP8 weights
(FP8 E4M3 elements, E8M0 scale per 32 along K): ``X = floor(log2(amax)) -
8``, elements = torch's float8_e4m3fn cast of the quotient clamped to 448.
The layer receives codes and scales as given.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "draw_x", "draw_router",
           "draw_bias", "draw_shared_gate", "expert_seed"]


@dataclass(frozen=True)
class Workload:
    """Shape and draw parameters of one synthetic MoE layer."""
    name: str
    m: int                 # tokens
    hidden: int            # H
    experts: int           # E
    topk: int              # k
    inter: int             # I (per routed expert)
    shared_inter: int      # I_s, 0 = no shared expert
    dtype: str             # "f32" | "bf16" | "fp8" | "mxfp4" | "mxfp8" (weights)
    gating: str            # "softmax" | "sigmoid" | "sqrtsoftplus"
    routed_scale: float    # multiplier after renormalisation
    seed: int
    router_subseed: int = 0
    zipf_alpha: float = 0.0  # > 0: selection-only Zipf bias
    zipf_s: float = 1.2
    zipf_head: float = 0.0   # extra gap below the most popular expert
    block: int = 128         # fp8 block edge
    renormalize: bool = True   # divide the selected weights by their sum
    shared_gate: bool = False  # shared expert scaled by sigmoid(x . g)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.m * self.topk

    @property
    def act_dtype(self) -> str:
        return "f32" if self.dtype == "f32" else "bf16"


# The router sub-seed of the prefill workload and the bias strengths of the
# skewed workloads are found by tests/golden/make_workload_params.py (which
# runs the fp64 oracle's gating) and re-checked by the CPU test suite.
# skew_fp8: a pure Zipf(1.2) bias whose strength leaves 20 experts without a
# token (the middle of the range of strengths that do; at its edges one
# top-k near-tie decides an expert's only token); its busiest expert then
# takes 3.4 % of the assignments (the > 10 % asked alongside cannot hold
# with 20 idle experts under a pure Zipf bias).  skew_head_fp8
# (supplementary): the same bias with a gap below the most popular expert,
# which gives both (20 idle, top expert > 10 %).
PREFILL_ROUTER_SUBSEED = 31
SKEW_ZIPF_ALPHA = 0.04326865809483731
SKEW_HEAD_ZIPF_HEAD = 0.7
SKEW_HEAD_ZIPF_ALPHA = 0.04088530535399924

WORKLOADS: dict[str, Workload] = {
    # Tiny fp32 layer, softmax top-2 renormalised, no shared expert.
    "tiny_f32": Workload("tiny_f32", m=4, hidden=64, experts=8, topk=2,
                         inter=32, shared_inter=0, dtype="f32",
                         gating="softmax", routed_scale=1.0, seed=0),
    # Decode-shaped bf16 layer; m in {1, 4, 16} are prefixes of one 16-row draw.
    "decode_bf16": Workload("decode_bf16", m=16, hidden=2048, experts=128,
                            topk=8, inter=768, shared_inter=0, dtype="bf16",
                            gating="softmax", routed_scale=1.0, seed=2),
    # The decode layer with MXFP4 expert weights (same x and router draws).
    "decode_mxfp4": Workload("decode_mxfp4", m=16, hidden=2048, experts=128,
                             topk=8, inter=768, shared_inter=0, dtype="mxfp4",
                             gating="softmax", routed_scale=1.0, seed=2),
    "decode_mxfp8": Workload("decode_mxfp8", m=16, hidden=2048, experts=128,
                             topk=8, inter=768, shared_inter=0, dtype="mxfp8",
                             gating="softmax", routed_scale=1.0, seed=2),
    # Prefill bf16 layer with one unweighted shared expert (I_s = 2048).
    "prefill_bf16": Workload("prefill_bf16", m=1024, hidden=2048,
                             experts=128, topk=8, inter=768,
                             shared_inter=2048, dtype="bf16",
                             gating="softmax", routed_scale=1.0, seed=3,
                             router_subseed=PREFILL_ROUTER_SUBSEED),
    # Large fp8 layer: sigmoid top-8 renormalised and scaled by 2.5.
    "large_fp8": Workload("large_fp8", m=4096, hidden=7168, experts=256,
                          topk=8, inter=2048, shared_inter=2048, dtype="fp8",
                          gating="sigmoid", routed_scale=2.5, seed=4),
    # MFMA-bound shapes (about 1024 / 512 rows per expert): the prefill
    # layer with m = 16384 and the large fp8 layer with m = 16384.
    "dense_bf16": Workload("dense_bf16", m=16384, hidden=2048, experts=128,
                           topk=8, inter=768, shared_inter=2048, dtype="bf16",
                           gating="softmax", routed_scale=1.0, seed=6),
    "dense_fp8": Workload("dense_fp8", m=16384, hidden=7168, experts=256,
                          topk=8, inter=2048, shared_inter=2048, dtype="fp8",
                          gating="sigmoid", routed_scale=2.5, seed=7),
    # Skewed routing on the large-fp8 shapes with m = 2048.
    "skew_fp8": Workload("skew_fp8", m=2048, hidden=7168, experts=256,
                         topk=8, inter=2048, shared_inter=2048, dtype="fp8",
                         gating="sigmoid", routed_scale=2.5, seed=5,
                         zipf_alpha=SKEW_ZIPF_ALPHA),
    # The skewed layer with a hot expert (supplementary load-imbalance case).
    "skew_head_fp8": Workload("skew_head_fp8", m=2048, hidden=7168, experts=256,
                              topk=8, inter=2048, shared_inter=2048, dtype="fp8",
                              gating="sigmoid", routed_scale=2.5, seed=5,
                              zipf_alpha=SKEW_HEAD_ZIPF_ALPHA,
                              zipf_head=SKEW_HEAD_ZIPF_HEAD),
}


def _np_rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def expert_seed(seed: int, stream: int, e: int) -> int:
    """64-bit torch seed for one expert's draw."""
    st = np.random.SeedSequence([seed, stream, e]).generate_state(1, np.uint64)
    return int(st[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def draw_x(wl: Workload) -> np.ndarray:
    """fp32 N(0,1) activations ``[m, H]`` (before storage rounding)."""
    return _np_rng(wl.seed, 3).standard_normal((wl.m, wl.hidden),
                                               dtype=np.float32)


def draw_router(wl: Workload, subseed: int | None = None) -> np.ndarray:
    """fp32 N(0, 0.02) router weights ``[E, H]`` (before storage rounding)."""
    r = wl.router_subseed if subseed is None else subseed
    g = _np_rng(wl.seed, 0, r)
    return (np.float32(0.02) *
            g.standard_normal((wl.experts, wl.hidden), dtype=np.float32))


def draw_bias(wl: Workload, alpha: float | None = None) -> np.ndarray | None:
    """Selection-only Zipf bias ``[E]`` fp32, or None."""
    a = wl.zipf_alpha if alpha is None else alpha
    if a <= 0.0:
        return None
    perm = _np_rng(wl.seed, 4).permutation(wl.experts)
    rank = np.empty(wl.experts, dtype=np.float64)
    rank[perm] = np.arange(1, wl.experts + 1, dtype=np.float64)
    b = -a * wl.zipf_s * np.log(rank) - wl.zipf_head * (rank >= 2)
    return b.astype(np.float32)


def draw_shared_gate(wl: Workload) -> np.ndarray:
    """fp32 N(0, 0.02) shared-expert gate vector ``[H]`` (before storage
    rounding)."""
    return (np.float32(0.02) *
            _np_rng(wl.seed, 5).standard_normal(wl.hidden, dtype=np.float32))


def _store_act(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "f32":
        return t.to(device)
    return t.to(torch.bfloat16).to(device)


def _block_fp8(w: torch.Tensor, block: int) -> tuple[torch.Tensor, torch.Tensor]:
    """Store a 2-D fp32 matrix as e4m3 codes with fp32 per-block scales."""
    r, c = w.shape
    wb = w.reshape(r // block, block, c // block, block)
    amax = wb.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (wb / scale[:, None, :, None]).clamp(-448.0, 448.0)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(r, c)
    return codes.contiguous(), scale.contiguous()


def _mx_fp4(w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Store a 2-D fp32 matrix as packed MXFP4 codes and E8M0 scale bytes
    (one per 32 consecutive elements of a row)."""
    r, c = w.shape
    wb = w.reshape(r, c // 32, 32)
    amax = wb.abs().amax(dim=-1)
    X = torch.floor(torch.log2(amax.clamp_min(2.0 ** -126))) - 2
    X = torch.where(amax > 0, X, torch.full_like(X, -127.0)).clamp(-127.0, 127.0)
    q = wb / torch.exp2(X)[..., None]
    mag = q.abs()
    # index of the nearest e2m1 magnitude, ties to the even code
    idx = ((mag > 0.25).int() + (mag >= 0.75).int() + (mag > 1.25).int() +
           (mag >= 1.75).int() + (mag > 2.5).int() + (mag >= 3.5).int() + (mag > 5.0).int())
    code = (idx | ((q < 0).int() << 3)).reshape(r, c)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).to(torch.uint8)
    return packed.contiguous(), (X + 127).to(torch.uint8).contiguous()


def _mx_fp8(w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Store a 2-D fp32 matrix as MXFP8 codes (e4m3fn bytes) and E8M0 scale
    bytes (one per 32 consecutive elements of a row)."""
    r, c = w.shape
    wb = w.reshape(r, c // 32, 32)
    amax = wb.abs().amax(dim=-1)
    X = torch.floor(torch.log2(amax.clamp_min(2.0 ** -126))) - 8
    X = torch.where(amax > 0, X, torch.full_like(X, -127.0)).clamp(-127.0, 127.0)
    q = (wb / torch.exp2(X)[..., None]).clamp(-448.0, 448.0)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(r, c)
    return codes.contiguous(), (X + 127).to(torch.uint8).contiguous()


def _draw_matrix(seed: int, rows: int, cols: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((rows, cols), generator=g, device=device,
                       dtype=torch.float32) * 0.02


def _store_weight(w: torch.Tensor, dtype: str, block: int):
    if dtype == "f32":
        return w, None
    if dtype == "bf16":
        return w.to(torch.bfloat16), None
    if dtype == "mxfp4":
        return _mx_fp4(w)
    if dtype == "mxfp8":
        return _mx_fp8(w)
    return _block_fp8(w, block)


def make_inputs(wl: Workload, device="cpu", m: int | None = None) -> dict:
    """All layer inputs for workload ``wl`` as torch tensors on ``device``.

    Keys: ``x [m,H]``, ``router_w [E,H]``, ``w13 [E,2I,H]``, ``w2 [E,H,I]``,
    ``w13_scale [E,2I/128,H/128]`` / ``w2_scale [E,H/128,I/128]`` (fp8 only),
    ``shared_w13 [2Is,H]``, ``shared_w2 [H,Is]`` (+ scales), ``shared_gate
    [H]`` (activation format), ``bias [E]``.
    Absent entries are None.  ``m`` takes a prefix of the token draw (at most
    ``wl.m`` tokens: a larger batch is a workload of its own, ``wl.replace(m=...)``).
    """
    device = torch.device(device)
    x = draw_x(wl)
    if m is not None:
        if m > wl.m:
            raise ValueError(f"{wl.name}: m = {m} exceeds the workload's {wl.m} tokens")
        x = x[:m]
    out = {"x": _store_act(x, wl.act_dtype, device),
           "router_w": _store_act(draw_router(wl), wl.act_dtype, device)}
    b = draw_bias(wl)
    out["bias"] = None if b is None else torch.from_numpy(b).to(device)
    E, H, I = wl.experts, wl.hidden, wl.inter
    wdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8,
           "mxfp4": torch.uint8, "mxfp8": torch.uint8}[wl.dtype]
    pk = 2 if wl.dtype == "mxfp4" else 1     # elements per stored byte along K
    w13 = torch.empty((E, 2 * I, H // pk), dtype=wdt, device=device)
    w2 = torch.empty((E, H, I // pk), dtype=wdt, device=device)
    s13 = s2 = None
    if wl.dtype in ("mxfp4", "mxfp8"):
        s13 = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=device)
        s2 = torch.empty((E, H, I // 32), dtype=torch.uint8, device=device)
    if wl.dtype == "fp8":
        B = wl.block
        s13 = torch.empty((E, 2 * I // B, H // B), dtype=torch.float32, device=device)
        s2 = torch.empty((E, H // B, I // B), dtype=torch.float32, device=device)
    for e in range(E):
        a = _draw_matrix(expert_seed(wl.seed, 1, e), 3 * I, H, device)
        # rows [0, 2I) are w1 then w3; the last I rows, transposed, are w2.
        c13, sc13 = _store_weight(a[: 2 * I], wl.dtype, wl.block)
        c2, sc2 = _store_weight(a[2 * I:].t().contiguous(), wl.dtype, wl.block)
        w13[e].copy_(c13)
        w2[e].copy_(c2)
        if s13 is not None:
            s13[e].copy_(sc13)
            s2[e].copy_(sc2)
    out.update(w13=w13, w2=w2, w13_scale=s13, w2_scale=s2)
    out.update(shared_w13=None, shared_w2=None, shared_w13_scale=None,
               shared_w2_scale=None, shared_gate=None)
    if wl.shared_inter > 0:
        Is = wl.shared_inter
        a = _draw_matrix(expert_seed(wl.seed, 2, 0), 3 * Is, H, device)
        c13, sc13 = _store_weight(a[: 2 * Is], wl.dtype, wl.block)
        c2, sc2 = _store_weight(a[2 * Is:].t().contiguous(), wl.dtype, wl.block)
        out.update(shared_w13=c13.contiguous(), shared_w2=c2.contiguous(),
                   shared_w13_scale=sc13, shared_w2_scale=sc2)
        if wl.shared_gate:
            out["shared_gate"] = _store_act(draw_shared_gate(wl), wl.act_dtype, device)
    return out
