"""fp64 oracle of one MoE FFN layer forward (test infrastructure only).

The layer is the pipeline that forward_prefill.rs (page 3,
``MoeLayer::forward_prefill``, doc comment "Pipeline") names: router product,
top-k gating, sort by expert, gate/up product with SiLU gating, down product,
unpermute with the weighted top-k reduction, and the shared-expert blend.
The grouped, sorted pipeline reaches exactly the plain definition of the
layer -- a top-k gated sum of SwiGLU experts plus a shared expert -- so this
file writes that definition out, one step per function, in float64 over the
exact values of the quantised inputs.

Readings where the pages leave a step open (each is also listed in the design
notes of the repository):

* top-k order: descending score, equal scores -> lower expert index first;
* softmax gating ranks the softmax probabilities over all E experts and the
  k selected ones are divided by their sum (``norm_topk_prob``, page 3,
  top-k dispatch);
* sigmoid gating ranks ``sigmoid(l) + bias`` (page 3, top-k dispatch: the
  bias only chooses the experts, the weights are taken from the scores
  before it), weights are the unbiased sigmoid scores renormalised then
  multiplied by the routed scaling factor;
* sqrtsoftplus gating (page 3, top-k dispatch: the DeepSeek-V4 scoring
  function, with the same correction bias) scores ``sqrt(softplus(l))``
  with ``softplus(l) = ln(1 + e^l)`` and is otherwise handled like sigmoid;
* softmax with a correction bias (page 3, top-k dispatch, the softmax +
  bias branch) ranks ``p + bias`` and weights the unbiased probabilities;
* the routing weight multiplies at the combine (page 3, step 7
  ``moe_unpermute_reduce_indexed``), not inside the SwiGLU;
* SwiGLU is ``silu(w1 x) * (w3 x)`` with no clamp; the expert intermediate is
  rounded to the GEMM operand format (bf16, or fp8 per row per 128 columns)
  before the down product;
* each expert's down output enters the weighted reduce unrounded: only the
  operands of the two expert products (x or its fp8 codes, the weights, the
  rounded intermediate) and the layer output are rounded.  The storage of
  the per-pair down output between the two steps is accumulator precision,
  which the output tolerance covers (page 3 keeps it in BF16; one BF16 step
  of a stored row is a 0.4 % change of a summand, which next to an output
  that cancels to a tenth of the output rms reads as a several-percent
  output error, so the reduce takes fp32 rows);
* the shared expert is added with weight 1 (page 2, ``MoeV41::forward``:
  routed and shared rows are summed into one fp32 accumulator, cleared first),
  or, when the layer has a shared-expert gate vector g, with weight
  ``sigmoid(x . g)`` per token (page 3, step 8, the shared-expert blend: a
  per-token logistic factor of the input's dot product with a gate vector
  scales the shared row).  The dot product takes the layer input as given,
  never its fp8 quantisation;
* the output is rounded once, from the fp64 sum, to the activation format.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .codec import (bf16_decode, bf16_round, dequant_blocks,
                    e4m3_decode, e4m3_quantize_rows, mxfp4_decode, mxfp8_decode)


@dataclass
class LayerSpec:
    """Shape and options of one layer, as plain numbers."""
    hidden: int
    experts: int
    topk: int
    inter: int
    shared_inter: int
    dtype: str            # "f32" | "bf16" | "fp8" | "mxfp4" | "mxfp8" (MX: weights only; x and h bf16)
    gating: str           # "softmax" | "sigmoid" | "sqrtsoftplus"
    routed_scale: float = 1.0
    renormalize: bool = True
    block: int = 128


# ------------------------------------------------------------ values in ---

def act_values(x, dtype: str) -> np.ndarray:
    """Exact fp64 values of an activation / router tensor."""
    x = np.asarray(x)
    if dtype == "f32":
        return x.astype(np.float64)
    return bf16_decode(x.view(np.uint16) if x.dtype != np.uint16 else x)


def weight_values(w, scale, dtype: str, block: int) -> np.ndarray:
    """Exact fp64 values of one expert's weight matrix."""
    w = np.asarray(w)
    if dtype == "f32":
        return w.astype(np.float64)
    if dtype == "bf16":
        return bf16_decode(w.view(np.uint16) if w.dtype != np.uint16 else w)
    if dtype == "mxfp4":
        return mxfp4_decode(w.view(np.uint8), np.asarray(scale).view(np.uint8), 32)
    if dtype == "mxfp8":
        return mxfp8_decode(w.view(np.uint8), np.asarray(scale).view(np.uint8), 32)
    return dequant_blocks(w.view(np.uint8), np.asarray(scale, np.float32), block)


# ------------------------------------------------------------------ O1 ---

def quantize_activations(x_vals: np.ndarray, block: int):
    """fp8 layer: x -> (codes, scales, exact dequantised values).

    Per token and per ``block`` columns of H, with the block rule of
    ``codec``.  x holds bf16 values, which fp32 represents exactly.
    """
    codes, scales = e4m3_quantize_rows(x_vals.astype(np.float32), block)
    xt = e4m3_decode(codes) * np.repeat(scales.astype(np.float64), block, axis=1)
    return codes, scales, xt


# ------------------------------------------------------------------ O2 ---

def router_logits(x_vals: np.ndarray, wr_vals: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * Wr[e, h] in fp64 (page 3, step 1 gate GEMM)."""
    return x_vals @ wr_vals.T


# -------------------------------------------------------------- O3 - O5 ---

def gate_scores(logits: np.ndarray, gating: str):
    """(probability used for the weights, score used for ranking)."""
    if gating == "softmax":
        z = logits - logits.max(axis=1, keepdims=True)
        ez = np.exp(z)
        p = ez / ez.sum(axis=1, keepdims=True)
        return p, p
    if gating == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-logits))
        return s, s
    if gating == "sqrtsoftplus":
        # softplus(l) = ln(e^0 + e^l), evaluated without overflow
        s = np.sqrt(np.logaddexp(0.0, logits))
        return s, s
    raise ValueError(gating)


def top_k(score: np.ndarray, k: int):
    """Top-k by descending score, ties to the lower expert index.

    Returns ``(idx [m,k] int32, gap [m])`` where gap is the score difference
    between the k-th and (k+1)-th ranked experts (+inf when k == E).
    """
    m, E = score.shape
    order = np.argsort(-score, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    if k < E:
        kth = np.take_along_axis(score, order[:, k - 1:k], axis=1)[:, 0]
        nxt = np.take_along_axis(score, order[:, k:k + 1], axis=1)[:, 0]
        gap = kth - nxt
    else:
        gap = np.full(m, np.inf)
    return idx, gap


def gate_weights(prob: np.ndarray, idx: np.ndarray, renormalize: bool,
                 scale: float) -> np.ndarray:
    """w[t, j] = scale * prob[idx] / sum_j prob[idx]  (renormalised)."""
    sel = np.take_along_axis(prob, idx.astype(np.int64), axis=1)
    if renormalize:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel * scale


# ------------------------------------------------------------------ O6 ---

def permute(idx: np.ndarray, experts: int):
    """Sort (token, slot) pairs by expert: histogram, exclusive scan, scatter.

    Pair p = t*k + j carries expert idx[t, j].  Within an expert the pairs
    keep ascending p.  Returns ``counts [E], offsets [E+1],
    sorted_pair [te], slot_of_pair [te]`` (page 3, step 3 sort-by-expert:
    sorted ids, expert offsets and the token-to-slot map).
    """
    e_of_p = np.asarray(idx, dtype=np.int64).reshape(-1)
    te = e_of_p.size
    counts = np.zeros(experts, dtype=np.int64)
    for e in e_of_p:                      # histogram
        counts[e] += 1
    offsets = np.zeros(experts + 1, dtype=np.int64)
    for e in range(experts):              # exclusive scan
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    sorted_pair = np.empty(te, dtype=np.int64)
    slot_of_pair = np.empty(te, dtype=np.int64)
    for p in range(te):                   # stable scatter, ascending p
        s = cursor[e_of_p[p]]
        cursor[e_of_p[p]] += 1
        sorted_pair[s] = p
        slot_of_pair[p] = s
    return counts, offsets, sorted_pair, slot_of_pair


# -------------------------------------------------------------- O7 / O8 ---

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def round_intermediate(a: np.ndarray, dtype: str, block: int):
    """Round the SwiGLU output to the down product's operand format.

    Returns ``(values fp64, codes or None, scales or None)``.
    """
    if dtype == "f32":
        return a, None, None
    if dtype in ("bf16", "mxfp4", "mxfp8"):   # MX weights: bf16 intermediate
        return bf16_round(a), None, None
    codes, scales = e4m3_quantize_rows(a.astype(np.float32), block)
    vals = e4m3_decode(codes) * np.repeat(scales.astype(np.float64), block, axis=1)
    return vals, codes, scales


def expert_mlp(a_rows: np.ndarray, w13: np.ndarray, w2: np.ndarray,
               inter: int, dtype: str, block: int, h_ties=None):
    """SwiGLU expert on rows ``a_rows [n, H]`` with exact fp64 weights.

    ``w13 [2I, H]`` holds w1 (gate) in rows [0, I) and w3 (up) in [I, 2I);
    ``w2 [H, I]``.  Returns ``(y [n, H] unrounded, h values [n, I], h codes,
    h scales, h before rounding)``.

    ``h_ties``: optional ``(rows, cols, values)`` -- rounded intermediate
    values taken at near-ties: where the exact value lies next to the
    midpoint of two neighbouring codes, either code is a correct rounding,
    and the down product then continues from the one given (the caller
    checks that each given value is the other neighbour of such a tie).
    """
    g = a_rows @ w13[:inter].T
    u = a_rows @ w13[inter:].T
    h = silu(g) * u
    hv, hc, hs = round_intermediate(h, dtype, block)
    if h_ties is not None and len(h_ties[0]):
        hv = hv.copy()
        hv[h_ties[0], h_ties[1]] = h_ties[2]
    return hv @ w2.T, hv, hc, hs, h


# ------------------------------------------------------------------ all ---

def forward(spec: LayerSpec, x, router_w, w13, w2, w13_scale=None,
            w2_scale=None, shared=None, bias=None, tokens=None,
            idx_override=None, keep_h=False, h_ties=None) -> dict:
    """Oracle forward of the layer.

    ``x [m,H]``: bf16 bit patterns (uint16) or fp32.  ``router_w [E,H]``
    likewise.  ``w13[e]``, ``w2[e]`` (and ``w13_scale[e]``, ``w2_scale[e]``
    for fp8) are indexed per expert, so callers may pass lazy containers.
    ``shared`` is ``None`` or a dict with ``w13, w2`` (+ ``w13_scale,
    w2_scale``, and ``gate [H]`` in the activation format for the
    sigmoid-gated blend).  ``bias [E]`` fp32 is a selection-only bias.

    ``tokens``: optional sorted token subset for which expert outputs and
    ``out`` are evaluated (gating and permutation are always computed for
    all m tokens).  ``idx_override [m,k]``: evaluate with these expert
    indices instead of the oracle's own top-k (weights from the oracle's fp64
    probabilities at those indices).  ``keep_h``: also return, per pair p
    (routed) and per token (shared), the intermediate before rounding
    (``h_pre``, ``h_sh_pre``), its rounded values (``h``, ``h_sh``) and, for
    fp8, its scales (``h_scale``, ``h_sh_scale``).  ``h_ties``: near-tie
    choices of the rounded intermediate, ``(routed, shared)`` with ``routed``
    a dict pair -> ``(cols, values)`` and ``shared`` a dict token -> ``(cols,
    values)`` (see ``expert_mlp``); like ``idx_override`` for a top-k
    near-tie, they select between two correct roundings.

    Returns a dict with ``logits, prob, score, idx, gap, w, counts, offsets,
    sorted_pair, slot_of_pair, out64 [n,H], out [n,H]`` (rounded to the
    activation format and returned as fp64 values), ``tokens``, and for fp8
    ``xq, sx``.
    """
    B = spec.block
    act = "f32" if spec.dtype == "f32" else "bf16"
    xv = act_values(x, act)
    m, H = xv.shape
    E, k, I = spec.experts, spec.topk, spec.inter
    res = {}
    if spec.dtype == "fp8":
        xq, sx, xt = quantize_activations(xv, B)
        res.update(xq=xq, sx=sx)
    else:
        xt = xv
    logits = router_logits(xv, act_values(router_w, act))
    prob, score = gate_scores(logits, spec.gating)
    if bias is not None:
        score = score + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    idx, gap = top_k(score, k)
    if idx_override is not None:
        idx = np.asarray(idx_override, dtype=np.int32)
    w = gate_weights(prob, idx, spec.renormalize, spec.routed_scale)
    counts, offsets, sorted_pair, slot_of_pair = permute(idx, E)
    res.update(logits=logits, prob=prob, score=score, idx=idx, gap=gap, w=w,
               counts=counts, offsets=offsets, sorted_pair=sorted_pair,
               slot_of_pair=slot_of_pair)

    tok = np.arange(m) if tokens is None else np.asarray(sorted(tokens))
    pos_of_tok = {int(t): i for i, t in enumerate(tok)}
    acc = np.zeros((len(tok), H))
    h_rows, h_pre, h_sc = {}, {}, {}
    # routed experts: walk the sorted pairs expert by expert (grouped GEMM).
    for e in range(E):
        seg = sorted_pair[offsets[e]:offsets[e + 1]]
        seg = [int(p) for p in seg if int(p) // k in pos_of_tok]
        if not seg:
            continue
        rows = np.array([p // k for p in seg])
        w13e = weight_values(w13[e], None if w13_scale is None else w13_scale[e],
                             spec.dtype, B)
        w2e = weight_values(w2[e], None if w2_scale is None else w2_scale[e],
                            spec.dtype, B)
        ties = None
        if h_ties is not None and h_ties[0]:
            tr, tc, tv = [], [], []
            for i, p in enumerate(seg):
                if p in h_ties[0]:
                    cols, vals = h_ties[0][p]
                    tr += [i] * len(cols)
                    tc += list(cols)
                    tv += list(vals)
            ties = (np.array(tr, dtype=np.int64), np.array(tc, dtype=np.int64), np.array(tv))
        y, hv, _, hs, hp = expert_mlp(xt[rows], w13e, w2e, I, spec.dtype, B, ties)
        if keep_h:
            for i, p in enumerate(seg):
                h_rows[p] = hv[i]
                h_pre[p] = hp[i]
                if hs is not None:
                    h_sc[p] = hs[i]
        # unpermute + weighted reduce: each pair adds into its token's row
        for i, p in enumerate(seg):
            t, j = divmod(p, k)
            acc[pos_of_tok[t]] += w[t, j] * y[i]
    if shared is not None and spec.shared_inter > 0:
        s13 = weight_values(shared["w13"], shared.get("w13_scale"), spec.dtype, B)
        s2 = weight_values(shared["w2"], shared.get("w2_scale"), spec.dtype, B)
        ties = None
        if h_ties is not None and h_ties[1]:
            tr, tc, tv = [], [], []
            for i, t in enumerate(tok):
                if int(t) in h_ties[1]:
                    cols, vals = h_ties[1][int(t)]
                    tr += [i] * len(cols)
                    tc += list(cols)
                    tv += list(vals)
            ties = (np.array(tr, dtype=np.int64), np.array(tc, dtype=np.int64), np.array(tv))
        ysh, hv, _, hs, hp = expert_mlp(xt[tok], s13, s2, spec.shared_inter,
                                        spec.dtype, B, ties)
        if keep_h:
            res.update(h_sh=hv, h_sh_pre=hp, h_sh_scale=hs)
        if shared.get("gate") is not None:
            gl = xv[tok] @ act_values(shared["gate"], act)
            res["shared_gate"] = 1.0 / (1.0 + np.exp(-gl))
            ysh = res["shared_gate"][:, None] * ysh
        acc += ysh
    res["tokens"] = tok
    res["out64"] = acc
    res["out"] = acc if act == "f32" else bf16_round(acc)
    if spec.dtype == "f32":
        res["out"] = acc.astype(np.float32).astype(np.float64)
    if keep_h:
        res.update(h=h_rows, h_pre=h_pre, h_scale=h_sc)
    return res
