"""Brute-force dense evaluation of the MoE layer (test infrastructure only).

A second, deliberately different formulation used to pin ``oracle.layer``
on tiny inputs: every expert is evaluated on every token with one einsum,
the routing enters as a dense ``[m, E]`` mask holding the gate weight of each
selected expert (0 elsewhere), and top-k uses ``np.lexsort`` instead of an
argsort.  No permutation, no per-expert grouping.
"""
from __future__ import annotations

import numpy as np

from .codec import bf16_round, e4m3_decode, e4m3_quantize_rows


def _round_h(a: np.ndarray, dtype: str, block: int) -> np.ndarray:
    """Round a ``[..., I]`` SwiGLU output to the down operand format."""
    if dtype == "f32":
        return a
    if dtype in ("bf16", "mxfp4", "mxfp8"):
        return bf16_round(a)
    flat = a.reshape(-1, a.shape[-1]).astype(np.float32)
    codes, scales = e4m3_quantize_rows(flat, block)
    v = e4m3_decode(codes) * np.repeat(scales.astype(np.float64), block, axis=1)
    return v.reshape(a.shape)


def dense_mask(logits: np.ndarray, k: int, gating: str, bias=None,
               scale: float = 1.0, renormalize: bool = True) -> np.ndarray:
    """``M[t, e]`` = gate weight of expert e for token t, 0 if not selected."""
    m, E = logits.shape
    M = np.zeros((m, E))
    b = None if bias is None else np.asarray(bias, np.float32).astype(np.float64)
    for t in range(m):
        l = logits[t]
        if gating == "softmax":
            if b is None:
                # ranking by softmax probability == ranking by logit
                rank_key = l.copy()
            else:
                e = np.exp(l - l.max())
                rank_key = e / e.sum() + b
        else:
            if gating == "sigmoid":
                rank_key = 1.0 / (1.0 + np.exp(-l))
            else:   # sqrtsoftplus; the tiny inputs keep e^l finite
                rank_key = np.sqrt(np.log1p(np.exp(l)))
            if b is not None:
                rank_key = rank_key + b
        order = np.lexsort((np.arange(E), -rank_key))
        sel = order[:k]
        if gating == "softmax":
            if renormalize:
                # renormalised softmax over the selected logits only
                z = l[sel] - l[sel].max()
                w = np.exp(z) / np.exp(z).sum()
            else:
                z = l - l.max()
                w = (np.exp(z) / np.exp(z).sum())[sel]
        else:
            if gating == "sigmoid":
                s = 1.0 / (1.0 + np.exp(-l[sel]))
            else:
                s = np.sqrt(np.log1p(np.exp(l[sel])))
            w = s / s.sum() if renormalize else s
        M[t, sel] = w * scale
    return M


def dense_forward(xt: np.ndarray, logits: np.ndarray, k: int, gating: str,
                  W13: np.ndarray, W2: np.ndarray, inter: int, dtype: str,
                  bias=None, scale: float = 1.0, shared=None,
                  shared_inter: int = 0, block: int = 128,
                  renormalize: bool = True, x_gate=None,
                  gate=None) -> np.ndarray:
    """Dense fp64 layer output ``[m, H]`` (unrounded).

    ``xt [m,H]``: expert input values (dequantised for fp8);
    ``logits [m,E]``: router logits; ``W13 [E,2I,H]``, ``W2 [E,H,I]``:
    exact weight values; ``shared``: ``(W13s [2Is,H], W2s [H,Is])`` or None;
    ``gate [H]`` with ``x_gate [m,H]`` (the unquantised input): the shared
    row of token t is scaled by ``1 / (1 + exp(-x_gate[t] . gate))``.
    """
    M = dense_mask(logits, k, gating, bias, scale, renormalize)
    g = np.einsum("th,eih->tei", xt, W13[:, :inter, :])
    u = np.einsum("th,eih->tei", xt, W13[:, inter:, :])
    a = g / (1.0 + np.exp(-g)) * u
    a = _round_h(a, dtype, block)
    y = np.einsum("tei,ehi->teh", a, W2)     # down outputs enter the reduce unrounded
    out = np.einsum("te,teh->th", M, y)
    if shared is not None and shared_inter > 0:
        S13, S2 = shared
        gs = xt @ S13[:shared_inter].T
        us = xt @ S13[shared_inter:].T
        hs = _round_h(gs / (1.0 + np.exp(-gs)) * us, dtype, block)
        ys = hs @ S2.T
        if gate is not None:
            ys = ys / (1.0 + np.exp(-(x_gate @ gate)))[:, None]
        out = out + ys
    return out
