"""Parity of the HIP layer against the fp64 oracle (test infrastructure).

Acceptance rules:

* ``topk_idx``: bit-exact, except tokens whose k-th and (k+1)-th oracle
  scores differ by less than ``NEAR_TIE`` (1e-5); those are counted and, if
  their selection differs, re-checked against the oracle evaluated with the
  GPU's own indices (a different choice at a near-tie is a correct result).
* ``topk_w``: |gpu - oracle| <= 1e-5.
* permutation (counts, offsets, sorted_pair, slot_of_pair): bit-exact
  against the oracle's permutation of the GPU's ``topk_idx``.
* ``out``: err = max |o - r| / max(|r|, 0.1 * rms(r)) over the checked
  tokens, r the unrounded fp64 oracle output (computed from the layer's
  inputs alone, nothing taken from the GPU besides a near-tie choice): at
  most 2e-2 (bf16 and the MX formats, whose arithmetic is bf16), 4e-2
  (fp8), 1e-4 (fp32); and the relative L2 error ||o - r|| / ||r|| at most
  5e-3, 8e-3, 1e-5.  The same maximum with the floor at rms(r) is reported
  (``out_err_rms``).
* fp8 SwiGLU codes (when the debug buffers hold them) are decisions taken
  by floating point: each is the rounding of a value that the GPU forms in
  fp32 and the oracle in fp64.  Where the exact value lies within ``H_TIE``
  (relative) of the midpoint between two neighbouring e4m3 codes, both
  codes are correct roundings and the two sides may differ.  Such codes are
  treated like a near-tie top-k choice: counted (``h_ties``), and the
  output is then compared with the oracle rerun with the GPU's choice at
  exactly those codes (expressed in the oracle's own scale); every other
  code and every output element is compared with the oracle computed from
  the inputs alone.  A code that differs from the oracle's away from such a
  tie is counted as ``h_hard`` and left to the output gate; the error
  against the unconditioned oracle is reported as ``out_err_raw``.  Every
  GPU h scale must lie within ``H_SCALE_TOL`` of the oracle's.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import oracle.layer as OL
from oracle.codec import e4m3_decode, e4m3_encode
from tests.conftest import oracle_inputs, to_np

NEAR_TIE = 1e-5
W_TOL = 1e-5
# MXFP4 / MXFP8 weights are exact in bf16 and multiplied on the bf16 MFMA: the bf16
# bounds apply
OUT_TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 4e-2, "mxfp4": 2e-2, "mxfp8": 2e-2}
L2_TOL = {"f32": 1e-5, "bf16": 5e-3, "fp8": 8e-3, "mxfp4": 5e-3, "mxfp8": 5e-3}
H_SCALE_TOL = 1e-5     # relative, GPU h scale vs the oracle's amax / 448
H_TIE = 1e-5           # relative distance of an exact quotient from a code midpoint


@dataclass
class Report:
    tokens_checked: int = 0
    near_ties: int = 0
    near_tie_mismatch: int = 0
    hard_mismatch: int = 0
    max_w_err: float = 0.0
    out_err: float = 0.0
    out_err_rms: float = 0.0
    out_abs: float = 0.0
    rel_l2: float = 0.0
    out_err_raw: float = 0.0
    h_checked: int = 0
    h_ties: int = 0
    h_hard: int = 0
    h_scale_rel: float = 0.0
    failures: list = field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures


def out_error(o: np.ndarray, r: np.ndarray, floor_abs: float) -> float:
    """max |o - r| / max(|r|, floor_abs)."""
    if o.size == 0:
        return 0.0
    return float((np.abs(o - r) / np.maximum(np.abs(r), floor_abs)).max())


def gpu_out_values(out: torch.Tensor) -> np.ndarray:
    return out.detach().float().cpu().numpy().astype(np.float64)


def h_compare(pre, o_vals, o_scales, g_codes, g_scales, block: int = 128):
    """Compare the GPU's fp8 codes of some h rows with the oracle's.

    ``pre [n, I]``: exact (fp64) values before rounding; ``o_vals``,
    ``o_scales``: the oracle's rounded values and scales; ``g_codes``,
    ``g_scales``: the GPU's codes and scales of the same rows.  Returns
    ``(max relative scale difference, ties, hard)``: ``ties`` a list of
    ``(row, col, value)`` -- codes where the two sides differ at a near-tie,
    with the GPU's code in the oracle's scale -- and ``hard`` the number of
    differing codes away from a tie.
    """
    n, I = pre.shape
    so = np.repeat(np.asarray(o_scales, np.float64).reshape(n, -1), block, axis=1)
    sg = np.asarray(g_scales, np.float64).reshape(n, -1)
    srel = float((np.abs(sg - so[:, ::block]) / so[:, ::block]).max(initial=0.0))
    oc = e4m3_decode(e4m3_encode((o_vals / so).astype(np.float32)))   # oracle code values
    gc = e4m3_decode(g_codes)
    diff = oc != gc
    q = pre / so
    mid = 0.5 * (oc + gc)
    step = np.abs(oc - gc)
    # a tie: q lies between the two codes, within H_TIE of their midpoint
    # (the oracle's code being the nearest to q, the two are then neighbours)
    lo, hi = np.minimum(oc, gc), np.maximum(oc, gc)
    inside = (q >= lo) & (q <= hi)
    tie = diff & inside & (np.abs(q - mid) <= H_TIE * np.abs(q) + H_TIE * 2.0 ** -9) & (step > 0)
    r, c = np.nonzero(tie)
    ties = [(int(i), int(j), float(gc[i, j] * so[i, j])) for i, j in zip(r, c)]
    return srel, ties, int((diff & ~tie).sum())


class SortedRows:
    """fp8 codes and scales of a GPU intermediate whose rows are kept in
    sorted (by expert) order: ``rows(pairs)`` are the rows of those pairs
    (through ``slot_of_pair``; token order when it is None)."""

    def __init__(self, codes, scales, slot_of_pair=None, block=128):
        self.codes, self.scales, self.slot, self.block = codes, scales, slot_of_pair, block

    def rows(self, idx):
        idx = np.asarray(idx, dtype=np.int64)
        return idx if self.slot is None else self.slot[idx]


def check_layer(wl, inp, out, topk_idx, topk_w, tokens=None, debug=None,
                lazy=False) -> Report:
    """Compare one GPU forward with the oracle.

    ``tokens``: token subset for the output comparison (None = all).
    ``debug``: stage tensors from ``moe_forward_debug`` (optional).
    """
    spec, args = oracle_inputs(wl, inp, lazy=lazy)
    want_h = wl.dtype == "fp8" and debug is not None and "h" in debug
    ref = OL.forward(spec, **args, tokens=tokens, keep_h=want_h)
    rep = Report()
    g_idx = to_np(topk_idx).astype(np.int64)
    g_w = to_np(topk_w).astype(np.float64)
    o_idx = ref["idx"].astype(np.int64)
    m = g_idx.shape[0]
    # ---- top-k ----
    near = ref["gap"] < NEAR_TIE
    rep.near_ties = int(near.sum())
    diff = np.any(g_idx != o_idx, axis=1)
    rep.near_tie_mismatch = int((diff & near).sum())
    rep.hard_mismatch = int((diff & ~near).sum())
    if rep.hard_mismatch:
        bad = np.nonzero(diff & ~near)[0][:5]
        rep.failures.append(f"top-k mismatch on tokens {bad.tolist()} with gap >= {NEAR_TIE}")
    # weights: against the oracle's probabilities at the GPU's indices
    w_ref = OL.gate_weights(ref["prob"], g_idx, spec.renormalize, spec.routed_scale)
    rep.max_w_err = float(np.abs(g_w - w_ref).max(initial=0.0))
    if rep.max_w_err > W_TOL:
        rep.failures.append(f"topk_w error {rep.max_w_err:.3g} > {W_TOL}")
    # ---- output ----
    ref_out = ref
    if rep.near_tie_mismatch:
        ref_out = OL.forward(spec, **args, tokens=tokens, idx_override=g_idx, keep_h=want_h)
    tok = ref_out["tokens"]
    o = gpu_out_values(out)[tok]
    r = ref_out["out64"]
    rms = float(np.sqrt(np.mean(r ** 2))) if r.size else 0.0
    rep.tokens_checked = len(tok)
    rep.out_err = out_error(o, r, 0.1 * rms)
    rep.out_err_rms = out_error(o, r, rms)
    rep.rel_l2 = float(np.linalg.norm(o - r) / max(np.linalg.norm(r), 1e-300))
    rep.out_abs = float(np.abs(o - r).max(initial=0.0))
    rep.out_err_raw = rep.out_err
    if want_h:
        # fp8: the GPU's h codes against the oracle's; near-ties as choices
        slot = to_np(debug["slot_of_pair"]).astype(np.int64)
        routed = SortedRows(to_np(debug["h"]), to_np(debug["h_scale"]), slot, wl.block)
        pairs = sorted(ref_out["h_pre"])
        ties_r, ties_s = {}, {}
        if pairs:
            rows = routed.rows(pairs)
            srel, ties, hard = h_compare(np.stack([ref_out["h_pre"][p] for p in pairs]),
                                         np.stack([ref_out["h"][p] for p in pairs]),
                                         np.stack([ref_out["h_scale"][p] for p in pairs]),
                                         routed.codes[rows], routed.scales[rows], wl.block)
            rep.h_scale_rel, rep.h_hard = srel, hard
            rep.h_checked += len(pairs) * wl.inter
            for i, c, v in ties:
                cols, vals = ties_r.setdefault(pairs[i], ([], []))
                cols.append(c)
                vals.append(v)
        if wl.shared_inter > 0 and "h_shared" in debug:
            codes, scales = to_np(debug["h_shared"]), to_np(debug["h_shared_scale"])
            srel, ties, hard = h_compare(ref_out["h_sh_pre"], ref_out["h_sh"], ref_out["h_sh_scale"],
                                         codes[tok], scales[tok], wl.block)
            rep.h_scale_rel, rep.h_hard = max(rep.h_scale_rel, srel), rep.h_hard + hard
            rep.h_checked += len(tok) * wl.shared_inter
            for i, c, v in ties:
                cols, vals = ties_s.setdefault(int(tok[i]), ([], []))
                cols.append(c)
                vals.append(v)
        rep.h_ties = sum(len(v[0]) for v in ties_r.values()) + sum(len(v[0]) for v in ties_s.values())
        if rep.h_scale_rel > H_SCALE_TOL:
            rep.failures.append(f"h scale error {rep.h_scale_rel:.3g} > {H_SCALE_TOL}")
        if rep.h_ties:
            cond = OL.forward(spec, **args, tokens=tokens,
                              idx_override=g_idx if rep.near_tie_mismatch else None,
                              h_ties=(ties_r, ties_s))
            r = cond["out64"]
            rep.out_err = out_error(o, r, 0.1 * rms)
            rep.out_err_rms = out_error(o, r, rms)
            rep.out_abs = float(np.abs(o - r).max(initial=0.0))
    if not np.all(np.isfinite(o)):
        rep.failures.append("non-finite output")
    tol = OUT_TOL[wl.dtype]
    if rep.out_err > tol:
        rep.failures.append(f"output error {rep.out_err:.3g} > {tol}")
    if rep.rel_l2 > L2_TOL[wl.dtype]:
        rep.failures.append(f"relative L2 error {rep.rel_l2:.3g} > {L2_TOL[wl.dtype]}")
    # ---- stages ----
    if debug is not None:
        counts, offsets, sp, slot = OL.permute(g_idx.astype(np.int32), wl.experts)
        for name, want in (("counts", counts), ("offsets", offsets),
                           ("sorted_pair", sp), ("slot_of_pair", slot)):
            got = to_np(debug[name]).astype(np.int64)
            if not np.array_equal(got, want):
                rep.failures.append(f"{name} differs from the oracle permutation")
        if wl.dtype == "fp8" and "xq" in debug:
            if not np.array_equal(to_np(debug["xq"]), ref["xq"]):
                n = int((to_np(debug["xq"]) != ref["xq"]).sum())
                rep.failures.append(f"xq codes differ in {n} places")
            if not np.array_equal(to_np(debug["sx"]), ref["sx"]):
                rep.failures.append("sx differs")
        if "logits" in debug:
            lg = to_np(debug["logits"]).astype(np.float64)
            rel = np.abs(lg - ref["logits"]).max() / max(np.abs(ref["logits"]).max(), 1e-30)
            if rel > 1e-5:
                rep.failures.append(f"logits rel error {rel:.3g} > 1e-5")
    return rep


def debug_buffers(wl, m, device):
    """Stage-output tensors for ``moe_forward_debug``."""
    te, E, H = m * wl.topk, wl.experts, wl.hidden
    d = {"logits": torch.empty((m, E), dtype=torch.float32, device=device),
         "counts": torch.empty(E, dtype=torch.int32, device=device),
         "offsets": torch.empty(E + 1, dtype=torch.int32, device=device),
         "sorted_pair": torch.empty(te, dtype=torch.int32, device=device),
         "slot_of_pair": torch.empty(te, dtype=torch.int32, device=device)}
    if wl.dtype == "fp8":
        I, Is = wl.inter, wl.shared_inter
        d["xq"] = torch.empty((m, H), dtype=torch.uint8, device=device)
        d["sx"] = torch.empty((m, H // 128), dtype=torch.float32, device=device)
        d["h"] = torch.empty((te, I), dtype=torch.uint8, device=device)
        d["h_scale"] = torch.empty((te, I // 128), dtype=torch.float32, device=device)
        if Is > 0:
            d["h_shared"] = torch.empty((m, Is), dtype=torch.uint8, device=device)
            d["h_shared_scale"] = torch.empty((m, Is // 128), dtype=torch.float32, device=device)
    return d
