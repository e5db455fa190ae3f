"""Pins of the oracle's layer forward (CPU only).

The sparse oracle (``oracle.layer``) is pinned against:

* brute-force dense evaluation (``oracle.dense``: every expert on every
  token, masked by the gate weights) on the tiny fp32 workload, on 60
  random tiny layers covering fp32 / bf16 / fp8, softmax / sigmoid, a
  selection bias, k = 1 and k = E, and a shared expert, and on 30 more
  covering the gating variants (sqrtsoftplus, softmax with a correction
  bias, no renormalisation, the sigmoid-gated shared blend);
* closed forms of the gating (renormalised softmax == softmax of the
  selected logits; weights sum to the routed scale; k = E gives the full
  softmax; x = 0 gives experts 0..k-1 with equal weights);
* library routines (``np.lexsort`` top-k, ``np.argsort(kind="stable")`` and
  ``np.bincount`` for the permutation, ``torch.nn.functional.silu`` for the
  one-expert reduction);
* symmetries (token permutation, expert relabelling, doubling w2).

The last tests plant mistakes in a copy of the oracle and check that these
pins catch them.
"""
import numpy as np
import pytest
import torch

import oracle.layer as OL
import synth
from oracle.codec import (bf16_decode, dequant_blocks, e2m1_decode, e4m3_decode,
                          e4m3_quantize_rows)
from oracle.dense import dense_forward
from tests.conftest import oracle_inputs, to_np


def _values(wl, inp):
    """Exact fp64 values of every input, decoded with the codec only."""
    def act(t):
        a = to_np(t)
        return a.astype(np.float64) if wl.dtype == "f32" else bf16_decode(a)

    def wt(t, s):
        a = to_np(t)
        if wl.dtype == "f32":
            return a.astype(np.float64)
        if wl.dtype == "bf16":
            return bf16_decode(a)
        if wl.dtype == "mxfp8":
            return e4m3_decode(a) * np.exp2(np.repeat(to_np(s).astype(np.float64) - 127.0, 32, axis=-1))
        if wl.dtype == "mxfp4":
            # unpacked here with shifts on the stacked array and a lookup
            # table of the element values, independently of mxfp4_decode
            table = e2m1_decode(np.arange(16))
            lo, hi = table[a & 15], table[a >> 4]
            vals = np.empty(a.shape[:-1] + (2 * a.shape[-1],))
            vals[..., 0::2], vals[..., 1::2] = lo, hi
            return vals * np.exp2(np.repeat(to_np(s).astype(np.float64) - 127.0, 32, axis=-1))
        s = to_np(s)
        if a.ndim == 3:
            return np.stack([dequant_blocks(a[e], s[e], wl.block) for e in range(a.shape[0])])
        return dequant_blocks(a, s, wl.block)

    x = act(inp["x"])
    if wl.dtype == "fp8":
        c, s = e4m3_quantize_rows(x.astype(np.float32), wl.block)
        xt = e4m3_decode(c) * np.repeat(s.astype(np.float64), wl.block, axis=1)
    else:
        xt = x
    out = dict(x=x, xt=xt, wr=act(inp["router_w"]),
               W13=wt(inp["w13"], inp["w13_scale"]), W2=wt(inp["w2"], inp["w2_scale"]))
    if wl.shared_inter:
        out["shared"] = (wt(inp["shared_w13"], inp["shared_w13_scale"]),
                         wt(inp["shared_w2"], inp["shared_w2_scale"]))
    if inp.get("shared_gate") is not None:
        out["gate"] = act(inp["shared_gate"])
    return out


def _dense(wl, inp):
    v = _values(wl, inp)
    logits = v["x"] @ v["wr"].T
    return dense_forward(v["xt"], logits, wl.topk, wl.gating, v["W13"], v["W2"],
                         wl.inter, wl.dtype, bias=to_np(inp["bias"]),
                         scale=wl.routed_scale, shared=v.get("shared"),
                         shared_inter=wl.shared_inter, block=wl.block,
                         renormalize=wl.renormalize, x_gate=v["x"], gate=v.get("gate"))


def _oracle(wl, inp, **kw):
    spec, args = oracle_inputs(wl, inp)
    return OL.forward(spec, **args, **kw)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _random_workloads(n=60):
    rng = np.random.default_rng(77)
    out = []
    for i in range(n):
        dt = ["f32", "bf16", "fp8"][i % 3]
        sizes = [128, 256] if dt == "fp8" else [32, 64, 128, 256]
        E = int(rng.integers(1, 17))
        k = int(rng.integers(1, E + 1))
        if i % 10 == 0:
            k = E
        gating = "sigmoid" if i % 2 else "softmax"
        wl = synth.Workload(f"rand{i}", m=int(rng.integers(1, 9)),
                            hidden=int(rng.choice(sizes)), experts=E, topk=k,
                            inter=int(rng.choice(sizes)),
                            shared_inter=int(rng.choice([0] + sizes)),
                            dtype=dt, gating=gating,
                            routed_scale=2.5 if gating == "sigmoid" else 1.0,
                            seed=1000 + i,
                            zipf_alpha=0.3 if (gating == "sigmoid" and i % 4 == 1) else 0.0,
                            zipf_head=0.2)
        out.append(wl)
    return out


def _variant_workloads(n=30):
    """Gating variants: sqrtsoftplus and softmax with a correction bias, no
    renormalisation, and the sigmoid-gated shared-expert blend."""
    rng = np.random.default_rng(78)
    out = []
    for i in range(n):
        dt = ["f32", "bf16", "fp8"][i % 3]
        sizes = [128, 256] if dt == "fp8" else [32, 64, 128]
        E = int(rng.integers(2, 17))
        k = int(rng.integers(1, E + 1))
        gating = ["sqrtsoftplus", "softmax", "sigmoid"][(i // 3) % 3]
        out.append(synth.Workload(
            f"var{i}", m=int(rng.integers(1, 9)), hidden=int(rng.choice(sizes)),
            experts=E, topk=k, inter=int(rng.choice(sizes)),
            shared_inter=int(rng.choice(sizes)) if i % 4 != 3 else 0,
            dtype=dt, gating=gating, routed_scale=float(rng.choice([1.0, 1.5, 2.5])),
            seed=2000 + i,
            # softmax probabilities are ~1/E: a bias of the same order
            zipf_alpha=(0.02 if gating == "softmax" else 0.3) if i % 2 == 0 else 0.0,
            zipf_head=0.0 if gating == "softmax" else 0.2,
            renormalize=(i % 5) != 1, shared_gate=(i % 4) in (0, 1)))
    return out


def test_tiny_workload_sparse_equals_dense():
    wl = synth.WORKLOADS["tiny_f32"]
    inp = synth.make_inputs(wl)
    r = _oracle(wl, inp)
    assert _rel(r["out64"], _dense(wl, inp)) < 1e-12


@pytest.mark.parametrize("wl", _random_workloads(), ids=lambda w: w.name)
def test_random_tiny_layers_sparse_equals_dense(wl):
    inp = synth.make_inputs(wl)
    r = _oracle(wl, inp)
    d = _dense(wl, inp)
    # ties in fp8 / bf16 rounding of h are computed identically on both
    # sides, so the two formulations agree to fp64 accumulation error
    assert _rel(r["out64"], d) < 1e-12


def _mxfp4_workloads(n=10):
    """MXFP4 expert weights (bf16 x, h and y): random tiny layers."""
    rng = np.random.default_rng(79)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 13))
        gating = ["softmax", "sigmoid", "sqrtsoftplus"][i % 3]
        out.append(synth.Workload(
            f"mx{i}", m=int(rng.integers(1, 9)), hidden=int(rng.choice([32, 64, 256])),
            experts=E, topk=int(rng.integers(1, E + 1)), inter=int(rng.choice([32, 96, 256])),
            shared_inter=int(rng.choice([0, 64, 256])), dtype="mxfp4", gating=gating,
            routed_scale=2.5 if gating != "softmax" else 1.0, seed=3000 + i,
            zipf_alpha=0.3 if i % 2 else 0.0, zipf_head=0.2, shared_gate=i % 4 == 0))
    return out


@pytest.mark.parametrize("wl", _mxfp4_workloads() + [
    w.replace(name=w.name.replace("mx", "mx8_"), dtype="mxfp8") for w in _mxfp4_workloads(6)],
    ids=lambda w: w.name)
def test_mxfp4_layers_sparse_equals_dense(wl):
    inp = synth.make_inputs(wl)
    r = _oracle(wl, inp)
    assert _rel(r["out64"], _dense(wl, inp)) < 1e-12


def test_mxfp4_one_expert_is_swiglu_mlp_on_decoded_weights():
    """k = 1 of a single MXFP4 expert: torch's silu on the decoded weights,
    h rounded to bf16 as the layer defines, the down output unrounded."""
    wl = synth.Workload("mx_one", m=5, hidden=64, experts=1, topk=1, inter=32,
                        shared_inter=0, dtype="mxfp4", gating="softmax",
                        routed_scale=1.0, seed=14)
    inp = synth.make_inputs(wl)
    r = _oracle(wl, inp)
    v = _values(wl, inp)
    x = torch.from_numpy(v["x"])
    w13, w2 = torch.from_numpy(v["W13"][0]), torch.from_numpy(v["W2"][0])
    h = (torch.nn.functional.silu(x @ w13[:32].T) * (x @ w13[32:].T)).to(torch.bfloat16).double()
    ref = h @ w2.T
    assert np.max(np.abs(r["out64"] - ref.numpy())) <= 1e-12 * np.abs(ref.numpy()).max()


@pytest.mark.parametrize("wl", _variant_workloads(), ids=lambda w: w.name)
def test_gating_variants_sparse_equals_dense(wl):
    inp = synth.make_inputs(wl)
    r = _oracle(wl, inp)
    assert _rel(r["out64"], _dense(wl, inp)) < 1e-12


# --------------------------------------------------------------- gating ---

def test_sqrtsoftplus_closed_forms():
    """sqrt(softplus): s(0)^2 = ln 2; s(l)^2 - s(-l)^2 = l (softplus(l) -
    softplus(-l) = l); s(l)^2 -> l for large l and -> e^l for very negative
    l; ranking equals logit ranking."""
    l = np.linspace(-30.0, 30.0, 601)[None, :]
    _, s = OL.gate_scores(l, "sqrtsoftplus")
    _, s0 = OL.gate_scores(np.zeros((1, 1)), "sqrtsoftplus")
    assert s0[0, 0] == pytest.approx(np.sqrt(np.log(2.0)), rel=1e-15)
    _, sn = OL.gate_scores(-l, "sqrtsoftplus")
    assert np.max(np.abs(s ** 2 - sn ** 2 - l)) < 1e-12
    _, big = OL.gate_scores(np.array([[60.0, -60.0]]), "sqrtsoftplus")
    assert big[0, 0] ** 2 == pytest.approx(60.0, rel=1e-15)
    assert big[0, 1] ** 2 == pytest.approx(np.exp(-60.0), rel=1e-12)
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((20, 32))
    idx, _ = OL.top_k(OL.gate_scores(lg, "sqrtsoftplus")[1], 6)
    for t in range(20):
        assert np.array_equal(idx[t], np.lexsort((np.arange(32), -lg[t]))[:6])


def test_softmax_correction_bias_selects_but_does_not_weight():
    """A large bias on experts {3, 9} forces them in with k = 2; the weights
    are the unbiased softmax probabilities (renormalised: the softmax of the
    two logits; not renormalised: scipy's softmax over all experts)."""
    from scipy.special import softmax
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((10, 16))
    b = np.zeros(16)
    b[[3, 9]] = 1.0
    p, score = OL.gate_scores(lg, "softmax")
    idx, _ = OL.top_k(score + b[None, :], 2)
    assert all(set(row) == {3, 9} for row in idx.tolist())
    w = OL.gate_weights(p, idx, True, 1.0)
    assert np.allclose(w, softmax(np.take_along_axis(lg, idx.astype(np.int64), 1), axis=1),
                       rtol=1e-14, atol=0)
    w_raw = OL.gate_weights(p, idx, False, 1.0)
    assert np.allclose(w_raw, np.take_along_axis(softmax(lg, axis=1), idx.astype(np.int64), 1),
                       rtol=1e-14, atol=0)


def test_shared_gate_zero_halves_the_shared_expert():
    """g = 0 gives the factor sigmoid(0) = 1/2 exactly: out = routed +
    (ungated - routed) / 2."""
    wl = synth.Workload("sg", m=7, hidden=64, experts=5, topk=2, inter=32,
                        shared_inter=64, dtype="bf16", gating="softmax",
                        routed_scale=1.0, seed=12, shared_gate=True)
    inp = synth.make_inputs(wl)
    spec, args = oracle_inputs(wl, inp)
    gated0 = dict(args, shared=dict(args["shared"], gate=np.zeros(64, np.uint16)))
    ungated = dict(args, shared=dict(args["shared"], gate=None))
    routed = dict(args, shared=None)
    o0 = OL.forward(spec, **gated0)["out64"]
    ou = OL.forward(spec, **ungated)["out64"]
    orr = OL.forward(spec, **routed)["out64"]
    assert np.max(np.abs(o0 - (orr + 0.5 * (ou - orr)))) < 1e-12 * np.abs(ou).max()
    # the factor uses the unquantised input and the stored gate values
    from scipy.special import expit
    r = OL.forward(spec, **args)
    xg = bf16_decode(to_np(inp["x"])) @ bf16_decode(to_np(inp["shared_gate"]))
    assert np.allclose(r["shared_gate"], expit(xg), rtol=1e-14, atol=0)



def test_softmax_renormalised_equals_softmax_of_selected(np_rng):
    logits = np_rng.standard_normal((50, 16)) * 2
    p, s = OL.gate_scores(logits, "softmax")
    idx, _ = OL.top_k(s, 4)
    w = OL.gate_weights(p, idx, True, 1.0)
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    ref = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
    assert np.max(np.abs(w - ref)) < 1e-14
    assert np.max(np.abs(w.sum(1) - 1)) < 1e-12


def test_sigmoid_weights_sum_to_scale(np_rng):
    logits = np_rng.standard_normal((50, 32)) * 2
    p, s = OL.gate_scores(logits, "sigmoid")
    ref = torch.sigmoid(torch.from_numpy(logits)).numpy()
    assert np.max(np.abs(p - ref)) < 1e-15
    idx, _ = OL.top_k(s, 8)
    w = OL.gate_weights(p, idx, True, 2.5)
    assert np.max(np.abs(w.sum(1) - 2.5)) < 1e-12


def test_k_equals_E_gives_full_softmax(np_rng):
    logits = np_rng.standard_normal((10, 8))
    p, s = OL.gate_scores(logits, "softmax")
    idx, gap = OL.top_k(s, 8)
    w = OL.gate_weights(p, idx, True, 1.0)
    full = torch.softmax(torch.from_numpy(logits), 1).numpy()
    assert np.max(np.abs(w - np.take_along_axis(full, idx.astype(np.int64), 1))) < 1e-15
    assert np.all(np.isinf(gap))


def test_zero_input_ties_break_to_lower_index():
    logits = np.zeros((3, 16))
    p, s = OL.gate_scores(logits, "softmax")
    idx, gap = OL.top_k(s, 5)
    assert np.array_equal(idx, np.tile(np.arange(5), (3, 1)))
    assert np.all(gap == 0)
    w = OL.gate_weights(p, idx, True, 1.0)
    assert np.allclose(w, 0.2, atol=1e-15)


def test_top_k_matches_lexsort(np_rng):
    # coarse values force many exact ties
    s = np.round(np_rng.standard_normal((200, 64)), 1)
    idx, gap = OL.top_k(s, 8)
    for t in range(200):
        order = np.lexsort((np.arange(64), -s[t]))
        assert np.array_equal(idx[t], order[:8])
        assert gap[t] == s[t, order[7]] - s[t, order[8]]


# --------------------------------------------------------- permutation ---

@pytest.mark.parametrize("m,k,E", [(1, 1, 1), (7, 3, 5), (64, 8, 128), (300, 8, 256)])
def test_permutation_invariants(m, k, E, np_rng):
    idx = np.stack([np_rng.choice(E, size=k, replace=False) for _ in range(m)]).astype(np.int32)
    counts, offsets, sp, slot = OL.permute(idx, E)
    e_of_p = idx.reshape(-1)
    assert np.array_equal(counts, np.bincount(e_of_p, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == m * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(sp, np.argsort(e_of_p, kind="stable"))
    assert np.array_equal(slot[sp], np.arange(m * k))
    for e in range(E):
        seg = sp[offsets[e]:offsets[e + 1]]
        assert np.all(e_of_p[seg] == e) and np.all(np.diff(seg) > 0)


# ------------------------------------------------------ reductions -------

def test_one_expert_top1_is_swiglu_mlp():
    wl = synth.Workload("one", m=5, hidden=64, experts=1, topk=1, inter=32,
                        shared_inter=0, dtype="f32", gating="softmax",
                        routed_scale=1.0, seed=9)
    inp = synth.make_inputs(wl)
    r = _oracle(wl, inp)
    x = inp["x"].double()
    w13, w2 = inp["w13"][0].double(), inp["w2"][0].double()
    ref = (torch.nn.functional.silu(x @ w13[:32].T) * (x @ w13[32:].T)) @ w2.T
    # nothing is rounded in the fp32 layer before the output
    assert np.max(np.abs(r["out64"] - ref.numpy())) < 1e-12 * np.abs(ref.numpy()).max()
    assert np.all(r["w"] == 1.0)


def test_shared_only_contribution_and_unit_weight():
    """With w2 of all routed experts zeroed, out == shared SwiGLU MLP."""
    wl = synth.Workload("sh", m=6, hidden=64, experts=4, topk=2, inter=32,
                        shared_inter=64, dtype="f32", gating="softmax",
                        routed_scale=1.0, seed=11)
    inp = synth.make_inputs(wl)
    inp["w2"].zero_()
    r = _oracle(wl, inp)
    x = inp["x"].double()
    s13, s2 = inp["shared_w13"].double(), inp["shared_w2"].double()
    ref = (torch.nn.functional.silu(x @ s13[:64].T) * (x @ s13[64:].T)) @ s2.T
    assert np.max(np.abs(r["out64"] - ref.numpy())) < 1e-6 * np.abs(ref.numpy()).max()


def test_kept_h_rounds_the_pre_rounding_values():
    """fp8 intermediates: each kept value is the rounding of its exact value
    (within one e4m3 step of the row's scale)."""
    wl = synth.Workload("hov", m=9, hidden=256, experts=5, topk=2, inter=256,
                        shared_inter=128, dtype="fp8", gating="sigmoid",
                        routed_scale=2.5, seed=13)
    inp = synth.make_inputs(wl)
    spec, args = oracle_inputs(wl, inp)
    r = OL.forward(spec, **args, keep_h=True)
    te = wl.m * wl.topk
    h = np.stack([r["h"][p] for p in range(te)])
    assert np.all(np.abs(np.stack([r["h_pre"][p] for p in range(te)]) - h) <=
                  np.abs(h) * 2.0 ** -3 + 2.0 ** -9 * np.repeat(
                      np.stack([r["h_scale"][p] for p in range(te)]), 128, axis=1))


def test_h_ties_with_own_values_are_the_identity():
    """A near-tie choice equal to the oracle's own rounded value changes
    nothing; the neighbouring code at one position changes the output of
    that pair's token only."""
    wl = synth.Workload("ties", m=9, hidden=256, experts=5, topk=2, inter=256,
                        shared_inter=128, dtype="fp8", gating="sigmoid",
                        routed_scale=2.5, seed=13)
    inp = synth.make_inputs(wl)
    spec, args = oracle_inputs(wl, inp)
    r = OL.forward(spec, **args, keep_h=True)
    p, c = 5, 17
    same = OL.forward(spec, **args, h_ties=({p: ([c], [r["h"][p][c]])}, {3: ([4], [r["h_sh"][3][4]])}))
    assert np.array_equal(same["out64"], r["out64"])
    other = r["h"][p][c] * (1 + 2.0 ** -3)
    moved = OL.forward(spec, **args, h_ties=({p: ([c], [other])}, {}))
    changed = np.nonzero(np.any(moved["out64"] != r["out64"], axis=1))[0]
    assert changed.tolist() == [p // wl.topk]


# ---------------------------------------------------------- symmetries ---

def test_token_permutation_equivariance():
    wl = synth.Workload("tp", m=8, hidden=128, experts=6, topk=3, inter=128,
                        shared_inter=128, dtype="fp8", gating="sigmoid",
                        routed_scale=2.5, seed=21)
    inp = synth.make_inputs(wl)
    r = _oracle(wl, inp)
    perm = np.random.default_rng(3).permutation(8)
    inp2 = dict(inp)
    inp2["x"] = inp["x"][torch.from_numpy(perm)]
    r2 = _oracle(wl, inp2)
    assert np.array_equal(r2["idx"], r["idx"][perm])
    assert np.max(np.abs(r2["w"] - r["w"][perm])) < 1e-15
    assert _rel(r2["out64"], r["out64"][perm]) < 1e-12


def test_expert_relabelling():
    wl = synth.Workload("rl", m=8, hidden=64, experts=7, topk=2, inter=64,
                        shared_inter=0, dtype="bf16", gating="softmax",
                        routed_scale=1.0, seed=22)
    inp = synth.make_inputs(wl)
    r = _oracle(wl, inp)
    pi = np.random.default_rng(5).permutation(7)       # new label e' holds old pi[e']
    inp2 = dict(inp)
    t = torch.from_numpy(pi)
    inp2["router_w"], inp2["w13"], inp2["w2"] = inp["router_w"][t], inp["w13"][t], inp["w2"][t]
    r2 = _oracle(wl, inp2)
    inv = np.argsort(pi)
    # the same old experts are selected, in the same order
    assert np.array_equal(pi[r2["idx"]], r["idx"])
    assert np.array_equal(r2["idx"], inv[r["idx"]])
    assert _rel(r2["out64"], r["out64"]) < 1e-12


def test_doubling_w2_doubles_output_exactly():
    wl = synth.Workload("x2", m=4, hidden=64, experts=4, topk=2, inter=64,
                        shared_inter=64, dtype="bf16", gating="softmax",
                        routed_scale=1.0, seed=23)
    inp = synth.make_inputs(wl)
    r = _oracle(wl, inp)
    inp2 = dict(inp)
    inp2["w2"] = inp["w2"] * 2
    inp2["shared_w2"] = inp["shared_w2"] * 2
    r2 = _oracle(wl, inp2)
    assert np.array_equal(r2["out64"], 2 * r["out64"])


def test_token_subset_and_idx_override():
    wl = synth.WORKLOADS["tiny_f32"]
    inp = synth.make_inputs(wl)
    full = _oracle(wl, inp)
    sub = _oracle(wl, inp, tokens=[3, 1])
    assert np.array_equal(sub["tokens"], [1, 3])
    # BLAS may block a 2-row product differently from a 4-row one
    assert _rel(sub["out64"], full["out64"][[1, 3]]) < 1e-14
    same = _oracle(wl, inp, idx_override=full["idx"])
    assert np.array_equal(same["out64"], full["out64"])


# ------------------------------------------------- planted mistakes -------

def _dense_mismatch(monkeypatch, attr, fn):
    monkeypatch.setattr(OL, attr, fn)
    bad = 0
    for wl in _random_workloads(12):
        inp = synth.make_inputs(wl)
        try:
            r = _oracle(wl, inp)
        except Exception:
            bad += 1
            continue
        bad += _rel(r["out64"], _dense(wl, inp)) > 1e-9
    return bad


def test_planted_wrong_activation_is_caught(monkeypatch):
    assert _dense_mismatch(monkeypatch, "silu", lambda z: z / (1 + np.exp(z))) > 0


def test_planted_unnormalised_weights_are_caught(monkeypatch):
    orig = OL.gate_weights
    assert _dense_mismatch(monkeypatch, "gate_weights",
                           lambda p, i, r, s: orig(p, i, False, s)) > 0


def test_planted_swapped_gate_up_is_caught(monkeypatch):
    orig = OL.expert_mlp

    def swapped(a, w13, w2, inter, dt, blk):
        return orig(a, np.concatenate([w13[inter:], w13[:inter]]), w2, inter, dt, blk)
    assert _dense_mismatch(monkeypatch, "expert_mlp", swapped) > 0


def test_planted_dropped_shared_expert_is_caught(monkeypatch):
    orig = OL.forward

    def no_shared(spec, *a, **kw):
        kw["shared"] = None
        return orig(spec, *a, **kw)
    monkeypatch.setattr(OL, "forward", no_shared)
    bad = 0
    for wl in _random_workloads(12):
        if wl.shared_inter == 0:
            continue
        inp = synth.make_inputs(wl)
        bad += _rel(_oracle(wl, inp)["out64"], _dense(wl, inp)) > 1e-9
    assert bad > 0


def _variant_mismatch(monkeypatch, attr, fn, n=12):
    monkeypatch.setattr(OL, attr, fn)
    bad = 0
    for wl in _variant_workloads(n):
        inp = synth.make_inputs(wl)
        bad += _rel(_oracle(wl, inp)["out64"], _dense(wl, inp)) > 1e-9
    return bad


def test_planted_sqrtsoftplus_sign_error_is_caught(monkeypatch):
    orig = OL.gate_scores

    def wrong(l, gating):
        if gating == "sqrtsoftplus":
            s = np.sqrt(np.logaddexp(0.0, -l))
            return s, s
        return orig(l, gating)
    assert _variant_mismatch(monkeypatch, "gate_scores", wrong) > 0


def test_planted_biased_weights_are_caught(monkeypatch):
    """Weights taken from the biased score instead of the unbiased one."""
    orig_top_k = OL.top_k
    seen = {}

    def top_k_keep(score, k):
        seen["score"] = score
        return orig_top_k(score, k)
    orig_w = OL.gate_weights
    monkeypatch.setattr(OL, "top_k", top_k_keep)
    assert _variant_mismatch(monkeypatch, "gate_weights",
                             lambda p, i, r, s: orig_w(seen["score"], i, r, s)) > 0


def test_planted_ignored_shared_gate_is_caught(monkeypatch):
    orig = OL.forward

    def no_gate(spec, *a, **kw):
        if kw.get("shared") is not None:
            kw["shared"] = dict(kw["shared"], gate=None)
        return orig(spec, *a, **kw)
    monkeypatch.setattr(OL, "forward", no_gate)
    bad = 0
    for wl in _variant_workloads(12):
        if not wl.shared_gate or wl.shared_inter == 0:
            continue
        inp = synth.make_inputs(wl)
        bad += _rel(_oracle(wl, inp)["out64"], _dense(wl, inp)) > 1e-9
    assert bad > 0


def test_planted_high_index_tie_break_is_caught(np_rng):
    s = np.round(np_rng.standard_normal((50, 64)), 1)

    def wrong_top_k(score, k):   # ties resolved towards the higher index
        E = score.shape[1]
        order = E - 1 - np.argsort(-score[:, ::-1], axis=1, kind="stable")
        return order[:, :k]
    wrong = wrong_top_k(s, 8)
    assert any(not np.array_equal(wrong[t], np.lexsort((np.arange(64), -s[t]))[:8])
               for t in range(50))


def test_planted_unstable_permutation_is_caught(np_rng):
    idx = np_rng.integers(0, 4, size=(40, 2)).astype(np.int32)
    e_of_p = idx.reshape(-1)
    wrong = np.argsort(e_of_p, kind="stable")
    for e in range(4):                    # reverse order inside each segment
        sel = e_of_p[wrong] == e
        wrong[sel] = wrong[sel][::-1]
    _, _, sp, _ = OL.permute(idx, 4)
    assert not np.array_equal(wrong, sp)
    assert np.array_equal(sp, np.argsort(e_of_p, kind="stable"))
