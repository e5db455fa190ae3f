"""Choose the two routing parameters of the synthetic workloads.

Runs the fp64 oracle's gating only (no GPU, no HIP library) and prints:

* the router sub-seed of ``prefill_bf16``: the first r = 0, 1, 2, ... for
  which every expert's token count lies within +-30 % of m*k/E (for m=1024,
  k=8, E=128: [45, 83]);
* the Zipf bias strength ``alpha`` of ``skew_fp8`` (a pure Zipf(1.2) bias)
  and of ``skew_head_fp8`` (the same with a fixed gap below the most popular
  expert): bisection so that the number of experts receiving no token is as
  close to 20 as the sample allows, then the top expert's share of the m*k
  assignments (asked > 10 %: skew_fp8 does not reach it, skew_head_fp8
  does).

The chosen values are written into ``synth/__init__.py`` by hand and
re-checked by ``tests/test_workloads.py``.

    python tests/golden/make_workload_params.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))

from oracle.codec import bf16_decode, bf16_encode  # noqa: E402
from oracle.layer import gate_scores, router_logits, top_k  # noqa: E402
import synth  # noqa: E402


def _bf16_vals(a32):
    return bf16_decode(bf16_encode(a32))


def counts_for(wl, subseed=None, alpha=None, logits=None):
    if logits is None:
        x = _bf16_vals(synth.draw_x(wl))
        wr = _bf16_vals(synth.draw_router(wl, subseed))
        logits = router_logits(x, wr)
    prob, score = gate_scores(logits, wl.gating)
    b = synth.draw_bias(wl, alpha)
    if b is not None:
        score = score + b.astype(np.float64)[None, :]
    idx, _ = top_k(score, wl.topk)
    return np.bincount(idx.reshape(-1), minlength=wl.experts), logits


def prefill_subseed():
    wl = synth.WORKLOADS["prefill_bf16"]
    mean = wl.m * wl.topk / wl.experts
    lo, hi = int(np.ceil(0.7 * mean)), int(np.floor(1.3 * mean))
    for r in range(200):
        c, _ = counts_for(wl, subseed=r)
        if c.min() >= lo and c.max() <= hi:
            print(f"prefill_bf16: router_subseed={r} counts in [{c.min()}, {c.max()}] "
                  f"(allowed [{lo}, {hi}])")
            return r
    raise SystemExit("no sub-seed found")


def skew_alpha(name):
    """The middle of the range of alpha that leaves 20 experts idle (at its
    edges a near-tie of the top-k decides one expert's only token)."""
    wl = synth.WORKLOADS[name]
    _, logits = counts_for(wl.replace(zipf_alpha=0.0))
    zeros = lambda a: int((counts_for(wl, alpha=a, logits=logits)[0] == 0).sum())

    def edge(target):   # smallest alpha with at least `target` idle experts
        lo, hi = 1e-4, 10.0
        for _ in range(60):
            mid = 0.5 * (lo + hi)
            if zeros(mid) < target:
                lo = mid
            else:
                hi = mid
        return hi

    a20, a21 = edge(20), edge(21)
    best = 0.5 * (a20 + a21)
    print(f"{name}: 20 idle experts for alpha in [{a20!r}, {a21!r})")
    c, _ = counts_for(wl, alpha=best, logits=logits)
    share = c.max() / c.sum()
    print(f"{name}: alpha={best!r} zero-token experts={int((c == 0).sum())} "
          f"top share={share:.4f} (top count {c.max()} of {c.sum()})")
    print("histogram (descending):", sorted(c.tolist(), reverse=True))
    return best


if __name__ == "__main__":
    prefill_subseed()
    skew_alpha("skew_fp8")        # pure Zipf(1.2) bias
    skew_alpha("skew_head_fp8")   # with the head gap
