"""GPU parity: the HIP layer (through the C ABI) against the fp64 oracle.

Every workload runs on seeded synthetic inputs; each case prints its name
before it touches the GPU.  Full-size workloads compare every token where the
oracle is quick (decode, prefill) and a fixed token sample otherwise (the
large fp8 shapes); reduced shapes that still span several M tiles, partial N
tiles and ragged token counts compare every element on every path.
"""
import numpy as np
import pytest
import torch

import synth
from mixture_experts_ffn_06_amd import MoeLayer
from tests.conftest import to_np
from tests.parity import check_layer, debug_buffers

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def make_layer(wl, inp, path="auto", max_tokens=None):
    w = {k: v for k, v in inp.items() if k != "x" and v is not None}
    return MoeLayer(w, hidden=wl.hidden, num_experts=wl.experts, inter=wl.inter,
                    topk=wl.topk, max_tokens=max_tokens or inp["x"].shape[0],
                    shared_inter=wl.shared_inter, gating=wl.gating,
                    renormalize=wl.renormalize, routed_scale=wl.routed_scale,
                    weight_dtype=wl.dtype, path=path)


def run_case(wl, path="auto", m=None, tokens=None, lazy=False, inp=None):
    _say(f"case {wl.name} m={m or wl.m} path={path} tokens={'all' if tokens is None else len(tokens)}")
    if inp is None:
        inp = synth.make_inputs(wl, device=DEV, m=m)
    mm = inp["x"].shape[0]
    layer = make_layer(wl, inp, path)
    if path != "auto":
        assert layer.plan.path_for(mm) == path
    dbg = debug_buffers(wl, mm, DEV)
    out, idx, w = layer(inp["x"], debug=dbg)
    torch.cuda.synchronize()
    rep = check_layer(wl, inp, out, idx, w, tokens=tokens, debug=dbg, lazy=lazy)
    _say(f"  -> {rep}")
    assert rep.ok(), rep.failures
    return rep, layer, inp, (out, idx, w, dbg)


# ------------------------------------------------------------ workloads ---

def test_tiny_f32():
    run_case(synth.WORKLOADS["tiny_f32"])


@pytest.mark.parametrize("path", ["small_m", "grouped", "simple"])
@pytest.mark.parametrize("m", [1, 4, 16])
def test_decode_bf16(m, path):
    run_case(synth.WORKLOADS["decode_bf16"], path=path, m=m)


def test_prefill_bf16_all_tokens():
    rep, *_ = run_case(synth.WORKLOADS["prefill_bf16"], path="grouped")
    assert rep.tokens_checked == 1024


def _sample(m, n=6, seed=0):
    rng = np.random.default_rng(seed)
    return sorted({0, m - 1, *rng.choice(m, size=n, replace=False).tolist()})


def cover_experts(idx, experts, seed=0):
    """Tokens whose top-k choices together reach every expert in ``experts``
    (greedy: each pick reaches the most experts not yet reached; ties to a
    seeded random order)."""
    idx = np.asarray(idx)
    rng = np.random.default_rng(seed)
    order = rng.permutation(idx.shape[0])
    left, picked = set(int(e) for e in experts), []
    while left:
        gain = [(len(left.intersection(idx[t].tolist())), -i, t) for i, t in enumerate(order)]
        g, _, t = max(gain)
        if g == 0:
            break
        picked.append(int(t))
        left -= set(idx[t].tolist())
    return sorted(picked)


# Full-size fp8 layers are run once per module; the sampled comparisons are
# split into shards, each covering the active experts e with e % SHARDS ==
# shard (so that every active expert's tiles are compared with the oracle
# across the shards, and no single test runs the oracle for long).
SHARDS = 4
_RUNS = {}


def _full_size_run(name, m=None):
    if name not in _RUNS:
        wl = synth.WORKLOADS[name]
        _say(f"case {name}: full-size forward")
        inp = synth.make_inputs(wl, device=DEV, m=m)
        layer = make_layer(wl, inp, "grouped")
        mm = inp["x"].shape[0]
        dbg = debug_buffers(wl, mm, DEV)
        out, idx, w = layer(inp["x"], debug=dbg)
        torch.cuda.synchronize()
        _RUNS.clear()                      # one full-size layer held at a time
        _RUNS[name] = (wl, inp, out, idx, w, dbg)
    return _RUNS[name]


def _sampled_shard(name, shard, extra=()):
    wl, inp, out, idx, w, dbg = _full_size_run(name)
    g_idx = to_np(idx)
    counts = to_np(dbg["counts"])
    active = [e for e in range(wl.experts) if counts[e] > 0 and e % SHARDS == shard]
    tokens = sorted(set(cover_experts(g_idx, active, seed=shard)) | set(extra))
    _say(f"case {name} shard {shard}: {len(active)} experts, {len(tokens)} tokens")
    rep = check_layer(wl, inp, out, idx, w, tokens=tokens, debug=dbg, lazy=True)
    _say(f"  -> {rep}")
    assert rep.ok(), rep.failures
    reached = set(g_idx[tokens].reshape(-1).tolist())
    assert set(active) <= reached
    return rep, counts


@pytest.mark.timeout(600)
@pytest.mark.parametrize("shard", range(SHARDS))
def test_large_fp8_sampled(shard):
    """Every active expert of the large fp8 layer (4096 tokens, 256 experts)
    reached by the checked tokens, over the shards; plus the first and the
    last token."""
    _sampled_shard("large_fp8", shard, extra=(0, 4095) if shard == 0 else ())


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,shard", [("skew_fp8", s) for s in range(SHARDS)] + [("skew_head_fp8", 0)])
def test_skew_fp8_sampled(name, shard):
    """Skewed routing: every active expert of C5 (pure Zipf bias) reached
    over the shards; the supplementary hot-expert draw on one shard.  Each
    shard adds 16 tokens of the busiest expert (with the hot expert its rows
    span 13 M tiles)."""
    wl, inp, out, idx, w, dbg = _full_size_run(name)
    counts = to_np(dbg["counts"])
    hot = int(np.argmax(counts))
    g_idx = to_np(idx)
    on_hot = np.nonzero((g_idx == hot).any(axis=1))[0]
    rng = np.random.default_rng(100 + shard)
    extra = rng.choice(on_hot, size=min(16, len(on_hot)), replace=False).tolist()
    _sampled_shard(name, shard, extra=extra)
    assert int((counts == 0).sum()) == 20
    if name == "skew_head_fp8":
        assert counts.max() / counts.sum() > 0.10


@pytest.mark.parametrize("name", ["dense_bf16", "dense_fp8"])
def test_mfma_bound_sampled(name):
    """About 1024 (bf16) / 512 (fp8) rows per expert: several M tiles per
    expert on the large-tile configurations."""
    wl = synth.WORKLOADS[name]
    run_case(wl, path="grouped", tokens=_sample(wl.m, seed=2), lazy=True)


# ------------------------------------------- reduced shapes, all elements ---

RAGGED_FP8 = synth.Workload("ragged_fp8", m=300, hidden=512, experts=16, topk=4,
                            inter=256, shared_inter=384, dtype="fp8",
                            gating="sigmoid", routed_scale=2.5, seed=31,
                            zipf_alpha=0.3, zipf_head=0.2)
RAGGED_BF16 = synth.Workload("ragged_bf16", m=200, hidden=288, experts=8, topk=3,
                             inter=96, shared_inter=160, dtype="bf16",
                             gating="softmax", routed_scale=1.0, seed=32)
SIGMOID_BF16 = synth.Workload("sigmoid_bf16", m=77, hidden=256, experts=32, topk=6,
                              inter=128, shared_inter=0, dtype="bf16",
                              gating="sigmoid", routed_scale=2.5, seed=33,
                              zipf_alpha=0.2, zipf_head=0.1)


@pytest.mark.parametrize("path", ["grouped", "simple"])
def test_ragged_fp8_all(path):
    run_case(RAGGED_FP8, path=path)


@pytest.mark.parametrize("path", ["grouped", "simple"])
def test_ragged_bf16_all(path):
    run_case(RAGGED_BF16, path=path)


# More than 96 rows per expert on average: the large-tile configurations
# (bf16 gate/up 256-row tiles, bf16 down 128-row, fp8 192-row tiles), with
# experts of 61-368 rows, so some span two or three M tiles and the last
# tile of each is partly filled.
BIG_FP8 = synth.Workload("big_fp8", m=600, hidden=256, experts=8, topk=2, inter=256,
                         shared_inter=128, dtype="fp8", gating="sigmoid", routed_scale=2.5,
                         seed=37, zipf_alpha=0.05)
BIG_BF16 = synth.Workload("big_bf16", m=600, hidden=288, experts=8, topk=2, inter=96,
                          shared_inter=160, dtype="bf16", gating="sigmoid", routed_scale=1.0,
                          seed=38, zipf_alpha=0.05)


@pytest.mark.parametrize("wl", [BIG_FP8, BIG_BF16], ids=["fp8", "bf16"])
def test_large_tiles_all(wl):
    rep, *_, (out, idx, w, dbg) = run_case(wl, path="grouped")
    counts = to_np(dbg["counts"])
    assert wl.m * wl.topk > 96 * wl.experts       # the large-tile configurations
    assert counts.max() > 256 and counts.min() < 96


@pytest.mark.parametrize("m", [1, 7, 13, 16])
def test_small_m_with_shared_expert(m):
    run_case(RAGGED_BF16, path="small_m", m=m)


@pytest.mark.parametrize("wl", [RAGGED_BF16.replace(name="ragged_bf16_40", m=40),
                                RAGGED_BF16.replace(name="ragged_bf16_128", m=128),
                                RAGGED_BF16.replace(name="ragged_bf16_256", m=256),
                                SIGMOID_BF16], ids=["ragged40", "ragged128", "ragged256", "sigmoid77"])
def test_small_m_above_16_tokens(wl):
    """bf16 weights above 16 tokens stream each expert's rows in blocks of
    16 (the shared expert's 40 or 77 rows: a partial last block)."""
    run_case(wl, path="small_m")


@pytest.mark.timeout(300)
def test_decode_bf16_64_tokens_small_m_all():
    wl = synth.WORKLOADS["decode_bf16"].replace(name="decode_bf16_64", m=64)
    run_case(wl, path="small_m", lazy=True)


@pytest.mark.timeout(300)
def test_decode_bf16_256_tokens_small_m_all():
    """The streaming path at its bf16 limit, every token: experts of up to
    ~30 rows, two or three 16-row blocks each."""
    wl = synth.WORKLOADS["decode_bf16"].replace(name="decode_bf16_256", m=256)
    run_case(wl, path="small_m", lazy=True)


@pytest.mark.parametrize("path", ["grouped", "small_m"])
def test_sigmoid_bias_bf16(path):
    run_case(SIGMOID_BF16, path=path, m=16 if path == "small_m" else None)


MAX_EK = synth.Workload("max_E_k", m=20, hidden=256, experts=1024, topk=32, inter=128,
                        shared_inter=64, dtype="bf16", gating="sigmoid", routed_scale=2.5,
                        seed=46, zipf_alpha=0.05)


@pytest.mark.parametrize("path", ["grouped", "small_m", "simple"])
def test_max_experts_and_topk(path):
    """E = 1024 and k = 32, the plan's limits: 16 experts per lane in the
    top-k, the fused routing kernel of small batches near its LDS bound."""
    run_case(MAX_EK, path=path, m=16 if path == "small_m" else None)


def test_k_equals_E():
    wl = synth.Workload("k_eq_E", m=40, hidden=128, experts=4, topk=4, inter=64,
                        shared_inter=0, dtype="bf16", gating="softmax",
                        routed_scale=1.0, seed=34)
    run_case(wl, path="grouped")


def test_one_expert_top1():
    wl = synth.Workload("one", m=130, hidden=256, experts=1, topk=1, inter=128,
                        shared_inter=128, dtype="fp8", gating="softmax",
                        routed_scale=1.0, seed=35)
    run_case(wl, path="grouped")


def test_empty_experts_many_tiles():
    """Few tokens over many experts: most groups are empty."""
    wl = synth.Workload("sparse", m=20, hidden=256, experts=256, topk=2, inter=128,
                        shared_inter=128, dtype="fp8", gating="sigmoid",
                        routed_scale=1.0, seed=36)
    rep, *_, (out, idx, w, dbg) = run_case(wl, path="grouped")
    assert int((to_np(dbg["counts"]) == 0).sum()) >= 256 - 40


# Exact per-expert row counts around the gate/up tile edges (32-row token
# blocks, 160-row M tiles split evenly: 129 and 159 rows fill five blocks
# partly, 160 all five, 161 and 321 rows split into two and three tiles).
# Top-1 routing by construction: router row e is the unit vector at column
# e and token t carries a clear maximum at its expert's column, so the
# logits are x[t, :E] and every token's choice is far from a tie.
TILE_COUNTS = (1, 31, 129, 159, 160, 161, 320, 321, 0)


def _counted_inputs(wl, counts, seed):
    inp = synth.make_inputs(wl, device=DEV)
    rng = np.random.default_rng(seed)
    m, H, E = sum(counts), wl.hidden, wl.experts
    x = rng.standard_normal((m, H)).astype(np.float32)
    x[:, :E] = np.clip(0.5 * x[:, :E], -2.0, 2.0)
    owner = np.repeat(np.arange(E), counts)
    x[np.arange(m), owner] = 4.0
    rw = np.zeros((E, H), dtype=np.float32)
    rw[np.arange(E), np.arange(E)] = 1.0
    inp["x"] = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    inp["router_w"] = torch.from_numpy(rw).to(torch.bfloat16).to(DEV)
    return inp, owner


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_gateup_tile_edges_exact_counts(dtype):
    m = sum(TILE_COUNTS)
    wl = synth.Workload(f"tile_edges_{dtype}", m=m, hidden=256, experts=len(TILE_COUNTS), topk=1,
                        inter=256, shared_inter=128, dtype=dtype, gating="softmax",
                        routed_scale=1.0, seed=50)
    inp, owner = _counted_inputs(wl, TILE_COUNTS, seed=51)
    rep, *_, (out, idx, w, dbg) = run_case(wl, path="grouped", inp=inp)
    assert (to_np(idx)[:, 0] == owner).all()
    assert to_np(dbg["counts"]).tolist() == list(TILE_COUNTS)


# ------------------------------------------------------ gating variants ---
# sqrtsoftplus and softmax with a correction bias, no renormalisation, and
# the sigmoid-gated shared-expert blend (page 3, top-k dispatch and step 8).

SQRTSP_BF16 = synth.Workload("sqrtsp_bf16", m=77, hidden=256, experts=32, topk=6,
                             inter=128, shared_inter=160, dtype="bf16",
                             gating="sqrtsoftplus", routed_scale=1.5, seed=40,
                             zipf_alpha=0.2, zipf_head=0.1, shared_gate=True)
SOFTMAX_BIAS_BF16 = synth.Workload("softmax_bias_bf16", m=77, hidden=256, experts=32,
                                   topk=6, inter=128, shared_inter=96, dtype="bf16",
                                   gating="softmax", routed_scale=1.0, seed=41,
                                   zipf_alpha=0.005, renormalize=False)
GATED_FP8 = synth.Workload("gated_fp8", m=300, hidden=512, experts=16, topk=4,
                           inter=256, shared_inter=384, dtype="fp8",
                           gating="sqrtsoftplus", routed_scale=2.5, seed=42,
                           zipf_alpha=0.3, zipf_head=0.2, shared_gate=True)
GATED_F32 = synth.Workload("gated_f32", m=9, hidden=64, experts=8, topk=2, inter=32,
                           shared_inter=64, dtype="f32", gating="softmax",
                           routed_scale=1.0, seed=43, zipf_alpha=0.01,
                           renormalize=False, shared_gate=True)


@pytest.mark.parametrize("path", ["grouped", "small_m", "simple"])
def test_sqrtsoftplus_bias_gated_shared_bf16(path):
    run_case(SQRTSP_BF16, path=path, m=16 if path == "small_m" else None)


@pytest.mark.parametrize("path", ["grouped", "small_m"])
def test_softmax_bias_unrenormalised_bf16(path):
    run_case(SOFTMAX_BIAS_BF16, path=path, m=13 if path == "small_m" else None)


@pytest.mark.parametrize("path", ["grouped", "simple"])
def test_sqrtsoftplus_gated_shared_fp8(path):
    run_case(GATED_FP8, path=path)


def test_gated_shared_unrenormalised_f32():
    run_case(GATED_F32)


def test_prefill_gated_shared_full_size():
    """The prefill layer with the sigmoid-gated shared blend, every token."""
    wl = synth.WORKLOADS["prefill_bf16"].replace(name="prefill_gated", shared_gate=True)
    run_case(wl, path="grouped")


def test_large_fp8_sqrtsoftplus_gated_shared_sampled():
    """H = 7168: every token's row spans four combine blocks, each forming
    the gate's dot product itself; sqrtsoftplus with a selection bias."""
    wl = synth.WORKLOADS["large_fp8"].replace(name="large_gated", m=512, gating="sqrtsoftplus",
                                              zipf_alpha=0.05, shared_gate=True)
    run_case(wl, path="grouped", tokens=_sample(wl.m, seed=3), lazy=True)


def test_decode_sqrtsoftplus_bias_full_size():
    wl = synth.WORKLOADS["decode_bf16"].replace(name="decode_sqrtsp", gating="sqrtsoftplus",
                                                routed_scale=2.5, zipf_alpha=0.05)
    run_case(wl, path="small_m")


# ---------------------------------------------------------- MXFP4 experts ---
# OCP MX FP4 weights with E8M0 scales on the weight-streaming path.

MX_SMALL = synth.Workload("mx_small", m=16, hidden=512, experts=16, topk=4, inter=256,
                          shared_inter=256, dtype="mxfp4", gating="sqrtsoftplus",
                          routed_scale=2.5, seed=44, zipf_alpha=0.3, zipf_head=0.2,
                          shared_gate=True)


@pytest.mark.parametrize("m", [1, 4, 16])
def test_decode_mxfp4(m):
    run_case(synth.WORKLOADS["decode_mxfp4"], path="small_m", m=m)


@pytest.mark.parametrize("m", [1, 7, 13, 16])
def test_mxfp4_shared_gated_small(m):
    run_case(MX_SMALL, path="small_m", m=m)


@pytest.mark.parametrize("m", [1, 4, 16])
def test_decode_mxfp8(m):
    run_case(synth.WORKLOADS["decode_mxfp8"], path="small_m", m=m)


@pytest.mark.parametrize("m", [1, 7, 16])
def test_mxfp8_shared_gated_small(m):
    run_case(MX_SMALL.replace(name="mx8_small", dtype="mxfp8", inter=384, shared_inter=128),
             path="small_m", m=m)


# Long rows (H = 4096, I = I_s = 1536): gate/up items of 16 (MXFP4) and 32
# (MXFP8) stages split over four waves, down items of 6 and 12 stages split
# over two and four waves; the decode-size layers keep one wave per MXFP4
# gate/up item.
MX_WIDE = MX_SMALL.replace(name="mx_wide", hidden=4096, experts=8, topk=2, inter=1536,
                           shared_inter=1536)


@pytest.mark.parametrize("fmt,m", [("mxfp4", 16), ("mxfp4", 5), ("mxfp8", 16)])
def test_mx_long_rows_split_over_waves(fmt, m):
    run_case(MX_WIDE.replace(name=f"{fmt}_wide", dtype=fmt), path="small_m", m=m)


@pytest.mark.parametrize("fmt,m", [("mxfp4", 40), ("mxfp4", 128), ("mxfp8", 33)])
def test_mx_above_16_tokens_on_the_streaming_path(fmt, m):
    """Above 16 tokens the MX streaming kernels take each expert's rows in
    blocks of 16 (33 tokens: a last block of one shared-expert row)."""
    run_case(MX_SMALL.replace(name=f"{fmt}_rows", m=m, dtype=fmt), path="small_m")


@pytest.mark.parametrize("fmt,m", [("mxfp4", 128), ("mxfp4", 1024), ("mxfp8", 300)])
def test_mx_streaming_many_tokens_sampled(fmt, m):
    """Full-size MX layers at prefill-sized batches (up to 64 row blocks per
    expert), checked on sampled tokens."""
    wl = synth.WORKLOADS[f"decode_{fmt}"].replace(name=f"decode_{fmt}_{m}", m=m)
    run_case(wl, path="small_m", tokens=_sample(m), lazy=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt,m", [("mxfp4", 2048), ("mxfp8", 2048), ("mxfp4", 4096)])
def test_mx_large_batches_every_expert(fmt, m):
    """MX weights above 1024 tokens stay on the streaming path (experts of
    ~128-256 rows: 8-16 row blocks each); the checked tokens' top-k reaches
    every active expert."""
    wl = synth.WORKLOADS[f"decode_{fmt}"].replace(name=f"decode_{fmt}_{m}", m=m)
    inp = synth.make_inputs(wl, device=DEV)
    layer = make_layer(wl, inp, "auto")
    assert layer.plan.path_for(m) == "small_m"
    dbg = debug_buffers(wl, m, DEV)
    out, idx, w = layer(inp["x"], debug=dbg)
    torch.cuda.synchronize()
    g_idx, counts = to_np(idx), to_np(dbg["counts"])
    active = [e for e in range(wl.experts) if counts[e] > 0]
    tokens = sorted(set(cover_experts(g_idx, active)) | {0, m - 1})
    _say(f"case {wl.name}: {len(active)} experts, {len(tokens)} tokens")
    rep = check_layer(wl, inp, out, idx, w, tokens=tokens, debug=dbg, lazy=True)
    _say(f"  -> {rep}")
    assert rep.ok(), rep.failures
    assert set(active) <= set(g_idx[tokens].reshape(-1).tolist())


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_mx_above_16_tokens_on_the_valu_path(fmt):
    """Above 16 tokens MX weights run on the fp32 VALU path (AUTO), which
    also serves as a cross-check of the MX decode at small sizes."""
    wl = MX_SMALL.replace(name=f"{fmt}_valu", m=40, dtype=fmt)
    run_case(wl, path="simple")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_mx_scale_bytes_at_the_format_edges(fmt):
    """E8M0 scale bytes at the ends of the format (OCP MX: byte b means
    2^(b - 127), byte 255 is NaN), on three of the experts the batch uses
    (the busiest two and the least busy): the busiest with scale bytes 0 and
    1 on every block (weights near 2^-127), the next with byte 254 (2^127) on
    blocks whose elements are all zero codes, the least busy with byte 255 on
    one gate/up block.  Tokens routed to that one must come out NaN on every
    column, as in the oracle; every other token is checked against the oracle
    as usual."""
    import oracle.layer as OL
    from tests.conftest import oracle_inputs
    wl = MX_SMALL.replace(name=f"{fmt}_edges", dtype=fmt, shared_inter=0, shared_gate=False)
    inp = synth.make_inputs(wl, device=DEV)
    spec, kw = oracle_inputs(wl, inp)
    counts = OL.forward(spec, **kw)["counts"]
    used = [e for e in np.argsort(-counts, kind="stable").tolist() if counts[e] > 0]
    e_tiny, e_big, e_nan = used[0], used[1], used[-1]
    s13, s2, w13, w2 = inp["w13_scale"], inp["w2_scale"], inp["w13"], inp["w2"]
    pk = 2 if fmt == "mxfp4" else 1
    s13[e_tiny].copy_(torch.arange(s13[e_tiny].numel(), device=DEV).reshape(s13[e_tiny].shape) % 2)
    s2[e_tiny].copy_(torch.arange(s2[e_tiny].numel(), device=DEV).reshape(s2[e_tiny].shape) % 2)
    w13[e_big, :, : 32 // pk] = 0       # first K block of every gate/up row: zero codes ...
    s13[e_big, :, 0] = 254              # ... at scale 2^127
    w2[e_big, :, : 32 // pk] = 0
    s2[e_big, :, 0] = 254
    s13[e_nan, 5, 3] = 255              # one gate/up block: NaN
    layer = make_layer(wl, inp, "small_m")
    _say(f"case {wl.name} edge scale bytes (experts {e_tiny}, {e_big}, {e_nan})")
    out, idx, w = layer(inp["x"])
    torch.cuda.synchronize()
    nan_tok = [t for t in range(wl.m) if e_nan in to_np(idx[t]).tolist()]
    fin_tok = [t for t in range(wl.m) if t not in nan_tok]
    assert nan_tok and fin_tok
    o = to_np(out.float())
    assert np.isnan(o[nan_tok]).all(), "tokens routed to the NaN-scaled expert must be NaN"
    spec, kw = oracle_inputs(wl, inp)
    ref = OL.forward(spec, **kw, tokens=np.array(nan_tok))
    assert np.isnan(ref["out64"]).all()
    rep = check_layer(wl, inp, out, idx, w, tokens=np.array(fin_tok))
    _say(f"  -> {rep}")
    assert rep.ok(), rep.failures


def test_mxfp4_k_equals_E():
    wl = synth.Workload("mx_keqE", m=9, hidden=256, experts=4, topk=4, inter=512,
                        shared_inter=0, dtype="mxfp4", gating="softmax",
                        routed_scale=1.0, seed=45, renormalize=False)
    run_case(wl, path="small_m")


# ------------------------------------------------------------ behaviour ---

def test_m_zero_is_a_noop():
    wl = RAGGED_BF16
    inp = synth.make_inputs(wl, device=DEV)
    layer = make_layer(wl, inp)
    out = torch.full((1, wl.hidden), 7.0, dtype=torch.bfloat16, device=DEV)
    _say("case m=0")
    layer.plan.forward(inp["x"], inp["router_w"], inp["w13"], inp["w2"], out,
                       torch.empty(1, wl.topk, dtype=torch.int32, device=DEV),
                       torch.empty(1, wl.topk, dtype=torch.float32, device=DEV),
                       layer.workspace, shared=layer.shared, m=0)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("wl,path,m", [(RAGGED_FP8, "grouped", None), (RAGGED_BF16, "grouped", None),
                                       (RAGGED_BF16, "small_m", 16), (RAGGED_BF16, "small_m", 5)])
def test_repeat_calls_are_bit_identical_on_a_dirty_workspace(wl, path, m):
    inp = synth.make_inputs(wl, device=DEV, m=m)
    layer = make_layer(wl, inp, path)
    _say(f"case determinism {wl.name} {path}")
    o1, i1, w1 = [t.clone() for t in layer(inp["x"])]
    layer.workspace.fill_(0xA5)
    o2, i2, w2 = layer(inp["x"])
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(w1, w2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
