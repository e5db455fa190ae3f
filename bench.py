#!/usr/bin/env python3
"""Benchmark of one MoE FFN layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--m M] [--launch eager|graph]

A step is one full layer forward (router, gating + top-k, sort by expert,
[fp8 activation quantisation,] gate/up + SwiGLU, down, combine) over one batch
of seeded synthetic tokens whose inputs are already resident in HBM.  The
expert weights are held in several identical copies that the steps rotate
through, so every step streams its weights from HBM rather than from the
256 MB last-level cache.

Prints one JSON line: layer tokens/s (``value``), the layer's GB/s and
TFLOP/s against the HBM and MFMA peaks, a ``roofline`` entry for the
dominant kernel (its duration measured with HIP events recorded around it on
the launch stream inside the timed steps; its HBM traffic from the rocprofv3
byte counters recorded in profiles/hbm_traffic.json, null once the kernel's
sources differ from the ones counted), and ``cpu_baseline``: the fp64 CPU
oracle timed on the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# MXFP4 / MXFP8 weights and the fp8 layer's e4m3 codes are converted to their
# exact bf16 values in registers and multiplied on the bf16 MFMA (the fp8 MFMA
# does not accumulate in full fp32), so their products take the bf16 peak
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 2500.0, "f32": 157.3, "mxfp4": 2500.0, "mxfp8": 2500.0}
COMPUTE_DTYPE = {"mxfp4": "bf16", "mxfp8": "bf16", "fp8": "bf16"}
METRIC = "MoE layer tokens/s; prefill TFLOP/s vs MFMA peak; decode GB/s vs HBM peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_fp8",
                    help="the headline workload (default: the largest configuration, 4096 tokens "
                         "of the fp8 layer)")
    ap.add_argument("--configs", choices=("all", "none"), default="all",
                    help="all: also measure the decode (1, 4, 16 tokens), prefill and skewed "
                         "layers into the line's configs array")
    ap.add_argument("--m", type=int, default=None, help="tokens (default: the workload's)")
    ap.add_argument("--path", default="auto")
    ap.add_argument("--copies", type=int, default=None,
                    help="weight copies rotated across steps (default: >= 2 GB in total)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens in the CPU-oracle sample")
    ap.add_argument("--kernel-events", choices=("timed", "off"), default="timed",
                    help="timed: record HIP events around the dominant kernel inside the timed "
                         "steps (its duration for the roofline); off: time it in a separate loop")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="graph: each weight copy's layer forward (with its timing events) is "
                         "captured once in a HIP graph and the timed steps replay the graphs")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="before the timed region, run one plain device copy of this many MiB "
                         "(a known-size reference for HBM byte counters)")
    return ap.parse_args()


def esz(dtype):
    return {"f32": 4, "bf16": 2, "fp8": 1, "mxfp4": 0.5, "mxfp8": 1}[dtype]


# Source files of the dominant (gate/up) kernel of each expert path: HBM byte
# counters recorded in profiles/hbm_traffic.json stand only while these files
# are unchanged.
KERNEL_SOURCES = {"small_m": ("small_m.hip", "lds.h", "common.h", "kernels.h"),
                  "grouped": ("gateup.hip", "lds.h", "common.h", "kernels.h")}


def recorded_traffic(workload, m, stage, path):
    """HBM bytes per launch (read + write) of a kernel, from the rocprofv3
    FETCH_SIZE / WRITE_SIZE runs summarised in profiles/, or None when there is
    no record for it or its sources changed since the counters were taken."""
    import hashlib
    files = KERNEL_SOURCES.get(path)
    rec_path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not files or not os.path.exists(rec_path):
        return None
    rec = json.load(open(rec_path)).get(f"{workload}|m={m}|{stage}")
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mixture_experts_ffn_06_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec["read_bytes"] + rec["write_bytes"]


def layer_counts(wl, m, D):
    """Algorithmic flops and bytes of the layer and of each expert kernel.

    D: number of distinct routed experts that received >= 1 token.
    Weights of every active expert are read once (codes + fp32 block scales
    for fp8); x is read once, out written once; the sorted intermediates
    (h, fp32 y) count as the producing and consuming kernels' traffic.
    """
    H, E, I, Is, k = wl.hidden, wl.experts, wl.inter, wl.shared_inter, wl.topk
    te = m * k
    we = esz(wl.dtype)
    ae = 4 if wl.dtype == "f32" else 2              # x / out element bytes
    if wl.dtype == "fp8":
        sc = lambda r, c: (r // 128) * (c // 128) * 4     # fp32 per 128x128 block
    elif wl.dtype in ("mxfp4", "mxfp8"):
        sc = lambda r, c: r * (c // 32)                    # E8M0 byte per 32 along K
    else:
        sc = lambda r, c: 0
    w13 = D * (2 * I * H * we + sc(2 * I, H)) + (2 * Is * H * we + sc(2 * Is, H) if Is else 0)
    w2 = D * (H * I * we + sc(H, I)) + (H * Is * we + sc(H, Is) if Is else 0)
    hb = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp4": 2, "mxfp8": 2}[wl.dtype]   # h element bytes
    h_bytes = (te * I + m * Is) * hb + ((te * I + m * Is) // 128 * 4 if wl.dtype == "fp8" else 0)
    x_in = m * H * (1 + 4 / 128 if wl.dtype == "fp8" else ae)
    y_bytes = (te + (m if Is else 0)) * H * 4       # fp32 down outputs
    flops_gateup = 2 * te * 2 * I * H + 2 * m * 2 * Is * H
    flops_down = 2 * te * H * I + 2 * m * H * Is
    flops = 2 * m * E * H + flops_gateup + flops_down
    bytes_layer = w13 + w2 + E * H * ae + m * H * ae * 2
    return {
        "flops": flops, "bytes": bytes_layer,
        "gateup": {"bytes": w13 + x_in + h_bytes, "flops": flops_gateup},
        "down": {"bytes": w2 + h_bytes + y_bytes, "flops": flops_down},
    }


def host_info():
    """CPU model, cores available to this process and the BLAS numpy uses."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    import numpy  # noqa: F401  (loads the BLAS that threadpool_info reports)
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    vendor = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in blas})) or "unknown"
    threads = max([p.get("num_threads", 1) for p in blas] + [1])
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0)),
            "blas": vendor, "blas_threads": threads}


def cpu_baseline(wl, inp, m, sample, repeats):
    """Time the fp64 oracle (as it stands) on the host for ``sample`` tokens."""
    import numpy as np
    import torch
    import oracle.layer as OL

    def np_of(t):
        if t is None:
            return None
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    spec = OL.LayerSpec(hidden=wl.hidden, experts=wl.experts, topk=wl.topk,
                        inter=wl.inter, shared_inter=wl.shared_inter, dtype=wl.dtype,
                        gating=wl.gating, routed_scale=wl.routed_scale, block=wl.block)

    class PerExpert:
        """One expert at a time to the host (the large layers' weights do not
        need a full host copy)."""
        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            return np_of(self.t[e])

    lazy = lambda t: None if t is None else PerExpert(t)
    args = dict(x=np_of(inp["x"]), router_w=np_of(inp["router_w"]),
                w13=lazy(inp["w13"]), w2=lazy(inp["w2"]),
                w13_scale=lazy(inp["w13_scale"]), w2_scale=lazy(inp["w2_scale"]),
                bias=np_of(inp["bias"]))
    if wl.shared_inter:
        args["shared"] = {k: np_of(inp["shared_" + k]) for k in
                          ("w13", "w2", "w13_scale", "w2_scale")}
    tokens = None if sample >= m else list(range(0, m, max(1, m // sample)))[:sample]
    times, res = [], None
    for _ in range(repeats):
        t0 = time.perf_counter()
        res = OL.forward(spec, **args, tokens=tokens)
        times.append(time.perf_counter() - t0)
    n = len(res["tokens"])
    med = statistics.median(times)
    hi = host_info()
    return {"value": n / med, "unit": "tokens/s", "cores": hi["blas_threads"],
            "kind": "oracle",
            "sample": (f"{n} of {m} tokens ({'all' if tokens is None else 'strided'}); "
                       "gating and permutation for all tokens, experts and combine for "
                       f"the sample; fp64 numpy; {repeats} run(s)"),
            "seconds": {"median": med, "p10": float(np.percentile(times, 10)),
                        "p90": float(np.percentile(times, 90))},
            "host": hi}, res


# Entries of the configuration sub-array of the default run: the decode
# layer at 1, 4 and 16 tokens (graph replay where a step is bound by the
# host's launches), the prefill layer and the skewed-routing fp8 layer.
CONFIG_RUNS = (("decode_bf16", 1, "graph"), ("decode_bf16", 4, "graph"),
               ("decode_bf16", 16, "eager"), ("prefill_bf16", 1024, "eager"),
               ("skew_fp8", 2048, "eager"))
# CPU-oracle sample (tokens) and repeats per workload: about 10-30 s of host work
CPU_SAMPLE = {"decode_bf16": (16, 3), "decode_mxfp4": (16, 3), "decode_mxfp8": (16, 3),
              "prefill_bf16": (32, 3), "large_fp8": (4, 1), "skew_fp8": (4, 1), "skew_head_fp8": (4, 1),
              "dense_bf16": (8, 1), "dense_fp8": (2, 1), "tiny_f32": (4, 3)}


def measure(wl, m, args, launch, cpu, min_warm_s=0.0):
    """One workload: K timed layer forwards (inputs resident in HBM), the
    dominant kernel against its roofline and, if ``cpu``, the CPU oracle.
    ``min_warm_s``: after the W warm-up steps, more untimed steps until that
    much time has passed (entries that follow another entry's host-only CPU
    leg, when the GPU sat idle, and whose timed region is a few ms)."""
    import numpy as np
    import torch
    import synth
    from mixture_experts_ffn_06_amd import MoeLayer

    if m > wl.m:   # a larger batch: the same recipe with more tokens drawn
        wl = wl.replace(m=m)
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(wl, device=dev, m=m)
    wbytes = sum(v.numel() * v.element_size() for k, v in inp.items()
                 if v is not None and k.startswith(("w", "shared")))
    copies = args.copies or max(1, int(np.ceil(2e9 / wbytes)))
    names = [k for k in inp if k != "x" and inp[k] is not None]
    layers = []
    for c in range(copies):
        w = {k: (inp[k] if c == 0 else inp[k].clone()) for k in names}
        layers.append(MoeLayer(w, hidden=wl.hidden, num_experts=wl.experts,
                               inter=wl.inter, topk=wl.topk, max_tokens=m,
                               shared_inter=wl.shared_inter, gating=wl.gating,
                               routed_scale=wl.routed_scale, weight_dtype=wl.dtype,
                               path=args.path))
    x = inp["x"]
    act = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    out = torch.empty((m, wl.hidden), dtype=act, device=dev)
    idx = torch.empty((m, wl.topk), dtype=torch.int32, device=dev)
    tw = torch.empty((m, wl.topk), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, debug=None):
        layers[i % copies](x, out=out, topk_idx=idx, topk_w=tw, stream=stream, debug=debug)

    if args.copy_mb:
        src = torch.ones(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    from mixture_experts_ffn_06_amd._lib import NUM_STAGES, STAGES, _event_handle
    dom = "gateup"
    di = STAGES.index(dom)

    def dom_events():
        """Events recorded by the library on the launch stream just before the
        dominant kernel and just before the next stage."""
        evs = [None] * (NUM_STAGES + 1)
        evs[di] = torch.cuda.Event(enable_timing=True)
        evs[di + 1] = torch.cuda.Event(enable_timing=True)
        for ev in (evs[di], evs[di + 1]):
            _event_handle(ev)          # create the HIP events outside the timed region
        return evs

    for i in range(args.warmup):
        step(i)
    graphs = None
    if launch == "graph":
        # one graph per weight copy; the library's one-time set-up ran eagerly
        # in the warm-up steps.  Event nodes inside a replayed graph do not
        # bracket the kernels on this stack (an 84 us kernel read 4.5 us), so
        # the graphs carry no events and the dominant kernel is timed by the
        # stage-event loop below
        kev = None
        torch.cuda.synchronize()
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layers[c](x, out=out, topk_idx=idx, topk_w=tw)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % copies].replay()
    else:
        kev = [dom_events() for _ in range(args.steps)] if args.kernel_events == "timed" else None
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < min_warm_s:
        for i in range(8):
            if graphs is not None:
                graphs[i % copies].replay()
            else:
                step(i)
        torch.cuda.synchronize()
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for ev in bounds:
        _event_handle(ev)
    torch.cuda.synchronize()
    # ---- timed region: exactly K steps ----
    t0 = time.perf_counter()
    bounds[0].record(stream)
    for i in range(args.steps):
        if graphs is not None:
            graphs[i % copies].replay()
        else:
            step(i, debug=None if kev is None else {"events": kev[i]})
        bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = np.array([bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)])
    gpu_ms = bounds[0].elapsed_time(bounds[-1]) / args.steps
    ms_per_step = max(wall * 1e3 / args.steps, gpu_ms)
    dom_timed_ms = (float(np.mean([e[di].elapsed_time(e[di + 1]) for e in kev]))
                    if kev is not None else None)

    # ---- per-stage durations: the same steps with HIP events between stages ----
    stage_ms = np.zeros(NUM_STAGES)
    for i in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(NUM_STAGES + 1)]
        step(i, debug={"events": evs})
        torch.cuda.synchronize()
        stage_ms += np.array([evs[j].elapsed_time(evs[j + 1]) for j in range(NUM_STAGES)])
    stage_ms /= args.steps

    D = int(torch.unique(idx).numel())
    per_expert = torch.bincount(idx.flatten().long(), minlength=wl.experts)
    routing = {"active_experts": D,
               "empty_experts": int((per_expert == 0).sum()),
               "max_expert_share": float(per_expert.max()) / float(idx.numel()),
               "max_expert_rows": int(per_expert.max())}
    cnt = layer_counts(wl, m, D)
    gb = cnt["bytes"] / (ms_per_step * 1e-3) / 1e9
    tf = cnt["flops"] / (ms_per_step * 1e-3) / 1e12
    dom_ms = dom_timed_ms if dom_timed_ms is not None else float(stage_ms[di])
    dom_gbps = cnt[dom]["bytes"] / (dom_ms * 1e-3) / 1e9
    dom_tflops = cnt[dom]["flops"] / (dom_ms * 1e-3) / 1e12
    # the kernel's bound: whichever of its bytes and flops takes longer at peak
    mfma_peak = MFMA_PEAK_TFLOPS[wl.dtype]
    mfma_bound = cnt[dom]["flops"] / (mfma_peak * 1e12) > cnt[dom]["bytes"] / (HBM_PEAK_GBPS * 1e9)
    floor_s = max(cnt["flops"] / (mfma_peak * 1e12), cnt["bytes"] / (HBM_PEAK_GBPS * 1e9))
    kernel_names = {"small_m": ("sm_mx_kernel<gateup, MXFP4>" if wl.dtype == "mxfp4" else
                                "sm_mx_kernel<gateup, MXFP8>" if wl.dtype == "mxfp8" else
                                "sm_kernel<gateup>"),
                    "grouped": "gu_kernel<gateup>", "simple": "simple_gateup_kernel"}
    path = layers[0].plan.path_for(m)
    res = {
        "value": m / (ms_per_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_per_step,
        "step_ms": {"median": float(np.median(per_step)), "p10": float(np.percentile(per_step, 10)),
                    "p90": float(np.percentile(per_step, 90))},
        "dtype": COMPUTE_DTYPE.get(wl.dtype, wl.dtype),
        "config": {"workload": f"{wl.name}: m={m} H={wl.hidden} E={wl.experts} "
                               f"k={wl.topk} I={wl.inter} I_s={wl.shared_inter} "
                               f"{wl.dtype} {wl.gating}",
                   "path": path, "active_experts": D, "routing": routing, "weight_copies": copies,
                   "launch": launch},
        "layer": {"gbps": gb, "hbm_frac": gb / HBM_PEAK_GBPS, "tflops": tf,
                  "mfma_frac": tf / mfma_peak, "attainable_frac": floor_s / (ms_per_step * 1e-3),
                  "algorithmic_bytes": cnt["bytes"], "algorithmic_flops": cnt["flops"],
                  "gpu_ms_per_step": gpu_ms},
        "stages_us": {s: float(stage_ms[j] * 1e3) for j, s in enumerate(STAGES)},
        "roofline": {"kernel": kernel_names.get(path, path),
                     "bound": "mfma" if mfma_bound else "hbm",
                     "achieved": dom_tflops if mfma_bound else dom_gbps,
                     "peak": mfma_peak if mfma_bound else HBM_PEAK_GBPS,
                     "unit": "TFLOP/s" if mfma_bound else "GB/s",
                     "frac": dom_tflops / mfma_peak if mfma_bound else dom_gbps / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic(wl.name, m, dom, path),
                     "traffic_unit": "HBM bytes per launch, read + written (rocprofv3 counters)",
                     "bytes_per_launch": cnt[dom]["bytes"], "flops_per_launch": cnt[dom]["flops"],
                     "us_per_launch": dom_ms * 1e3,
                     "timing": ("HIP events around the kernel inside the timed steps"
                                if dom_timed_ms is not None else
                                "HIP events around the kernel in a separate eager loop")},
    }
    if cpu:
        sample, repeats = CPU_SAMPLE.get(wl.name, (min(m, 16), 1))
        if args.cpu_sample:
            sample = args.cpu_sample
        cb, ref = cpu_baseline(wl, inp, m, min(sample, m), repeats)
        res["cpu_baseline"] = cb
        o = out.float().cpu().numpy().astype(np.float64)[ref["tokens"]]
        r = ref["out64"]
        res["parity"] = {"tokens": len(ref["tokens"]),
                         "rel_l2": float(np.linalg.norm(o - r) / np.linalg.norm(r)),
                         "topk_idx_equal": float(np.mean(idx.cpu().numpy() == ref["idx"]))}
    del layers, inp, out, idx, tw, graphs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): "
              "multi-GPU expert parallelism is not part of this build.", file=sys.stderr)
        sys.exit(2)
    import synth

    wl = synth.WORKLOADS[args.workload]
    m = args.m or wl.m
    print(f"bench: {wl.name} m={m}", file=sys.stderr, flush=True)
    head = measure(wl, m, args, args.launch, not args.no_cpu_baseline)
    result = {"metric": METRIC, "value": head.pop("value"), "unit": head.pop("unit"),
              "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": head.pop("ms_per_step"), "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": head.pop("dtype"),
              "data": "synthetic (seeded draws; no trained weights)"}
    result.update(head)
    if args.configs == "all":
        entries = []
        for name, mm, launch in CONFIG_RUNS:
            if name == wl.name and mm == m:
                continue
            print(f"bench: {name} m={mm} ({launch})", file=sys.stderr, flush=True)
            entries.append(measure(synth.WORKLOADS[name], mm, args, launch,
                                   not args.no_cpu_baseline, min_warm_s=0.2))
        result["configs"] = entries
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
