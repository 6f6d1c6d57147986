#!/usr/bin/env python3
"""Benchmark of the single-GPU MoE-layer forward on MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
resident in HBM: one moe_layer call (route -> align -> expert FFN: GEMM1 +
SwiGLU, GEMM2, slot-order combine), replayed from a HIP graph captured once.
The K timed steps run back to back, bracketed by synchronisation.

Default workload: the DeepSeek-V4-Flash-shaped layer (H 4096, E 256, k 6,
F 2048, sigmoid + bias top-6, MXFP4 expert weights x e4m3 activations with
per-32 power-of-two scales) at T = 8192 tokens, the largest configuration of
the headline metric.  Printed as one JSON line on stdout; diagnostics go to
stderr.

Also reported in the same line:
  span          - cold replays of the same graph (each after a 1 GiB read
                  that evicts the L2s and the last-level cache): median,
                  p10 and p90 of the event-pair time around one replay
  roofline      - the dominant kernel (grouped GEMM1 + SwiGLU) against the
                  published peak of the matrix-core instruction it issues
                  and against HBM; its launch time from HIP events on its
                  own stream in a staged loop with a fixed warm-up
  decode        - cold moe_layer calls (eager, and replays of the captured
                  graph) at every decode size of the five configurations:
                  us/layer (median, p10, p90) and the HBM rate on the
                  weights of the experts actually touched
  prefill       - the other prefill configurations: warm back-to-back
                  replays and cold replays, MFMA and HBM fractions
  router        - moe_route alone at T = 1 for every configuration (and GLM
                  at 8 and 512 rows) next to the bare read of its gate
                  weight and an empty kernel, cold; also with the gate rows
                  in bf16 (gate_is_fp32 = 0)
  ep_share      - one GPU's share of DeepSeek-V4 expert parallelism (32
                  MXFP4 experts), cold
  cpu_baseline  - the float64 oracle timed on a token sample of the
                  headline workload, and the routing near-tie report
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # B/s, MI355X published
# Published dense matrix-core peaks (FLOP/s) by the operand types of the
# instruction each weight format issues: bf16 x bf16; e4m3 x e4m3; e4m3
# activations x e2m1 weights, which issues at the fp8 rate (measured:
# profiles/mfma_rates.txt).
MFMA_PEAK = {"bf16": 2.5e15, "fp8": 5.0e15, "mxfp4": 5.0e15}
MFMA_ISSUED = {"bf16": "bf16 x bf16 (v_mfma_f32_16x16x32_bf16)",
               "fp8": "e4m3 x e4m3 (v_mfma_f32_16x16x128_f8f6f4)",
               "mxfp4": "e4m3 x e2m1 with e8m0 scales (v_mfma_scale_f32_16x16x128_f8f6f4)"}
DTYPE = {"bf16": "bf16", "fp8": "fp8 (e4m3)", "mxfp4": "fp8 x fp4 (e4m3 x e2m1)"}
METRIC = "MoE layer µs & tokens/s; HBM TB/s % (T≤256), MFMA % (T≥4k); router µs"
GEMM1_WARMUP = 30  # staged steps before the GEMM1 events, whatever --warmup says


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_file(cfg, T):
    return os.path.join(ROOT, "profiles", f"gemm1_{cfg.name}_T{T}_traffic.txt")


# ---------------------------------------------------------------- accounting
def w13_bytes(cfg):
    """Bytes of one expert's w13 [2F, H] with its scales."""
    H, F = cfg.H, cfg.F
    if cfg.wformat == "bf16":
        return 2 * F * H * 2
    if cfg.wformat == "fp8":
        return 2 * F * H + 4 * (2 * F // 128) * (H // 128)
    return 2 * F * H // 2 + 2 * F * H // 32


def gemm1_work(cfg, T, touched):
    """Algorithmic work of one grouped GEMM1 launch: the w13 bytes of the
    experts touched (scales included) and the FLOPs 2 * T * k * 2F * H
    (padding rows not counted)."""
    return touched * w13_bytes(cfg), 2 * T * cfg.k * 2 * cfg.F * cfg.H


def layer_flops(cfg, T):
    return 6 * T * cfg.k * cfg.H * cfg.F


def touched_experts(moe, torch, cfg, W, x):
    ids, _ = moe.route(x, W["gate"], W["bias"], cfg.k, cfg.scoring, cfg.n_group, cfg.topk_group,
                       cfg.renormalize, cfg.routed_scale)
    return int(torch.unique(ids).numel())


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("ffn_gemm.hip", "common.h", "launch.h", "quant.h"):
        with open(os.path.join(ROOT, "mixture_experts_layer_04_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg, T):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 counter
    summary, or None if absent or taken on another version of the kernel."""
    path = traffic_file(cfg, T)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def pct(ts, q):
    s = sorted(ts)
    i = min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))
    return s[i]


def summary(ts):
    return {"median": round(statistics.median(ts), 2), "p10": round(pct(ts, 0.1), 2),
            "p90": round(pct(ts, 0.9), 2), "n": len(ts)}


# ---------------------------------------------------------------- GPU parts
class Flush:
    """A read of 1 GiB: evicts the L2s and the 256 MB last-level cache
    without leaving dirty lines (a write would, and their write-back would
    overlap the timed work)."""

    def __init__(self, moe, torch):
        self.moe = moe
        self.buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        self.sink = torch.empty(int(moe.lib().moe_probe_read_sink_len(1 << 30)), dtype=torch.float32,
                                device="cuda")

    def __call__(self):
        self.moe.probe_read(self.buf, self.sink)


def cold_times(torch, flush, fn, reps):
    """Event-pair time (us) around fn() on the current stream, each after a
    flush; the events also hold the launch of the first kernel and the
    completion of the last (about 2-4 us more than the kernel span)."""
    fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        flush()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e) * 1000.0)
    return out


class LayerGraph:
    """moe_layer on preallocated buffers, captured once in a HIP graph."""

    def __init__(self, moe, torch, cfg, W, x, block_m=0):
        self.moe, self.torch, self.cfg, self.W, self.x = moe, torch, cfg, W, x
        T = x.shape[0]
        self.bm = block_m or moe.layer_block_m(T, cfg.k, cfg.E, cfg.F, cfg.wformat)
        self.y = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=x.device)
        self.ws = torch.zeros(moe.layer_workspace_size(T, cfg.H, cfg.E, cfg.F, cfg.k, self.bm, cfg.wformat, 0),
                              dtype=torch.uint8, device=x.device)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.eager()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.eager()
        torch.cuda.synchronize()

    def eager(self):
        c, W = self.cfg, self.W
        self.moe.layer(self.x, W["gate"], W["bias"], W["w13"], W["w2"], c.k, c.scoring, c.n_group, c.topk_group,
                       c.renormalize, c.routed_scale, wformat=c.wformat, w13_scale=W["w13_scale"],
                       w2_scale=W["w2_scale"], block_m=self.bm, ws=self.ws, out=self.y)

    def replay(self):
        self.graph.replay()

    def warm_ms(self, warmup, steps):
        """Mean time of `steps` back-to-back replays after `warmup` more."""
        torch = self.torch
        for _ in range(warmup):
            self.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3


class Staged:
    """The hot path through moe_route, moe_align and moe_expert_ffn_stages,
    so that HIP events on the launch stream bracket GEMM1 alone."""

    def __init__(self, moe, torch, cfg, W, x, block_m):
        self.moe, self.torch, self.cfg, self.W, self.x, self.bm = moe, torch, cfg, W, x, block_m
        T = x.shape[0]
        self.y = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=x.device)
        fmt = {"bf16": 0, "fp8": 1, "mxfp4": 2}[cfg.wformat]
        need = max(moe.lib().moe_route_workspace_size(T, cfg.H, cfg.E),
                   moe.lib().moe_align_workspace_size(T, cfg.k, cfg.E),
                   moe.lib().moe_expert_ffn_workspace_size(T, cfg.H, cfg.E, cfg.F, cfg.k, block_m, fmt))
        self.ws = torch.zeros(need, dtype=torch.uint8, device=x.device)

    def __call__(self, ev=None):
        c, W, moe = self.cfg, self.W, self.moe
        ids, w = moe.route(self.x, W["gate"], W["bias"], c.k, c.scoring, c.n_group, c.topk_group, c.renormalize,
                           c.routed_scale, ws=self.ws)
        sid, bexp, npp = moe.align(ids, c.E, self.bm, ws=self.ws)
        kw = dict(wformat=c.wformat, w13_scale=W["w13_scale"], w2_scale=W["w2_scale"], ws=self.ws, out=self.y)
        args = (self.x, W["w13"], W["w2"], ids, w, sid, bexp, npp, self.bm)
        moe.expert_ffn(*args, stages=("quant",), **kw)
        if ev is not None:
            ev[0].record()
        moe.expert_ffn(*args, stages=("gemm1",), **kw)
        if ev is not None:
            ev[1].record()
        moe.expert_ffn(*args, stages=("gemm2", "combine"), **kw)

    def gemm1_us(self, steps):
        torch = self.torch
        for _ in range(GEMM1_WARMUP):
            self()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            self(evs[i])
        torch.cuda.synchronize()
        return [s.elapsed_time(e) * 1000.0 for s, e in evs]


def roofline_entry(cfg, T, touched, us, traffic=None):
    nbytes, flops = gemm1_work(cfg, T, touched)
    peak_f = MFMA_PEAK[cfg.wformat]
    t_hbm, t_mfma = nbytes / HBM_PEAK, flops / peak_f
    sec = us * 1e-6
    if t_hbm >= t_mfma:
        bound, achieved, peak, unit = "hbm", nbytes / sec / 1e9, HBM_PEAK / 1e9, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", flops / sec / 1e12, peak_f / 1e12, "TFLOP/s"
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "kernel": "grouped GEMM1 + SwiGLU", "kernel_us": round(us, 2), "mfma_issued": MFMA_ISSUED[cfg.wformat],
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "mfma_frac": round(flops / sec / peak_f, 4), "hbm_frac": round(nbytes / sec / HBM_PEAK, 4)}


def headline(moe, torch, cfg, T, args, flush):
    from synth import make_weights, make_x
    W = make_weights(cfg, "cuda")
    x = make_x(cfg, T, "cuda")
    touched = touched_experts(moe, torch, cfg, W, x)
    bm = moe.layer_block_m(T, cfg.k, cfg.E, cfg.F, cfg.wformat)

    # GEMM1's launch time: a staged loop after a fixed warm-up of its own
    st = Staged(moe, torch, cfg, W, x, bm)
    g1 = st.gemm1_us(20)
    g1_us = statistics.mean(g1)
    del st

    # the timed region: W untimed replays, then exactly K, back to back
    lg = LayerGraph(moe, torch, cfg, W, x, bm)
    ms = lg.warm_ms(args.warmup, args.steps)
    span = cold_times(torch, flush, lg.replay, args.reps)
    roof = roofline_entry(cfg, T, touched, g1_us, measured_traffic(cfg, T))
    log(f"headline {cfg.name} T={T}: {ms:.3f} ms per step (warm replays), cold median {statistics.median(span):.1f} us, "
        f"GEMM1 {g1_us:.1f} us ({roof['frac']:.3f} of {roof['bound']} peak)")
    sec = ms * 1e-3
    wbytes = touched * cfg.expert_bytes()
    res = {"ms_per_step": ms, "span": summary(span), "touched": touched, "block_m": bm, "roofline": roof,
           "gemm1_us": summary(g1),
           "layer_mfma_frac": round(layer_flops(cfg, T) / sec / MFMA_PEAK[cfg.wformat], 4),
           "layer_hbm_frac": round(wbytes / sec / HBM_PEAK, 4), "weight_bytes": wbytes}
    return res, W, x, lg


DECODE = (("toy", 16), ("qwen3", 1), ("qwen3", 64), ("glm", 1), ("glm", 8), ("dsv3", 1), ("dsv3", 256),
          ("dsv4", 512))
PREFILL = (("qwen3", 4096), ("glm", 512), ("dsv3", 2048))


def layer_sweep(moe, torch, flush, cases, reps, warm, keep=None):
    """Cold (and for prefill warm) graph replays of moe_layer per case."""
    from synth import get_config, make_weights, make_x
    out = {}
    cache = dict(keep or {})
    for name, T in cases:
        cfg = get_config(name)
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cache[name] = make_weights(cfg, "cuda")
        W = cache[name]
        x = make_x(cfg, T, "cuda")
        lg = LayerGraph(moe, torch, cfg, W, x)
        # eager moe_layer calls and replays of the captured graph (the graph
        # launch costs a few us more here)
        ts = cold_times(torch, flush, lg.eager, reps)
        tg = cold_times(torch, flush, lg.replay, reps)
        touched = touched_experts(moe, torch, cfg, W, x)
        wbytes = touched * cfg.expert_bytes()
        us = statistics.median(ts)
        r = {"us_per_layer": summary(ts), "graph_replay_us": summary(tg),
             "tokens_per_s": round(T / (us * 1e-6), 1), "block_m": lg.bm,
             "experts_touched": touched, "weight_bytes": wbytes, "weights": cfg.wformat,
             "hbm_TBps": round(wbytes / (us * 1e-6) / 1e12, 3), "hbm_frac": round(wbytes / (us * 1e-6) / HBM_PEAK, 4)}
        if warm:
            ms = lg.warm_ms(10, 20)
            r["warm_us_per_layer"] = round(ms * 1e3, 2)
            r["warm_tokens_per_s"] = round(T / (ms * 1e-3), 1)
            r["mfma_frac_warm"] = round(layer_flops(cfg, T) / (ms * 1e-3) / MFMA_PEAK[cfg.wformat], 4)
            r["hbm_frac_warm"] = round(wbytes / (ms * 1e-3) / HBM_PEAK, 4)
            r["mfma_issued"] = MFMA_ISSUED[cfg.wformat]
        key = f"{name}_T{T}"
        out[key] = r
        log(f"{key}: cold {r['us_per_layer']} us (graph replay {r['graph_replay_us']['median']}), {touched} experts, {r['hbm_TBps']} TB/s ({r['hbm_frac']:.3f} of HBM)"
            + (f"; warm {r['warm_us_per_layer']} us, MFMA {r['mfma_frac_warm']:.3f}" if warm else ""))
        del lg
    cache.clear()
    torch.cuda.empty_cache()
    return out


ROUTER = (("toy", 1), ("qwen3", 1), ("glm", 1), ("glm", 8), ("glm", 512), ("dsv3", 1), ("dsv4", 1))
# also timed with the gate rows in bf16 ([Router] §1.1: 2.4 MB for GLM's 288 x 4096)
ROUTER_BF16_GATE = (("qwen3", 1), ("glm", 1), ("glm", 8), ("glm", 512), ("dsv3", 1), ("dsv4", 1))


MFMA_KINDS = [(0, "bf16 16x16x32", 2 * 16 * 16 * 32, (8, 16)), (1, "bf16 32x32x16", 2 * 32 * 32 * 16, (4, 8)),
              (2, "e4m3 x e4m3 16x16x128", 2 * 16 * 16 * 128, (8, 16)),
              (3, "e4m3 x e2m1 16x16x128", 2 * 16 * 16 * 128, (8, 16)),
              (4, "e2m1 x e2m1 16x16x128", 2 * 16 * 16 * 128, (8, 16))]


def summarize_profile(d):
    """Per-kernel figures of a rocprofv3 output directory (csv): for each
    libmoe kernel and grid size, the number of dispatches and the median,
    mean and minimum duration in us (kernel traces), or the median of each
    counter per dispatch (counter collections)."""
    import collections
    import csv
    import glob

    def name_of(r):
        n = r["Kernel_Name"].replace("void ", "").replace("moe::(anonymous namespace)::", "")
        return n.replace("moe::", "").split("(")[0]

    def grid_of(r):
        return r.get("Grid_Size_X") or r.get("Grid_Size") or "?"

    lines = []
    dur = collections.defaultdict(list)
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if "moe::" in r["Kernel_Name"]:
                    dur[(name_of(r), grid_of(r))].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for (n, g), v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {n} | {g} | {len(v)} | {statistics.median(v):.2f} | {statistics.mean(v):.2f} | {min(v):.2f} |")
    if lines:
        lines.insert(0, "| kernel | grid | dispatches | median us | mean us | min us |\n|---|---|---|---|---|---|")
    cnt = collections.defaultdict(list)
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if "moe::" in r["Kernel_Name"]:
                    cnt[(name_of(r), grid_of(r), r["Counter_Name"])].append(float(r["Counter_Value"]))
                elif "FillFunctor" in r["Kernel_Name"]:  # torch.zeros of --copy-probe
                    cnt[("torch fill", grid_of(r), r["Counter_Name"])].append(float(r["Counter_Value"]))
    if cnt:
        lines.append("| kernel | grid | counter | dispatches | median |\n|---|---|---|---|---|")
        for (n, g, c), v in sorted(cnt.items()):
            lines.append(f"| {n} | {g} | {c} | {len(v)} | {statistics.median(v):.6g} |")
    return "\n".join(lines)


def mfma_rates(moe, torch, iters=2048, grid=2048):
    """Issue rate of each matrix-core instruction over the whole chip
    (moe_probe_mfma: 2048 workgroups of 4 waves, independent accumulator
    chains); median of 5 timed launches after one untimed."""
    out = {}
    sink = torch.empty(int(moe.lib().moe_probe_mfma_sink_len(grid)), dtype=torch.float32, device="cuda")
    for kind, name, flop, accs in MFMA_KINDS:
        for na in accs:
            moe.probe_mfma(kind, na, grid, iters, sink)
            ts = []
            for _ in range(5):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                moe.probe_mfma(kind, na, grid, iters, sink)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3)
            t = statistics.median(ts)
            out[f"{name}, {na} accumulators"] = round(grid * 4 * iters * na * flop / t / 1e12, 1)
    return out


def router_probe(moe, torch, flush, reps):
    """moe_route alone next to the bare read of its gate weight
    (moe_probe_read, the same bytes) and an empty kernel, all cold; raw
    event-pair times (each holds the same few us of event overhead)."""
    from synth import get_config, make_router_weights, make_x
    empty = cold_times(torch, flush, lambda: moe.probe_empty(), reps)
    res = {"empty_kernel_us": summary(empty)}
    for name, T in ROUTER:
        cfg = get_config(name)
        gate, bias = make_router_weights(cfg, "cuda")
        x = make_x(cfg, T, "cuda")
        ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
        ws = torch.zeros(moe.lib().moe_route_workspace_size(T, cfg.H, cfg.E), dtype=torch.uint8, device="cuda")
        sink = torch.empty(int(moe.lib().moe_probe_read_sink_len(gate.numel() * 4)), dtype=torch.float32,
                           device="cuda")
        r = cold_times(torch, flush, lambda: moe.route(x, gate, bias, cfg.k, cfg.scoring, cfg.n_group,
                                                        cfg.topk_group, cfg.renormalize, cfg.routed_scale, ws=ws),
                       reps)
        b = cold_times(torch, flush, lambda: moe.probe_read(gate, sink), reps)
        rm, bm_ = statistics.median(r), statistics.median(b)
        res[f"{name}_T{T}"] = {"route_us": summary(r), "bare_gate_read_us": summary(b), "gate_bytes": gate.numel() * 4,
                               "ratio": round(rm / bm_, 3)}
        log(f"router {name} T={T}: {rm:.2f} us vs bare read {bm_:.2f} us (x{rm / bm_:.2f})")
        if (name, T) in ROUTER_BF16_GATE:
            # the same router on the gate rows rounded to bf16 (half the
            # bytes, one MFMA per K step), against the bare read of those bytes
            g16 = gate.to(torch.bfloat16)
            r = cold_times(torch, flush, lambda: moe.route(x, g16, bias, cfg.k, cfg.scoring, cfg.n_group,
                                                            cfg.topk_group, cfg.renormalize, cfg.routed_scale,
                                                            ws=ws), reps)
            b = cold_times(torch, flush, lambda: moe.probe_read(g16, sink), reps)
            rm, bm_ = statistics.median(r), statistics.median(b)
            res[f"{name}_T{T}_bf16_gate"] = {"route_us": summary(r), "bare_gate_read_us": summary(b),
                                             "gate_bytes": g16.numel() * 2, "ratio": round(rm / bm_, 3)}
            log(f"router {name} T={T}, bf16 gate: {rm:.2f} us vs bare read {bm_:.2f} us (x{rm / bm_:.2f})")
        del ids
    return res


# One GPU's share of DeepSeek-V4 expert parallelism over 8 GPUs: 32 local
# experts at DeepSeek-V4-Flash dimensions, random routing over them ([MegaMoE]
# §3.4, where the fused kernel ran this on one B300 with every fetch local).
EP_SHARE_T = (1, 4, 16, 64, 512)
EP_SHARE_PAGE_US = {1: 40.0, 4: 68.0, 16: 95.0, 64: 99.0, 512: 112.0}  # B300, the page's figures


def ep_share_sweep(moe, torch, flush, reps, Ts=EP_SHARE_T):
    """Cold alignment + expert FFN (fp8 quantisation, both grouped GEMMs and
    the combine) for 32 MXFP4 experts, k = 6, at the page's token counts."""
    from synth import get_config, make_topk_ids, make_weights, make_x
    cfg = get_config("dsv4", E=32)
    W = make_weights(cfg, "cuda")
    out = {}
    for T in Ts:
        x = make_x(cfg, T, "cuda")
        ids = make_topk_ids(T, cfg.k, cfg.E, seed=T, kind="uniform", device="cuda")
        g = torch.Generator(device="cpu").manual_seed(T)
        w = torch.rand((T, cfg.k), generator=g)
        w = (w / w.sum(dim=1, keepdim=True)).to("cuda")
        bm = moe.layer_block_m(T, cfg.k, cfg.E, cfg.F, cfg.wformat)
        y = torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(max(moe.lib().moe_expert_ffn_workspace_size(T, cfg.H, cfg.E, cfg.F, cfg.k, bm, 2),
                             moe.lib().moe_align_workspace_size(T, cfg.k, cfg.E)), dtype=torch.uint8, device="cuda")
        holder = {}

        def both():
            holder["a"] = s_, b_, n_ = moe.align(ids, cfg.E, bm, ws=ws)
            moe.expert_ffn(x, W["w13"], W["w2"], ids, w, s_, b_, n_, bm, wformat=cfg.wformat,
                           w13_scale=W["w13_scale"], w2_scale=W["w2_scale"], ws=ws, out=y)

        ts = cold_times(torch, flush, both, reps)
        us = statistics.median(ts)
        touched = int(torch.unique(ids).numel())
        nbytes = touched * cfg.expert_bytes()
        out[f"T{T}"] = {"us_align_ffn": summary(ts), "block_m": bm, "experts_touched": touched,
                        "weight_bytes": nbytes, "hbm_TBps": round(nbytes / (us * 1e-6) / 1e12, 3),
                        "page_b300_us": EP_SHARE_PAGE_US[T]}
        log(f"EP share (32 MXFP4 experts, k=6) T={T}: {us:.1f} us, {touched} experts, "
            f"{out[f'T{T}']['hbm_TBps']} TB/s; the page's B300 figure {EP_SHARE_PAGE_US[T]:.0f} us")
    del W
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- CPU oracle
def cpu_baseline(moe, torch, cfg, W, x, n_sample):
    """The oracle as it stands on a bounded sample of the same workload:
    route + dense-equivalent layer for the first n_sample tokens, with its
    expert loop on the host's threads.  Also, on all T tokens, the routing
    near-tie report: tokens whose oracle margin at the cut (or between kept
    and dropped groups) is at most 1e-5, and how many of them the GPU routes
    to other experts."""
    import numpy as np
    from oracle import ffn as offn
    from oracle import router as orouter
    from synth import to_numpy
    threads = len(os.sched_getaffinity(0))
    workers = max(1, min(16, threads))
    xs = to_numpy(x[:n_sample])
    gate, bias = to_numpy(W["gate"]), to_numpy(W["bias"])

    class Lazy:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            return to_numpy(self.t[e])

    Wn = offn.ExpertWeights(cfg.wformat, Lazy(W["w13"]), Lazy(W["w2"]),
                            None if W["w13_scale"] is None else Lazy(W["w13_scale"]),
                            None if W["w2_scale"] is None else Lazy(W["w2_scale"]))
    t0 = time.perf_counter()
    r = orouter.route(xs, gate, bias, cfg.k, cfg.scoring, cfg.n_group, cfg.topk_group, cfg.renormalize,
                      cfg.routed_scale)
    y, _ = offn.layer(xs, r, Wn, cfg.E, workers=workers)
    dt = time.perf_counter() - t0
    assert np.all(np.isfinite(y))
    T = x.shape[0]
    base = {"value": round(n_sample / dt, 3), "unit": "tokens/s", "cores": int(workers), "kind": "oracle",
            "sample": (f"first {n_sample} of the {T} tokens" if n_sample < T else f"all {T} tokens")
            + f" (router + float64 dense-equivalent layer, expert loop on {workers} threads), {dt:.1f} s",
            "seconds": round(dt, 2)}
    # near ties on every token
    ids, _ = moe.route(x, W["gate"], W["bias"], cfg.k, cfg.scoring, cfg.n_group, cfg.topk_group, cfg.renormalize,
                       cfg.routed_scale)
    torch.cuda.synchronize()
    rf = orouter.route(to_numpy(x), gate, bias, cfg.k, cfg.scoring, cfg.n_group, cfg.topk_group, cfg.renormalize,
                       cfg.routed_scale)
    near = ~((rf["margin"] > 1e-5) & (rf["group_margin"] > 1e-5))
    gi = ids.cpu().numpy()
    differ = int(np.sum(np.any(gi[near] != rf["ids"][near], axis=1)))
    clear_differ = int(np.sum(np.any(gi[~near] != rf["ids"][~near], axis=1)))
    ties = {"tokens": T, "near_tie_tokens": int(near.sum()), "near_tie_tokens_routed_differently": differ,
            "near_tie_mismatch_rate": round(differ / max(1, int(near.sum())), 4),
            "clear_tokens_routed_differently": clear_differ, "margin": 1e-5}
    return base, ties


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=30, help="cold replays per case")
    ap.add_argument("--T", type=int, default=8192)
    ap.add_argument("--config", default="dsv4")
    ap.add_argument("--cpu-sample", type=int, default=0, help="tokens the oracle baseline runs on (0: 64; its time is mostly the dequantisation of the experts the sample touches)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the decode, prefill, router and EP-share rows")
    ap.add_argument("--only", choices=("decode", "prefill", "router", "ep", "mfma"),
                    help="diagnostic: only these rows (for kernel traces), no benchmark line")
    ap.add_argument("--cases", metavar="NAME:T,...",
                    help="with --only decode / prefill: just these cases (e.g. glm:1,dsv3:256); with --only ep: "
                         "token counts (e.g. 1,512)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="print per-kernel durations / counters of a rocprofv3 csv output directory and exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first write MIB MiB with a fill kernel and read them once with moe_probe_read "
                         "(kernels of known traffic that calibrate rocprofv3 WRITE_SIZE / FETCH_SIZE)")
    args = ap.parse_args()
    if args.summarize:
        print(summarize_profile(args.summarize))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer keeps every expert on the one GPU and has no multi-GPU path. "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import mixture_experts_layer_04_amd as moe
    from synth import get_config

    if args.copy_probe:
        buf = torch.zeros(args.copy_probe << 20, dtype=torch.uint8, device="cuda")
        moe.probe_read(buf)
        torch.cuda.synchronize()
        del buf
    flush = Flush(moe, torch)
    if args.only:
        pick = None
        if args.cases and args.only in ("decode", "prefill"):
            pick = tuple((c.split(":")[0], int(c.split(":")[1])) for c in args.cases.split(","))
        rows = {"decode": lambda: layer_sweep(moe, torch, flush, pick or DECODE, args.reps, False),
                "prefill": lambda: layer_sweep(moe, torch, flush, pick or PREFILL, args.reps, True),
                "router": lambda: router_probe(moe, torch, flush, args.reps),
                "ep": lambda: ep_share_sweep(moe, torch, flush, args.reps,
                                             tuple(int(t) for t in args.cases.split(",")) if args.cases else EP_SHARE_T),
                "mfma": lambda: mfma_rates(moe, torch)}[args.only]()
        for key, v in rows.items():
            log(f"{key}: {v}")
        return 0

    cfg = get_config(args.config)
    T = args.T
    log(f"bench: {cfg.description}, T={T}")
    h, W, x, lg = headline(moe, torch, cfg, T, args, flush)
    ms = h["ms_per_step"]
    result = {
        "metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE[cfg.wformat], "data": "synthetic",
        "config": {"workload": f"{cfg.description}, T={T}", "T": T, "H": cfg.H, "E": cfg.E, "k": cfg.k,
                   "F": cfg.F, "block_m": h["block_m"], "weights": cfg.wformat, "experts_touched": h["touched"],
                   "step": "one HIP-graph replay of moe_layer (router, alignment, GEMM1 + SwiGLU, GEMM2, combine)"},
        "us_per_layer": round(ms * 1e3, 2),
        "span_cold_us": h["span"],
        "layer_mfma_frac": h["layer_mfma_frac"], "layer_hbm_frac": h["layer_hbm_frac"],
        "mfma_issued": MFMA_ISSUED[cfg.wformat],
        "roofline": h["roofline"],
        "gemm1_event_us": h["gemm1_us"],
    }
    if not args.no_cpu:
        n = args.cpu_sample if args.cpu_sample > 0 else min(T, 64)
        base, ties = cpu_baseline(moe, torch, cfg, W, x, n)
        result["cpu_baseline"] = base
        result["routing_near_ties"] = ties
        log(f"cpu oracle: {base['value']} tokens/s on {base['cores']} threads; near ties {ties}")
    del lg, W, x
    torch.cuda.empty_cache()
    if not args.no_extras:
        result["decode"] = layer_sweep(moe, torch, flush, DECODE, args.reps, False)
        result["prefill"] = layer_sweep(moe, torch, flush, PREFILL, max(10, args.reps // 3), True)
        result["router"] = router_probe(moe, torch, flush, args.reps)
        result["ep_share_dsv4_32_experts"] = ep_share_sweep(moe, torch, flush, args.reps)
        result["cold_timing"] = ("each call (eager moe_layer, or a replay of its captured graph) after a 1 GiB read; "
                                 "raw event-pair time around it (median, p10, p90), which includes the first "
                                 "kernel's launch and the last one's completion")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
