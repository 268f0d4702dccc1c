#!/usr/bin/env python3
"""Split-KV decode attention on one MI355X: one JSON line on stdout.

Headline step: one decode_attn call (partial-tile kernel + log-sum-exp merge)
on the Llama-3-8B-shaped batched decode (B=8, Hq=32, Hkv=8, D=128,
S_max=32768, ragged seq_lens ~ U[1, 32768] from a fixed seed), inputs resident
in HBM. Two copies of the cache alternate between steps so that no step finds
its data in the 256 MB Infinity Cache left there by the step before.

Every timed call runs inside a captured graph (the form a decode loop runs
in, all of a step's layer calls in one graph). value = algorithmic KV bytes
per call / µs per call, from one graph of the K timed calls on the two cache
copies in turn, timed with HIP events on the replay stream (a long read keeps
the GPU busy while the host launches it), median of 9 rounds (p10 and p90
reported beside it); each call's K/V was last read two calls earlier, with
487 MB of other K/V read since (more than the 256 MB Infinity Cache holds).
"launch_floor_us" replays the same launches with every length 0;
"one_tile_ablation" the same call with one tile per row (chunk = S_max), the
pages' baseline for split-KV. "one_call_per_graph" reports a graph of a
single call, warm and after a 1 GiB read that evicts the Infinity Cache, with
its own floor (each graph launch costs several µs on its own). The partial
kernel alone is replayed the same way for the roofline entry. The other four
workloads are timed per graph replay (median, p10, p90 of at least 50) and
reported under "workloads"; the steps around attention (rope_kv_write,
prefill_attn, the GEMV weight products, the speculative accept/reject step
spec_accept) under their own keys.

The fp64 CPU oracle runs first, before the GPU is touched, on every workload
(whole calls, or whole steps of layer calls): one BLAS thread in one process,
then the same independent slices over a pool of worker processes. The
headline's figure is "cpu_baseline"; the others sit in each workload's
"cpu_oracle".

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--headline-only]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/call + effective KV read GB/s (% of HBM peak) at 4k–32k ctx"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "partial_traffic.json")
KERNEL_SOURCES = ["partial_kernel.hpp", "device_common.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "stream_decode_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, chunk: int):
    """HBM bytes per launch of the partial kernel from committed counter runs, or
    None when they were taken on different kernel sources or launch shapes."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha() or t.get("workload") != workload \
            or t.get("chunk") != chunk:
        return None
    return t.get("fetch_bytes_per_launch", 0) + t.get("write_bytes_per_launch", 0)


def graph_of(torch, stream, fns):
    """One CUDA/HIP graph holding the work each fn enqueues on ``stream``."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for fn in fns:
            fn()
    return g


def back_to_back_us(torch, stream, graphs, steps, warmup, busy=None):
    """µs per replay of graphs[i % len] replayed back to back, timed with events on
    the replay stream. ``busy`` (a long read) is enqueued before the first event
    so that the GPU is not idle waiting for the host to launch the first graph."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
        stream.synchronize()
        if busy is not None:
            busy()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        e1.record(stream)
        e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def replay_dist_us(torch, stream, graphs, steps, warmup, busy=None):
    """µs of each of ``steps`` back-to-back replays of graphs[i % len], from an
    event recorded after every replay on the replay stream (``busy`` as in
    back_to_back_us). Returns the list of per-replay times."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
        stream.synchronize()
        if busy is not None:
            busy()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            graphs[i % len(graphs)].replay()
            ev[i + 1].record(stream)
        ev[-1].synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)]


def dist(xs, scale=1.0, nd=2):
    """median / p10 / p90 of xs (times scale), rounded."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64) * scale
    return {"median": round(float(np.median(a)), nd), "p10": round(float(np.percentile(a, 10)), nd),
            "p90": round(float(np.percentile(a, 90)), nd)}


def cold_us(torch, stream, graphs, n, flush):
    """Median µs of single replays, each preceded by ``flush`` (a 1 GiB read that
    evicts the 256 MB Infinity Cache and keeps the GPU busy while the host
    enqueues the replay, so the event pair brackets GPU time only)."""
    import numpy as np
    ts = []
    with torch.cuda.stream(stream):
        for i in range(n):
            flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graphs[i % len(graphs)].replay()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--chunk", type=int, default=0,
                    help="override the library's default tile size (workloads 2-5)")
    ap.add_argument("--only", type=str, default="", choices=["", "1", "2", "3", "5", "gemv", "prefill", "spec"],
                    help="profiling: run only this workload's (or step's) timing (no headline line)")
    ap.add_argument("--lengths", type=str, default="",
                    help="profiling: comma-separated lengths for workloads 2 and 3 instead of the listed ones")
    ap.add_argument("--no-floor", action="store_true",
                    help="profiling: skip the every-length-0 graphs, so every launch has the chosen lengths")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode-attention kernels run on a single device and "
              "this build has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import stream_decode_attention_amd as sda
    import workloads
    from stream_decode_attention_amd import roofline as rf

    # ---------------------------------------------- inputs, then the CPU oracle
    # (before anything touches the GPU: the oracle's worker processes fork)
    t = time.time()
    wl = int(args.only) if args.only.isdigit() else 0
    cfgs = (wl,) if wl else () if args.only else (4,) if args.headline_only else (1, 2, 3, 4, 5)
    inputs = {cfg: [workloads.make_config(cfg, layer=l) for l in range(workloads.CONFIGS[cfg].layers)]
              for cfg in cfgs}
    log(f"inputs generated in {time.time() - t:.1f}s")
    cpu = None if args.no_cpu_baseline else cpu_oracle_runs(inputs, rf)

    sda.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    # ------------------------------------------------------------ probe
    probe_buf = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    probe_buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(3):
        sda.probe_read(probe_buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        sda.probe_read(probe_buf, sink)
    e1.record()
    torch.cuda.synchronize()
    probe_gbps = 10 * probe_buf.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    log(f"probe: streaming read {probe_gbps:.0f} GB/s")

    # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter readings
    # calibrate the byte counters taken on the attention kernels
    calib = probe_buf[: 1 << 28]
    calib_dst = torch.empty_like(calib)
    sda.probe_copy(calib_dst, calib)
    torch.cuda.synchronize()
    del calib_dst

    flush_buf = probe_buf[: 1 << 30]

    def flush():
        sda.probe_read(flush_buf, sink, stream=stream)

    if args.only:
        # profiling run: one workload's (or step's) graphs, printed as JSON
        if wl:
            res = other_workloads(args, dev, up, sda, workloads, rf, np, torch, stream, flush, inputs)
        elif args.only == "gemv":
            res = gemv_runs(sda, np, torch, stream, flush)
        elif args.only == "prefill":
            res = prefill_runs(up, sda, workloads, np, torch, stream, flush)
        else:
            res = spec_runs(sda, workloads, np, torch, stream, flush)
        print(json.dumps(res), flush=True)
        return

    # ------------------------------------------------------ headline: workload 4
    c4 = inputs[4][0]
    w4 = c4["workload"]
    log(f"workload 4 lens {c4['lens'].tolist()}")
    q = up(c4["q"])
    ks = [up(c4["k"])]
    vs = [up(c4["v"])]
    ks.append(ks[0].clone())
    vs.append(vs[0].clone())
    lens = torch.from_numpy(c4["lens"]).to(dev)
    zero_lens = torch.zeros_like(lens)
    chunk = args.chunk or sda.default_chunk(w4.B, 1, w4.Hq, w4.Hkv, w4.D, w4.S_max)
    ws = torch.empty(sda.workspace_bytes(w4.B, 1, w4.Hq, w4.Hkv, w4.D, w4.S_max, chunk),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((w4.B, w4.Hq, w4.D), dtype=torch.bfloat16, device=dev)
    kv_bytes = rf.kv_bytes_decode(c4["lens"], w4.Hkv, w4.D, w4.S_max)

    def call(i, ln=lens):
        return lambda: sda.decode_attn(q, ks[i], vs[i], ln, c4["scale"], out, ws, chunk, stream=stream)

    def partial(i):
        return lambda: sda.attn_partial(q, ks[i], vs[i], lens, c4["scale"], ws, chunk=chunk, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(4):
            call(i % 2)()
        stream.synchronize()
    # A decode step's graph holds all its layer calls back to back, so the K timed
    # calls are one graph (W warm-up calls another), on the two cache copies in
    # turn: each call's K/V was last read two calls earlier, with 487 MB of other
    # K/V read since, more than the 256 MB Infinity Cache holds.
    K, W = args.steps, max(1, args.warmup)
    ROUNDS = 9

    def graphs_for(make):
        return (graph_of(torch, stream, [make(i % 2) for i in range(W)]),
                graph_of(torch, stream, [make(i % 2) for i in range(K)]))

    kinds = {"call": graphs_for(call),
             # the partial kernel alone, for its average launch duration
             "partial": graphs_for(partial),
             # the same launches with every length 0: every tile exits at once
             "floor": graphs_for(lambda i: call(i, zero_lens))}
    # rounds interleave the three so that clock and power state weigh on each alike;
    # each round replays W warm-up calls, then times K calls in one graph
    per_round = {name: [] for name in kinds}
    for _ in range(ROUNDS):
        for name, (warm, timed) in kinds.items():
            with torch.cuda.stream(stream):
                warm.replay()
            per_round[name].append(back_to_back_us(torch, stream, [timed], 1, 0, busy=flush) / K)
    us_call, us_part, us_floor = (float(np.median(per_round[n])) for n in ("call", "partial", "floor"))
    del kinds
    # the pages' baseline for split-KV: one tile per row (llm-decode-cuda's one
    # block per head), the same call with chunk = S_max
    ws_one = torch.empty(sda.workspace_bytes(w4.B, 1, w4.Hq, w4.Hkv, w4.D, w4.S_max, w4.S_max),
                         dtype=torch.uint8, device=dev)
    g_one_tile = graphs_for(lambda i: (lambda: sda.decode_attn(q, ks[i], vs[i], lens, c4["scale"], out, ws_one,
                                                               w4.S_max, stream=stream)))
    one_tile_rounds = []
    for _ in range(3):
        with torch.cuda.stream(stream):
            g_one_tile[0].replay()
        one_tile_rounds.append(back_to_back_us(torch, stream, [g_one_tile[1]], 1, 0, busy=flush) / K)
    us_one_tile = float(np.median(one_tile_rounds))
    del g_one_tile
    # one call per graph: what a lone replay costs, warm and after an Infinity Cache flush
    g_one = [graph_of(torch, stream, [call(i)]) for i in range(2)]
    g_one_floor = [graph_of(torch, stream, [call(i, zero_lens)]) for i in range(2)]
    us_one = back_to_back_us(torch, stream, g_one, K, W, busy=flush)
    us_one_floor = back_to_back_us(torch, stream, g_one_floor, K, W, busy=flush)
    cold_med, cold_p10, cold_p90 = cold_us(torch, stream, g_one, max(20, args.steps // 2), flush)

    # one call launched eagerly (two kernel launches on the stream, no graph):
    # the same lone call without a graph launch's own cost
    class Eager:
        def __init__(self, fn):
            self.replay = fn
    e_one = [Eager(call(i)) for i in range(2)]
    us_eager = back_to_back_us(torch, stream, e_one, K, W, busy=flush)
    us_eager_floor = back_to_back_us(torch, stream, [Eager(call(i, zero_lens)) for i in range(2)], K, W,
                                     busy=flush)
    eager_med, eager_p10, eager_p90 = cold_us(torch, stream, e_one, max(20, args.steps // 2), flush)
    # cold inside a step's graph: each call follows a 512 MiB read (twice the
    # Infinity Cache), as a layer's attention call follows other reads in a
    # decode step; per call = graph(flush, call, flush, call, ...) minus
    # graph(flush, flush, ...), both replayed on a busy GPU, median of rounds
    cold_buf = probe_buf[: 1 << 29]

    def flush_small():
        sda.probe_read(cold_buf, sink, stream=stream)

    KC = 20
    g_fc = graph_of(torch, stream, [f for i in range(KC) for f in (flush_small, call(i % 2))])
    g_f = graph_of(torch, stream, [flush_small] * KC)
    cold_rounds = []
    for _ in range(ROUNDS):
        a = back_to_back_us(torch, stream, [g_fc], 1, 1, busy=flush)
        b = back_to_back_us(torch, stream, [g_f], 1, 1, busy=flush)
        cold_rounds.append((a - b) / KC)
    cold_graph = float(np.median(cold_rounds))
    del g_fc, g_f
    ms_per_step = us_call / 1e3
    value = kv_bytes / (us_call / 1e6) / 1e9
    achieved = kv_bytes / (us_part / 1e6) / 1e9
    log(f"workload 4: {us_call:.1f} us/call ({value:.0f} GB/s), {K} calls in one graph; partial kernel "
        f"{us_part:.1f} us = {achieved:.0f} GB/s; launch floor {us_floor:.1f} us/call; one call per "
        f"graph {us_one:.1f} us (floor {us_one_floor:.1f}), cold {cold_med:.1f} us; eager {us_eager:.1f} us "
        f"(floor {us_eager_floor:.1f}), cold {eager_med:.1f} us; cold inside a graph "
        f"{cold_graph:.1f} us ({kv_bytes / cold_graph / 1e3:.0f} GB/s)")

    traffic = load_traffic(w4.name, chunk)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accum_dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w4.name, "B": w4.B, "Hq": w4.Hq, "Hkv": w4.Hkv, "D": w4.D, "S_max": w4.S_max,
            "seq_lens": c4["lens"].tolist(), "chunk": chunk, "kv_dtype": "bf16", "out_dtype": "bf16",
            "kv_bytes_per_call": kv_bytes,
        },
        "us_per_call": round(us_call, 2),
        "calls_per_graph": K,
        "rounds": ROUNDS,
        "us_per_call_rounds": [round(x, 2) for x in per_round["call"]],
        "us_per_call_dist": dist(per_round["call"]),
        "partial_us_dist": dist(per_round["partial"]),
        "launch_floor_us_dist": dist(per_round["floor"]),
        "one_tile_ablation": {
            "what": "the same call with chunk = S_max: one tile (one workgroup) per (sequence, kv head), the "
                    "pages' one-block-per-head baseline for split-KV",
            "chunk": w4.S_max, "us_per_call": round(us_one_tile, 2),
            "us_per_call_rounds": [round(x, 2) for x in one_tile_rounds],
            "GBps": round(kv_bytes / (us_one_tile / 1e6) / 1e9, 1),
            "split_kv_speedup": round(us_one_tile / us_call, 2)},
        "frac_of_hbm_peak": round(value / rf.HBM_PEAK_GBPS, 4),
        "launch_floor_us": round(us_floor, 2),
        "one_call_per_graph": {
            "us_per_call": round(us_one, 2), "launch_floor_us": round(us_one_floor, 2),
            "cold_us": {"median": round(cold_med, 2), "p10": round(cold_p10, 2), "p90": round(cold_p90, 2)},
            "cold_GBps": round(kv_bytes / (cold_med / 1e6) / 1e9, 1),
            "cold_frac_of_hbm_peak": round(kv_bytes / (cold_med / 1e6) / 1e9 / rf.HBM_PEAK_GBPS, 4)},
        "one_call_eager": {
            "what": "decode_attn launched on the stream with no graph: its two kernels back to back, warm, "
                    "and each call after the 1 GiB flush (the host enqueues it while the flush runs)",
            "us_per_call": round(us_eager, 2), "launch_floor_us": round(us_eager_floor, 2),
            "cold_us": {"median": round(eager_med, 2), "p10": round(eager_p10, 2), "p90": round(eager_p90, 2)},
            "cold_GBps": round(kv_bytes / (eager_med / 1e6) / 1e9, 1),
            "cold_frac_of_hbm_peak": round(kv_bytes / (eager_med / 1e6) / 1e9 / rf.HBM_PEAK_GBPS, 4)},
        "cold_in_graph": {
            "us_per_call": round(cold_graph, 2), "calls_per_graph": KC, "flush_bytes": 1 << 29,
            "us_per_call_rounds": [round(x, 2) for x in cold_rounds],
            "GBps": round(kv_bytes / (cold_graph / 1e6) / 1e9, 1),
            "frac_of_hbm_peak": round(kv_bytes / (cold_graph / 1e6) / 1e9 / rf.HBM_PEAK_GBPS, 4)},
        "probe_read_GBps": round(probe_gbps, 1),
        "frac_of_probe_read": round(value / probe_gbps, 4),
        "roofline": {
            "kernel": "split_kv_partial",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": rf.HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / rf.HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
            "avg_launch_us": round(us_part, 2),
        },
    }
    del g_one, g_one_floor

    # ------------------------------------------- the step before attention
    if not args.headline_only:
        result["rope_kv_write"] = [rope_step_headline(args, up, sda, workloads, rf, np, torch, stream, flush,
                                                      c4, q, ks, vs, lens)]

    # -------------------------------------------- many-token causal attention
    if not args.headline_only:
        result["prefill_attn"] = prefill_runs(up, sda, workloads, np, torch, stream, flush)

    # ----------------------------------------------- weight products (GEMV)
    if not args.headline_only:
        result["gemv"] = gemv_runs(sda, np, torch, stream, flush)

    # ---------------------------------------- speculative accept/reject step
    if not args.headline_only:
        result["spec_accept"] = spec_runs(sda, workloads, np, torch, stream, flush)

    # ------------------------------------------------------- other workloads
    if not args.headline_only:
        result["workloads"] = other_workloads(args, dev, up, sda, workloads, rf, np, torch, stream, flush,
                                             inputs)
        result["rope_kv_write"].append(result["workloads"][-1].pop("rope_kv_write"))

    # ------------------------------------------------------ CPU oracle baseline
    if cpu is not None:
        h = cpu[w4.name]
        result["cpu_baseline"] = {
            "value": h["all_cores"]["GBps"], "unit": "GB/s", "cores": h["all_cores"]["cores"], "kind": "oracle",
            "sample": f"the whole headline call (all {w4.B * w4.Hq} query rows, {kv_bytes} KV bytes), fp64 NumPy "
                      f"oracle, {h['sample'][len('the whole call, '):]} over {h['all_cores']['cores']} worker "
                      f"processes with one BLAS thread each; median of {h['all_cores']['runs']} runs of "
                      f"{h['all_cores']['s_per_unit']['median']:.3f} s",
            "s_per_call": h["all_cores"]["s_per_unit"],
            "single_core": {"value": h["GBps"], "unit": "GB/s", "cores": 1, "runs": h["runs"],
                            "s_per_call": h["s_per_unit"]}}
        for e in result.get("workloads", []):
            key = e["workload"] + (f"@{e['n']}" if e["workload"].startswith(("smollm2", "tinyllama")) and
                                   "calls_per_step" in e else "")
            if key in cpu:
                e["cpu_oracle"] = cpu[key]

    print(json.dumps(result), flush=True)


ROPE_THETA = 500000.0
ROPE_LLAMA3 = {"factor": 32.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0, "original_max_position": 8192.0}


def rope_bytes(B, T, Hq, Hkv, D):
    """Bytes a rope_kv_write call must move: q read and written, k and v read
    and written once (bf16)."""
    return B * T * D * 2 * (2 * Hq + 4 * Hkv)


def rope_timings(args, sda, torch, np, stream, flush, rope_call, attn_call, floor_call):
    """µs per call of rope alone, of its smallest launch (the floor) and of the
    rope + attention step, each in graphs of back-to-back calls, median of 5
    interleaved rounds."""
    K = 50
    graphs = {"rope": graph_of(torch, stream, [rope_call] * K),
              "floor": graph_of(torch, stream, [floor_call] * K),
              "step": graph_of(torch, stream, [f for _ in range(K // 2) for f in (rope_call, attn_call)]),
              "attn": graph_of(torch, stream, [attn_call] * (K // 2))}
    per = {n: [] for n in graphs}
    for _ in range(7):
        for n, g in graphs.items():
            calls = K if n in ("rope", "floor") else K // 2
            per[n].append(back_to_back_us(torch, stream, [g], 1, 1, busy=flush) / calls)
    res = {n: float(np.median(v)) for n, v in per.items()}
    res["dist"] = {n: dist(v) for n, v in per.items()}
    return res


def rope_step_headline(args, up, sda, workloads, rf, np, torch, stream, flush, c4, q, ks, vs, lens):
    """Decode step of the Llama-3-8B-shaped batch: rotate the new q/k, write
    k/v at each row's length, then attend over j < length + 1 (a T = 1 chunk
    call on the rotated q)."""
    w = c4["workload"]
    B, Hq, Hkv, D, S = w.B, w.Hq, w.Hkv, w.D, w.S_max
    pos0 = torch.clamp(lens, max=S - 1)
    qn = up(workloads.bf16_randn((B, 1, Hq, D), 411))
    kn = up(workloads.bf16_randn((B, 1, Hkv, D), 412))
    vn = up(workloads.bf16_randn((B, 1, Hkv, D), 413))
    q_rot = torch.empty_like(qn)
    chunk = sda.default_chunk(B, 1, Hq, Hkv, D, S)
    ws = torch.empty(sda.workspace_bytes(B, 1, Hq, Hkv, D, S, chunk), dtype=torch.uint8, device=qn.device)
    out = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device=qn.device)
    one = [up(workloads.bf16_randn((1, 1, 1, D), 414 + i)) for i in range(3)]
    kc1 = torch.zeros((1, 1, 16, D), dtype=torch.int16, device=qn.device)
    vc1 = torch.zeros_like(kc1)
    q1 = torch.empty_like(one[0])
    p1 = torch.zeros(1, dtype=torch.int32, device=qn.device)

    def rope_call():
        sda.rope_kv_write(qn, kn, vn, pos0, q_rot, ks[0], vs[0], ROPE_THETA, stream=stream)

    def attn_call():
        sda.chunk_attn(q_rot, ks[0], vs[0], pos0, c4["scale"], out, ws, chunk, stream=stream)

    def floor_call():
        sda.rope_kv_write(one[0], one[1], one[2], p1, q1, kc1, vc1, ROPE_THETA, stream=stream)

    t = rope_timings(args, sda, torch, np, stream, flush, rope_call, attn_call, floor_call)
    nb = rope_bytes(B, 1, Hq, Hkv, D)
    log(f"rope_kv_write, batched decode step: {t['rope']:.2f} us/call (floor {t['floor']:.2f}); rope + attention "
        f"{t['step']:.1f} us vs attention alone {t['attn']:.1f} us")
    return {"workload": "llama3-8b-batched-decode-step", "B": B, "T": 1, "Hq": Hq, "Hkv": Hkv, "D": D, "S_max": S,
            "theta": ROPE_THETA, "pairing": "half", "llama3_scaling": False, "calls_per_graph": 50,
            "us_per_call": round(t["rope"], 2), "launch_floor_us": round(t["floor"], 2),
            "bytes_per_call": nb, "GBps": round(nb / (t["rope"] / 1e6) / 1e9, 1),
            "step_us": round(t["step"], 2), "attention_alone_us": round(t["attn"], 2), "rounds_dist": t["dist"]}


MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak

PREFILL_CASES = [
    # name, B, T, Hq, Hkv, D, S_max, ctx
    ("llama3-8b-prefill-4096", 1, 4096, 32, 8, 128, 8192, 0),
    ("llama3-8b-chunked-prefill-2048-after-8192", 1, 2048, 32, 8, 128, 16384, 8192),
    ("smollm2-360m-prefill-4096", 1, 4096, 15, 5, 64, 8192, 0),
    ("tinyllama-1.1b-prefill-4096", 1, 4096, 32, 4, 64, 8192, 0),
]


def prefill_flops(B, T, Hq, D, ctx):
    """Algorithmic flops of causal attention: 4*D per (query row, attended key)."""
    keys = T * ctx + T * (T + 1) // 2
    return 4 * B * Hq * D * keys


def prefill_runs(up, sda, workloads, np, torch, stream, flush):
    """prefill_attn per call (graphs of 5 back-to-back calls, median of 5
    rounds) in both output modes, as TFLOP/s of algorithmic flops against the
    dense bf16 matrix peak."""
    res = []
    for ci, (name, B, T, Hq, Hkv, D, S, ctx) in enumerate(PREFILL_CASES):
        q = up(workloads.bf16_randn((B, T, Hq, D), 600 + 10 * ci + 1))
        k = up(workloads.bf16_randn((B, Hkv, S, D), 600 + 10 * ci + 2))
        v = up(workloads.bf16_randn((B, Hkv, S, D), 600 + 10 * ci + 3))
        lens = torch.full((B,), ctx, dtype=torch.int32, device=q.device)
        scale = float(np.float32(1 / np.sqrt(D)))
        entry = {"workload": name, "B": B, "T": T, "Hq": Hq, "Hkv": Hkv, "D": D, "S_max": S, "ctx": ctx,
                 "flops_per_call": prefill_flops(B, T, Hq, D, ctx), "calls_per_graph": 5}
        for dt, tag in ((torch.bfloat16, "bf16_out"), (torch.float32, "f32_out")):
            out = torch.empty((B, T, Hq, D), dtype=dt, device=q.device)
            with torch.cuda.stream(stream):
                sda.prefill_attn(q, k, v, lens, scale, out, stream=stream)
                stream.synchronize()
            g = graph_of(torch, stream, [lambda: sda.prefill_attn(q, k, v, lens, scale, out, stream=stream)] * 5)
            rounds = [back_to_back_us(torch, stream, [g], 1, 1, busy=flush) / 5 for _ in range(7)]
            us = float(np.median(rounds))
            tf = entry["flops_per_call"] / us / 1e6
            entry[tag] = {"us_per_call": round(us, 2), "us_per_call_dist": dist(rounds), "TFLOPs": round(tf, 1),
                          "frac_of_bf16_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
            del g
        log(f"prefill_attn {name}: bf16 out {entry['bf16_out']['us_per_call']:.1f} us "
            f"({entry['bf16_out']['TFLOPs']:.0f} TFLOP/s), fp32 out {entry['f32_out']['us_per_call']:.1f} us "
            f"({entry['f32_out']['TFLOPs']:.0f} TFLOP/s)")
        res.append(entry)
    return res


GEMV_MODELS = {
    # one decoder layer's weight products, fused as the pages' engine does:
    # q/k/v, o, gate/up, down ([N, K] row-major)
    "llama3-8b-layer": ([(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)], 3),
    "smollm2-360m-32-layers": ([(1600, 960), (960, 960), (5120, 960), (960, 2560)], 32),
}


def gemv_runs(sda, np, torch, stream, flush):
    """Weight products of decode steps: every layer's four matrices in one
    graph (layer copies rotate, so each matrix was last read hundreds of MB
    earlier), bf16 and INT8 weight-only, B = 1 and 8, GB/s of weight bytes
    read (INT8: codes and scales) against the 8 TB/s HBM peak."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(800)
    res = []
    for name, (mats, nl) in GEMV_MODELS.items():
        layers = [[torch.randn(m, generator=g, device=dev).to(torch.bfloat16) for m in mats] for _ in range(nl)]
        qlayers = []
        for L in layers:
            ql = []
            for W in L:
                q = torch.empty(W.shape, dtype=torch.int8, device=dev)
                sc = torch.empty(W.shape[0], dtype=torch.float32, device=dev)
                sda.quantize_rows_int8(W, q, sc)
                ql.append((q, sc))
            qlayers.append(ql)
        torch.cuda.synchronize()
        entry = {"workload": name, "matrices_NxK": [list(m) for m in mats], "layers_in_graph": nl}
        for int8 in (False, True):
            for B in (1, 8):
                xs = {K: torch.randn((B, K), generator=g, device=dev).to(torch.bfloat16) for _, K in mats}
                ys = [torch.empty((B, N), dtype=torch.bfloat16, device=dev) for N, _ in mats]

                def step(l, int8=int8, xs=xs, ys=ys):
                    for i, (N, K) in enumerate(mats):
                        if int8:
                            sda.gemv_int8(qlayers[l][i][0], qlayers[l][i][1], xs[K], ys[i], stream=stream)
                        else:
                            sda.gemv_bf16(layers[l][i], xs[K], ys[i], stream=stream)
                with torch.cuda.stream(stream):
                    step(0)
                    stream.synchronize()
                gr = graph_of(torch, stream, [lambda l=l: step(l) for l in range(nl)])
                rounds = [back_to_back_us(torch, stream, [gr], 1, 1, busy=flush) for _ in range(7)]
                us = float(np.median(rounds))
                wbytes = nl * sum(N * K * (1 if int8 else 2) + (4 * N if int8 else 0) for N, K in mats)
                gbps = wbytes / us / 1e3
                entry[f"{'int8' if int8 else 'bf16'}_B{B}"] = {
                    "us_per_graph": round(us, 1), "us_per_graph_dist": dist(rounds, nd=1), "launches": 4 * nl,
                    "weight_bytes": wbytes,
                    "GBps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / 8000.0, 4)}
                log(f"gemv {name} {'int8' if int8 else 'bf16'} B={B}: {us:.1f} us for {4 * nl} products, "
                    f"{gbps:.0f} GB/s of weights")
                del gr
        res.append(entry)
        del layers, qlayers
    return res


SPEC_CASES = [
    # name, B, T (= k + 1), V
    ("llama3.2-3b-verify-k5", 1, 6, 128256),      # tinydecode's example pairing, k = 5
    ("qwen2.5-verify-gamma8", 1, 9, 151936),      # FlashSpec's Qwen2.5 pair, gamma = 8
    ("llama3-vocab-batch64-k5", 64, 6, 128256),   # a batch of 64 rows: the bandwidth case
]


def spec_runs(sda, workloads, np, torch, stream, flush):
    """spec_accept per call, sampling (tau = 1) and greedy: graphs of 4 calls
    alternating between two copies of the inputs, median of 5 rounds. GB/s of
    algorithmic bytes: every logit read once (B*T*V*4) plus, when sampling,
    the one draft-probability row the residual needs (B*V*4)."""
    res = []
    for ci, (name, B, T, V) in enumerate(SPEC_CASES):
        entry = {"workload": name, "B": B, "T": T, "V": V, "calls_per_graph": 4}
        for tau, tag in ((1.0, "sampling"), (0.0, "greedy")):
            c = (workloads.spec_sampling_case(B, T, V, seed=700 + ci, tau=tau) if tau
                 else workloads.spec_greedy_case(B, T, V, seed=710 + ci))
            copies = []
            for _ in range(2):
                d = {k: torch.from_numpy(np.ascontiguousarray(c[k])).cuda()
                     for k in ("logits", "q", "drafts", "u", "r") if k in c}
                d["lens"] = torch.from_numpy(c["ctx"]).cuda()
                d["res"] = torch.empty((B, 2), dtype=torch.int32, device="cuda")
                d["ws"] = torch.empty(sda.spec_accept_workspace_bytes(B, T, V), dtype=torch.uint8, device="cuda")
                copies.append(d)

            def call(d):
                sda.spec_accept(d["logits"], d.get("q"), d["drafts"], d.get("u"), d.get("r"), tau, d["lens"],
                                d["res"], d["ws"], 1 << 30, stream=stream)
            with torch.cuda.stream(stream):
                call(copies[0])
                stream.synchronize()
            n_kept = copies[0]["res"][:, 0].float().mean().item()
            g = graph_of(torch, stream, [lambda d=d: call(d) for d in copies * 2])
            rounds = [back_to_back_us(torch, stream, [g], 1, 1, busy=flush) / 4 for _ in range(7)]
            us = float(np.median(rounds))
            alg = B * T * V * 4 + (B * V * 4 if tau else 0)
            gbps = alg / us / 1e3
            entry[tag] = {"us_per_call": round(us, 2), "us_per_call_dist": dist(rounds), "algorithmic_bytes": alg,
                          "GBps": round(gbps, 1),
                          "frac_of_hbm_peak": round(gbps / 8000.0, 4), "mean_drafts_kept": round(n_kept, 2),
                          "launches": 2 if tau == 0 else 3}
            log(f"spec_accept {name} {tag}: {us:.1f} us per call, {gbps:.0f} GB/s, "
                f"{n_kept:.2f} of {T - 1} drafts kept on average")
            del g, copies
        res.append(entry)
    return res


def other_workloads(args, dev, up, sda, workloads, rf, np, torch, stream, flush, inputs):
    """Workloads 1, 2, 3 and 5, each timed per graph replay over at least 50
    back-to-back replays: median, p10 and p90 of the per-replay times."""
    res = []
    steps = max(50, args.steps)
    run = lambda cfg: not args.only or args.only == str(cfg)

    # workload 1: one small call, 16 calls per graph, latency only
    if run(1):
        res.append(workload1(args, dev, up, sda, rf, torch, stream, flush, inputs, steps))

    # workloads 2 and 3: a graph of L independent layer calls per step, replayed
    # with the device-resident length rewritten; three cache sets rotate.
    # Workload 2 at its longest length also runs with one tile per row (chunk =
    # S_max), the pages' baseline for split-KV.
    for cfg in (2, 3):
        if run(cfg):
            res.extend(decode_layers(args, cfg, dev, up, sda, workloads, rf, np, torch, stream, flush, inputs, steps))

    # workload 5: verify chunk, eight calls per graph on eight cache copies
    if run(5):
        res.append(verify_chunk(args, dev, up, sda, workloads, rf, np, torch, stream, flush, inputs, steps))
    return res


def workload1(args, dev, up, sda, rf, torch, stream, flush, inputs, steps):
    """Workload 1: the single small call, 16 per graph."""
    res = []
    c = inputs[1][0]
    w = c["workload"]
    q, k, v = up(c["q"]), up(c["k"]), up(c["v"])
    lens = torch.from_numpy(c["lens"]).to(dev)
    ws = torch.empty(sda.workspace_bytes(1, 1, w.Hq, w.Hkv, w.D, w.S_max, w.chunk), dtype=torch.uint8, device=dev)
    out = torch.empty((1, w.Hq, w.D), dtype=torch.float32, device=dev)
    g1 = [graph_of(torch, stream, [lambda: sda.decode_attn(q, k, v, lens, c["scale"], out, ws, w.chunk,
                                                              stream=stream)] * 16)]
    d = dist(replay_dist_us(torch, stream, g1, steps, args.warmup, busy=flush), 1 / 16)
    res.append({"workload": w.name, "n": 64, "chunk": w.chunk, "calls_per_graph": 16, "us_per_call": d["median"],
                "us_per_call_dist": d, "kv_bytes_per_call": rf.kv_bytes_decode([64], w.Hkv, w.D, w.S_max)})
    log(f"workload 1: {d['median']:.2f} us/call (p10 {d['p10']:.2f}, p90 {d['p90']:.2f})")
    del g1
    return res[0]


def decode_layers(args, cfg, dev, up, sda, workloads, rf, np, torch, stream, flush, inputs, steps):
    """Workloads 2 and 3: graphs of a step's layer calls at each length."""
    res = []
    w = workloads.CONFIGS[cfg]
    lengths = [int(x) for x in args.lengths.split(",")] if args.lengths else list(w.lens)
    layers = inputs[cfg]
    lens = torch.zeros(1, dtype=torch.int32, device=dev)
    sets = []
    for si in range(3):
        tens = []
        for l, cl in enumerate(layers):
            kq = up(cl["q"])
            kk = up(cl["k"]) if si == 0 else sets[0][l][1].clone()
            vv = up(cl["v"]) if si == 0 else sets[0][l][2].clone()
            o = torch.empty((1, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
            tens.append((kq, kk, vv, o))
        sets.append(tens)
    scale = layers[0]["scale"]
    chunk = args.chunk or sda.default_chunk(1, 1, w.Hq, w.Hkv, w.D, w.S_max)

    def make_graphs(ch):
        wsl = [torch.empty(sda.workspace_bytes(1, 1, w.Hq, w.Hkv, w.D, w.S_max, ch), dtype=torch.uint8,
                           device=dev) for _ in layers]

        def step_fns(tens):
            return [lambda t=t, wl=wl: sda.decode_attn(t[0], t[1], t[2], lens, scale, t[3], wl, ch,
                                                       stream=stream)
                    for t, wl in zip(tens, wsl)]
        lens.fill_(max(lengths))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for tens in sets:
                for fn in step_fns(tens):
                    fn()
            stream.synchronize()
        return [graph_of(torch, stream, step_fns(tens)) for tens in sets], wsl

    graphs, _wsl = make_graphs(chunk)
    floor = {"median": None, "p10": None, "p90": None}
    if not args.no_floor:
        lens.fill_(0)
        torch.cuda.synchronize()
        floor = dist(replay_dist_us(torch, stream, graphs, steps, args.warmup, busy=flush))
    for n in lengths:
        lens.fill_(n)
        torch.cuda.synchronize()
        d = dist(replay_dist_us(torch, stream, graphs, steps, args.warmup, busy=flush))
        us = d["median"]
        kvb = rf.kv_bytes_decode([n], w.Hkv, w.D, w.S_max) * w.layers
        res.append({"workload": w.name, "n": n, "chunk": chunk, "calls_per_step": w.layers,
                    "us_per_step": us, "us_per_step_dist": d, "us_per_call": round(us / w.layers, 3),
                    "launch_floor_us_per_step": floor["median"], "launch_floor_us_per_step_dist": floor,
                    "kv_bytes_per_step": kvb, "GBps": round(kvb / (us / 1e6) / 1e9, 1),
                    "frac_of_hbm_peak": round(kvb / (us / 1e6) / 1e9 / rf.HBM_PEAK_GBPS, 4)})
        log(f"workload {cfg} n={n}: {us:.1f} us/step ({us / w.layers:.2f} us/call, p10 {d['p10']:.1f}, "
            f"p90 {d['p90']:.1f}), {res[-1]['GBps']:.0f} GB/s (floor {floor['median']} us/step)")
    del graphs, _wsl
    if cfg == 2 and not args.lengths:
        n = max(w.lens)
        graphs, _wsl = make_graphs(w.S_max)
        lens.fill_(n)
        torch.cuda.synchronize()
        d = dist(replay_dist_us(torch, stream, graphs, steps, args.warmup, busy=flush))
        kvb = rf.kv_bytes_decode([n], w.Hkv, w.D, w.S_max) * w.layers
        res[-1]["one_tile_ablation"] = {
            "what": "the same step with chunk = S_max: one tile (one workgroup) per kv head",
            "chunk": w.S_max, "us_per_step": d["median"], "us_per_step_dist": d,
            "us_per_call": round(d["median"] / w.layers, 3), "GBps": round(kvb / (d["median"] / 1e6) / 1e9, 1),
            "split_kv_speedup": round(d["median"] / res[-1]["us_per_step"], 2)}
        log(f"workload 2 n={n}, one tile per row: {d['median'] / w.layers:.2f} us/call "
            f"({res[-1]['one_tile_ablation']['split_kv_speedup']:.2f}x the split-KV time)")
        del graphs, _wsl
    torch.cuda.synchronize()
    del sets
    return res


def verify_chunk(args, dev, up, sda, workloads, rf, np, torch, stream, flush, inputs, steps):
    """Workload 5: the verify chunk, eight calls per graph on eight cache
    copies, then the rotary/K-V write of the verify step beside it."""
    res = []
    c = inputs[5][0]
    w = c["workload"]
    chunk = args.chunk or sda.default_chunk(w.B, w.T, w.Hq, w.Hkv, w.D, w.S_max)
    q = up(c["q"])
    k0, v0 = up(c["k"]), up(c["v"])
    kvs = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(7)]
    lens = torch.from_numpy(c["lens"]).to(dev)
    ws = torch.empty(sda.workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.D, w.S_max, chunk), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.T, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    with torch.cuda.stream(stream):
        sda.chunk_attn(q, k0, v0, lens, c["scale"], out, ws, chunk, stream=stream)
        stream.synchronize()
    g5 = [graph_of(torch, stream, [lambda kv=kv: sda.chunk_attn(q, kv[0], kv[1], lens, c["scale"], out, ws, chunk,
                                                                   stream=stream) for kv in kvs])]
    d = dist(replay_dist_us(torch, stream, g5, steps, args.warmup, busy=flush), 1 / len(kvs))
    us = d["median"]
    kvb = rf.kv_bytes_chunk(c["lens"], w.T, w.Hkv, w.D, w.S_max)
    res.append({"workload": w.name, "ctx": int(c["lens"][0]), "T": w.T, "chunk": chunk,
                "calls_per_graph": len(kvs), "us_per_call": us, "us_per_call_dist": d,
                "kv_bytes_per_call": kvb, "GBps": round(kvb / (us / 1e6) / 1e9, 1),
                "frac_of_hbm_peak": round(kvb / (us / 1e6) / 1e9 / rf.HBM_PEAK_GBPS, 4)})
    log(f"workload 5: {us:.1f} us/call (p10 {d['p10']:.1f}, p90 {d['p90']:.1f}), {res[-1]['GBps']:.0f} GB/s")
    del g5

    # the verify step before attention: rotate and write the T draft tokens
    # (llama3 frequency scaling), then the chunk call on the rotated q
    qn = up(workloads.bf16_randn((w.B, w.T, w.Hq, w.D), 511))
    kn = up(workloads.bf16_randn((w.B, w.T, w.Hkv, w.D), 512))
    vn = up(workloads.bf16_randn((w.B, w.T, w.Hkv, w.D), 513))
    q_rot = torch.empty_like(qn)
    one = [up(workloads.bf16_randn((1, 1, 1, w.D), 514 + i)) for i in range(3)]
    kc1 = torch.zeros((1, 1, 16, w.D), dtype=torch.int16, device=dev)
    vc1 = torch.zeros_like(kc1)
    q1 = torch.empty_like(one[0])
    p1 = torch.zeros(1, dtype=torch.int32, device=dev)

    def rope_call():
        sda.rope_kv_write(qn, kn, vn, lens, q_rot, k0, v0, ROPE_THETA, llama3=ROPE_LLAMA3, stream=stream)

    def attn_call():
        sda.chunk_attn(q_rot, k0, v0, lens, c["scale"], out, ws, chunk, stream=stream)

    def floor_call():
        sda.rope_kv_write(one[0], one[1], one[2], p1, q1, kc1, vc1, ROPE_THETA, llama3=ROPE_LLAMA3, stream=stream)

    t = rope_timings(args, sda, torch, np, stream, flush, rope_call, attn_call, floor_call)
    nb = rope_bytes(w.B, w.T, w.Hq, w.Hkv, w.D)
    log(f"rope_kv_write, verify step: {t['rope']:.2f} us/call (floor {t['floor']:.2f}); rope + chunk attention "
        f"{t['step']:.1f} us vs chunk attention alone {t['attn']:.1f} us")
    res[-1]["rope_kv_write"] = {
        "workload": "llama3.2-3b-verify-step", "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
        "S_max": w.S_max, "theta": ROPE_THETA, "pairing": "half", "llama3_scaling": ROPE_LLAMA3,
        "calls_per_graph": 50, "us_per_call": round(t["rope"], 2), "launch_floor_us": round(t["floor"], 2),
        "bytes_per_call": nb, "GBps": round(nb / (t["rope"] / 1e6) / 1e9, 1),
        "step_us": round(t["step"], 2), "attention_alone_us": round(t["attn"], 2), "rounds_dist": t["dist"]}
    return res[0]


# ------------------------------------------------------------ CPU oracle baseline
#
# The fp64 oracle, as it stands, timed on this host's cores in the same run as
# the GPU figures. It runs before the GPU is touched: the all-cores leg is a
# pool of forked worker processes, and a process that has initialised the GPU
# is not forked. Every workload's call (or step of layer calls) is split into
# independent slices -- one sequence and a range of kv heads with their query
# heads -- and each slice is the unchanged oracle on that part of the inputs
# (heads do not interact, so the slices' outputs are the call's output).

_ORACLE_INPUTS = {}     # name -> list of per-call inputs; forked workers inherit it


def _oracle_slice(task):
    """Oracle output of one slice: (name, call, b, kv0, kv1, n) -> array. A
    length n overrides the call's own (workloads 2 and 3 replay one cache at
    several lengths)."""
    import numpy as np
    import oracle
    name, call, b, kv0, kv1, n = task
    c = _ORACLE_INPUTS[name][call]
    k, v = c["k"][b:b + 1, kv0:kv1], c["v"][b:b + 1, kv0:kv1]
    G = c["q"].shape[-2] // c["k"].shape[1]
    lens = c["lens"][b:b + 1] if n is None else np.array([n], np.int32)
    if c["q"].ndim == 4:        # a verify chunk [B, T, Hq, D]
        return oracle.chunk_attention(c["q"][b:b + 1, :, kv0 * G:kv1 * G], k, v, lens, c["scale"])
    return oracle.decode_attention(c["q"][b:b + 1, kv0 * G:kv1 * G], k, v, lens, c["scale"])


def _limit_blas_threads():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _timed_runs(fn, budget_s, min_runs=3, max_runs=200):
    """Median, p10, p90 seconds of fn() over at least min_runs runs and about
    budget_s seconds, and the number of runs."""
    import numpy as np
    times = []
    while len(times) < min_runs or (sum(times) < budget_s and len(times) < max_runs):
        t = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t)
    return (float(np.median(times)), float(np.percentile(times, 10)), float(np.percentile(times, 90)),
            len(times))


def cpu_oracle_runs(inputs, rf, budget_s=1.5):
    """The oracle on every workload, one BLAS thread in one process, then the
    same slices over a pool of worker processes (one BLAS thread each). Returns
    {key: entry}; the keys name the workload (and length)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    plans = []      # (key, tasks, unit calls, kv bytes per unit, description)
    for cfg, cs in inputs.items():
        w = cs[0]["workload"]
        _ORACLE_INPUTS[w.name] = cs
        if cfg in (2, 3):
            for n in w.lens:
                tasks = [(w.name, l, 0, 0, w.Hkv, n) for l in range(len(cs))]
                kvb = rf.kv_bytes_decode([n], w.Hkv, w.D, w.S_max) * len(cs)
                plans.append((f"{w.name}@{n}", tasks, len(cs), kvb,
                              f"a whole step: {len(cs)} layer calls at n = {n}, one task per layer"))
        elif cfg == 5:
            tasks = [(w.name, 0, 0, h, h + 1, None) for h in range(w.Hkv)]
            kvb = rf.kv_bytes_chunk(cs[0]["lens"], w.T, w.Hkv, w.D, w.S_max)
            plans.append((w.name, tasks, 1, kvb, f"the whole call, one task per kv head ({w.Hkv})"))
        else:
            tasks = [(w.name, 0, b, h, h + 1, None) for b in range(w.B) for h in range(w.Hkv)]
            kvb = rf.kv_bytes_decode(cs[0]["lens"], w.Hkv, w.D, w.S_max)
            plans.append((w.name, tasks, 1, kvb, f"the whole call, one task per (sequence, kv head) "
                                                  f"({len(tasks)})"))
    res = {}
    with threadpool_limits(1):
        for key, tasks, calls, kvb, desc in plans:
            budget = budget_s * (3 if key.startswith("llama3-8b") else 1)
            med, p10, p90, runs = _timed_runs(lambda: [_oracle_slice(t) for t in tasks], budget)
            res[key] = {"kind": "oracle", "cores": 1, "sample": desc, "runs": runs,
                        "s_per_unit": {"median": med, "p10": p10, "p90": p90},
                        "us_per_call": round(med / calls * 1e6, 1), "GBps": round(kvb / med / 1e9, 4)}
            log(f"cpu oracle {key}, 1 core: {med * 1e3:.1f} ms ({kvb / med / 1e9:.3f} GB/s), {runs} runs")
    workers = min(16, len(os.sched_getaffinity(0)))
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("fork"),
                             initializer=_limit_blas_threads) as pool:
        list(pool.map(abs, range(4 * workers)))          # fork every worker before timing
        for key, tasks, calls, kvb, desc in plans:
            budget = budget_s * (3 if key.startswith("llama3-8b") else 1)
            med, p10, p90, runs = _timed_runs(lambda: list(pool.map(_oracle_slice, tasks)), budget)
            res[key]["all_cores"] = {"cores": workers, "runs": runs,
                                     "s_per_unit": {"median": med, "p10": p10, "p90": p90},
                                     "us_per_call": round(med / calls * 1e6, 1),
                                     "GBps": round(kvb / med / 1e9, 4),
                                     "sample": f"the same tasks over {workers} worker processes, "
                                               f"one BLAS thread each"}
            log(f"cpu oracle {key}, {workers} processes: {med * 1e3:.1f} ms ({kvb / med / 1e9:.3f} GB/s)")
    _ORACLE_INPUTS.clear()
    return res


if __name__ == "__main__":
    main()
