#!/usr/bin/env python3
"""Split-KV decode attention on one MI355X: one JSON line on stdout.

Headline step: one decode_attn call (partial-tile kernel + log-sum-exp merge)
on the Llama-3-8B-shaped batched decode (B=8, Hq=32, Hkv=8, D=128,
S_max=32768, ragged seq_lens ~ U[1, 32768] from a fixed seed), inputs resident
in HBM. Two copies of the cache alternate between steps so that no step finds
its data in the 256 MB Infinity Cache left there by the step before.

value = algorithmic KV bytes per step / wall time per step (GB/s); the partial
kernel alone is timed with HIP events on the launch stream for the roofline
entry. The other four workloads are timed the same way and reported under
"workloads". The fp64 CPU oracle is timed on the headline workload on this
host as "cpu_baseline".

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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--chunk", type=int, default=0, help="override the library's default tile size")
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

    sda.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

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

    # ------------------------------------------------------ headline: workload 4
    t = time.time()
    c4 = workloads.make_config(4)
    w4 = c4["workload"]
    log(f"workload 4 generated in {time.time() - t:.1f}s, lens {c4['lens'].tolist()}")
    q = up(c4["q"])
    ks = [up(c4["k"])]
    vs = [up(c4["v"])]
    ks.append(ks[0].clone())
    vs.append(vs[0].clone())
    lens = torch.from_numpy(c4["lens"]).to(dev)
    chunk = args.chunk or sda.default_chunk(w4.B, 1, w4.Hq, w4.Hkv, w4.D, w4.S_max)
    ws = torch.empty(sda.workspace_bytes(w4.B, 1, w4.Hq, w4.Hkv, w4.D, w4.S_max, chunk),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((w4.B, w4.Hq, w4.D), dtype=torch.bfloat16, device=dev)
    kv_bytes = rf.kv_bytes_decode(c4["lens"], w4.Hkv, w4.D, w4.S_max)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        sda.attn_partial(q, ks[i % 2], vs[i % 2], lens, c4["scale"], ws, chunk=chunk)
        if ev is not None:
            ev[1].record()
        sda.attn_merge(lens, out, ws, T=1, Hq=w4.Hq, Hkv=w4.Hkv, S_max=w4.S_max, chunk=chunk)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    partial_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    value = kv_bytes / (ms_per_step / 1e3) / 1e9
    achieved = kv_bytes / (partial_ms / 1e3) / 1e9
    log(f"workload 4: {ms_per_step * 1e3:.1f} us/call, {value:.0f} GB/s; partial kernel "
        f"{partial_ms * 1e3:.1f} us = {achieved:.0f} GB/s")

    # also without events between the kernels
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        sda.decode_attn(q, ks[i % 2], vs[i % 2], lens, c4["scale"], out, ws, chunk)
    torch.cuda.synchronize()
    plain_us = (time.perf_counter() - t0) * 1e6 / args.steps

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
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w4.name, "B": w4.B, "Hq": w4.Hq, "Hkv": w4.Hkv, "D": w4.D, "S_max": w4.S_max,
            "seq_lens": c4["lens"].tolist(), "chunk": chunk, "kv_dtype": "bf16", "out_dtype": "bf16",
            "kv_bytes_per_call": kv_bytes,
        },
        "us_per_call": round(ms_per_step * 1e3, 2),
        "us_per_call_without_events": round(plain_us, 2),
        "frac_of_hbm_peak": round(value / rf.HBM_PEAK_GBPS, 4),
        "probe_read_GBps": round(probe_gbps, 1),
        "roofline": {
            "kernel": "split_kv_partial",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": rf.HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / rf.HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
            "avg_launch_us": round(partial_ms * 1e3, 2),
        },
    }
    del ks, vs, q

    # ------------------------------------------------------- other workloads
    if not args.headline_only:
        result["workloads"] = other_workloads(args, dev, up, sda, workloads, rf, np, torch)

    # ------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(c4, rf, np)

    print(json.dumps(result), flush=True)


def timed_replays(fn, n, warm, torch):
    """Median and mean of n event-timed calls of fn(i) after warm untimed ones."""
    import numpy as np
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    times = []
    for i in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    return float(np.median(times)), float(np.mean(times))


def other_workloads(args, dev, up, sda, workloads, rf, np, torch):
    res = []
    reps = max(10, args.steps)

    # workload 1: one small call, latency only
    c = workloads.make_config(1)
    w = c["workload"]
    q, k, v = up(c["q"]), up(c["k"]), up(c["v"])
    lens = torch.from_numpy(c["lens"]).to(dev)
    ws = torch.empty(sda.workspace_bytes(1, 1, w.Hq, w.Hkv, w.D, w.S_max, w.chunk), dtype=torch.uint8, device=dev)
    out = torch.empty((1, w.Hq, w.D), dtype=torch.float32, device=dev)
    med, _ = timed_replays(lambda i: sda.decode_attn(q, k, v, lens, c["scale"], out, ws, w.chunk), reps, 3, torch)
    res.append({"workload": w.name, "n": 64, "chunk": w.chunk, "us_per_call": round(med, 2),
                "kv_bytes_per_call": rf.kv_bytes_decode([64], w.Hkv, w.D, w.S_max)})

    # workloads 2 and 3: a graph of L independent layer calls per step, replayed
    # with the device-resident length rewritten; three cache sets rotate
    for cfg in (2, 3):
        w = workloads.CONFIGS[cfg]
        layers = [workloads.make_config(cfg, layer=l) for l in range(w.layers)]
        chunk = sda.default_chunk(1, 1, w.Hq, w.Hkv, w.D, w.S_max)
        lens = torch.zeros(1, dtype=torch.int32, device=dev)
        sets = []
        for s in range(3):
            tens = []
            for l, cl in enumerate(layers):
                kq = up(cl["q"])
                kk = up(cl["k"]) if s == 0 else sets[0][l][1].clone()
                vv = up(cl["v"]) if s == 0 else sets[0][l][2].clone()
                wsl = torch.empty(sda.workspace_bytes(1, 1, w.Hq, w.Hkv, w.D, w.S_max, chunk),
                                  dtype=torch.uint8, device=dev)
                o = torch.empty((1, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
                tens.append((kq, kk, vv, wsl, o))
            sets.append(tens)
        scale = layers[0]["scale"]
        lens.fill_(max(w.lens))
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for tens in sets:
                for (kq, kk, vv, wsl, o) in tens:
                    sda.decode_attn(kq, kk, vv, lens, scale, o, wsl, chunk)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for tens in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for (kq, kk, vv, wsl, o) in tens:
                    sda.decode_attn(kq, kk, vv, lens, scale, o, wsl, chunk)
            graphs.append(g)
        for n in w.lens:
            lens.fill_(n)
            med, mean = timed_replays(lambda i: graphs[i % 3].replay(), reps, 3, torch)
            kvb = rf.kv_bytes_decode([n], w.Hkv, w.D, w.S_max) * w.layers
            res.append({"workload": w.name, "n": n, "chunk": chunk, "calls_per_step": w.layers,
                        "us_per_step": round(med, 2), "us_per_call": round(med / w.layers, 3),
                        "kv_bytes_per_step": kvb, "GBps": round(kvb / (med / 1e6) / 1e9, 1),
                        "frac_of_hbm_peak": round(kvb / (med / 1e6) / 1e9 / rf.HBM_PEAK_GBPS, 4)})
            log(f"workload {cfg} n={n}: {med:.1f} us/step ({med / w.layers:.2f} us/call), "
                f"{res[-1]['GBps']:.0f} GB/s")
        del graphs, sets, layers
        torch.cuda.synchronize()

    # workload 5: verify chunk, eight cache copies rotate
    c = workloads.make_config(5)
    w = c["workload"]
    chunk = sda.default_chunk(w.B, w.T, w.Hq, w.Hkv, w.D, w.S_max)
    q = up(c["q"])
    k0, v0 = up(c["k"]), up(c["v"])
    kvs = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(7)]
    lens = torch.from_numpy(c["lens"]).to(dev)
    ws = torch.empty(sda.workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.D, w.S_max, chunk), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.T, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    med, _ = timed_replays(lambda i: sda.chunk_attn(q, kvs[i % 8][0], kvs[i % 8][1], lens, c["scale"], out, ws, chunk),
                           reps, 3, torch)
    kvb = rf.kv_bytes_chunk(c["lens"], w.T, w.Hkv, w.D, w.S_max)
    res.append({"workload": w.name, "ctx": int(c["lens"][0]), "T": w.T, "chunk": chunk, "us_per_call": round(med, 2),
                "kv_bytes_per_call": kvb, "GBps": round(kvb / (med / 1e6) / 1e9, 1),
                "frac_of_hbm_peak": round(kvb / (med / 1e6) / 1e9 / rf.HBM_PEAK_GBPS, 4)})
    log(f"workload 5: {med:.1f} us/call, {res[-1]['GBps']:.0f} GB/s")
    return res


def cpu_baseline(c4, rf, np):
    """The fp64 oracle, as it stands, on every row of the headline workload, one thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    w = c4["workload"]
    kvb = rf.kv_bytes_decode(c4["lens"], w.Hkv, w.D, w.S_max)
    times = []
    with threadpool_limits(1):
        for _ in range(3):
            t = time.perf_counter()
            oracle.decode_attention(c4["q"], c4["k"], c4["v"], c4["lens"], c4["scale"])
            times.append(time.perf_counter() - t)
    med = float(np.median(times))
    log(f"cpu oracle: {med:.2f} s per call ({kvb / med / 1e9:.3f} GB/s)")
    return {"value": round(kvb / med / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole headline call (all {w.B * w.Hq} query rows, {kvb} KV bytes), "
                      f"fp64 NumPy, BLAS limited to 1 thread, median of 3 runs of {med:.2f} s"}


if __name__ == "__main__":
    main()
