#!/usr/bin/env python3
"""Benchmark of the paged-attention decode step on one MI355X.

A step is the whole hot path for one layer: pa_reshape_and_cache writes the
step's new token of every sequence into its slot, then pa_decode (partition
kernel + log-sum-exp reduce) attends over the paged K/V.  Inputs are seeded
synthetic tensors, already resident in HBM when the timed region starts.

    python bench.py [--steps K] [--warmup W] [--config C [--block-size B]
                    [--partition-size P]] [--kv-dtype fp16|fp8] [--no-flush]
                    [--no-cpu-baseline]

Prints ONE JSON line.  By default the headline is the largest single-GPU
workload, the LLaMA-13B-shaped layer (config 2: 256 sequences x 40 heads x
128, block size 16, 1024-token partitions), and `per_config` carries every
configuration in the same run: configs 0, 1, 2 at block sizes 16 and 32, 3
through pa_decode and through pa_decode_cascade (the shared prefix read once
per 64 sequences), and 4; each with its decode time, tokens/s/layer, the
fraction of the 8 TB/s HBM peak on its unique K/V bytes, and the median
decode time after a 1 GiB write that evicts the L2s and the MALL.  --config
measures one workload only.

value = K/V bytes the decode must read per step (sum of context lengths x
heads x head_dim x 2 tensors x 2 bytes) divided by the step time of K steps
run back to back between two HIP events, in GB/s; tokens/s/layer =
sequences / step time.  roofline: K decode calls back to back between two
HIP events on the stream the library launches on, against the 8 TB/s HBM3E
peak and the measured streaming-read peak; traffic: HBM bytes per launch from
the committed counter runs (profiles/traffic.json) when they were taken on
the current device code, with their source.  cpu_baseline: the CPU oracle
timed on a bounded sample of the headline workload on the host cores.

`--op cascade | multi_query | copy_blocks | swap` time the other entry
points; `--probe copy` runs a plain copy of known size (reshape_and_cache
over 1 GiB) for calibrating hardware byte counters; `--probe read` runs the
streaming-read probe (read_probe.hip, built by __graft_entry__.build()) whose
best rate is the achievable-peak figure the roofline also reports against.
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged-attn decode KV-read GB/s (fraction of HBM peak); decode tokens/s/layer"


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first (the GPU's clocks settle within some 20 ms)")
    ap.add_argument("--config", type=int, default=None,
                    help="one workload only; default: config 2 (B 16) as the headline, with "
                         "every configuration in per_config")
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--kv-dtype", choices=["fp16", "fp8"], default="fp16",
                    help="cache element type: fp16, or FP8 (OCP E4M3, one scale per cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=float, default=1.0e7,
                    help="cap on token-heads of oracle work in the CPU baseline sample")
    ap.add_argument("--cpu-repeats", type=int, default=3,
                    help="least number of timed oracle runs of the sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="keep repeating the oracle sample until this much wall time is spent")
    ap.add_argument("--op", choices=["step", "copy_blocks", "swap", "cascade", "multi_query"],
                    default="step",
                    help="step: the decode step (default); copy_blocks / swap: the block "
                         "copy-on-write and GPU<->host swap entry points on config 1's pool; "
                         "cascade: the shared-prefix step through pa_decode_cascade (config "
                         "3); multi_query: a chunked-prefill batch through pa_multi_query")
    ap.add_argument("--pairs", type=int, default=1024, help="blocks per copy/swap call")
    ap.add_argument("--probe", choices=["copy", "read"], default=None)
    ap.add_argument("--call", choices=["decode", "cascade"], default="decode",
                    help="with --config: the entry point timed (cascade: config 3 through "
                         "pa_decode_cascade, its 32 shared blocks as the prefix table)")
    ap.add_argument("--ingest-traffic", nargs=3, metavar=("KEY", "FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn the FETCH_SIZE / WRITE_SIZE counter csvs of rocprofv3 "
                         "--pmc runs of one workload into profiles/traffic.json[KEY]")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the flushed decode timings (a 1 GiB write before each call "
                         "evicts the L2s and the MALL)")
    ap.add_argument("--probe-mib", type=int, default=1024)
    return ap.parse_args()


def _code_sha(*paths):
    """sha256 (16 hex digits) of C/HIP sources with their comments and blank
    lines removed: a comment edit does not invalidate counters taken on the
    same code."""
    import re
    parts = []
    for path in paths:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
        parts.append("\n".join(ln for ln in lines if ln.strip()))
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()[:16]


CSRC = os.path.join(ROOT, "paged_kv_cache_155_amd", "csrc")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_code_sha():
    """Key of the library's device code: every csrc source and header
    (comments aside) and the compiler flags.  Counters recorded under another
    key were taken on other code and are not reported."""
    import glob
    from paged_kv_cache_155_amd import _build
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))
                  + [os.path.join(ROOT, "include", "pa.h")])
    flags = " ".join(f for f in _build.FLAGS if not f.startswith("-I"))  # no checkout paths
    return hashlib.sha256((_code_sha(*srcs) + flags).encode()).hexdigest()[:16]


def _traffic(config_name):
    """(per-launch HBM bytes, source) from the committed counter runs in
    profiles/traffic.json, if they were taken on the current device code;
    else (None, reason)."""
    if not os.path.exists(TRAFFIC_JSON):
        return None, "no profiles/traffic.json"
    try:
        rec = json.load(open(TRAFFIC_JSON)).get(config_name)
    except (ValueError, AttributeError):
        return None, "unreadable profiles/traffic.json"
    if not rec:
        return None, f"no counters for {config_name} in profiles/traffic.json"
    sha = kernel_code_sha()
    if rec.get("kernel_code_sha") != sha:
        return None, (f"profiles/traffic.json[{config_name}] was taken on code "
                      f"{rec.get('kernel_code_sha')}, current {sha}")
    return rec.get("bytes_per_launch"), f"profiles/traffic.json[{config_name}]@{sha}"


def _traffic_fields(config_name):
    b, src = _traffic(config_name)
    return {"traffic": b, "traffic_source": src}


def probe_copy(mib):
    import torch
    import paged_kv_cache_155_amd as pa
    H, D = 32, 128
    row = H * D * 2
    T = mib * 1024 * 1024 // (2 * row)  # K and V together = mib MiB read
    key = torch.randn(T, H, D, device="cuda").half()
    val = torch.randn(T, H, D, device="cuda").half()
    kc = torch.empty(T // 16, 16, H, D, dtype=torch.float16, device="cuda")
    vc = torch.empty_like(kc)
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    for _ in range(3):
        pa.reshape_and_cache(key, val, kc, vc, slots)
    torch.cuda.synchronize()
    assert torch.equal(kc.view(-1), key.view(-1))
    print(json.dumps({"probe": "copy", "kernel": "reshape_and_cache_kernel", "launches": 3,
                      "read_bytes_per_launch": 2 * T * row + 8 * T,
                      "write_bytes_per_launch": 2 * T * row}), flush=True)


PCIE5_X16_GBS = 63.0  # 32 GT/s x 16 lanes x 128/130 / 8, one direction


def _time_events(fn, iters, warmup=3):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def bench_blocks(op, pairs, iters, cpu=None):
    """copy_blocks: `pairs` random (src -> fresh dst) block copies inside
    config 1's K/V pool; swap: `pairs` blocks of K and of V out to pinned host
    memory and back in.  One JSON line per measured direction."""
    import numpy as np
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import make_workload
    w = make_workload(1, poison=False)
    kc = torch.from_numpy(w.k_cache).cuda()
    vc = torch.from_numpy(w.v_cache).cuda()
    block_bytes = w.k_cache[0].nbytes
    rng = np.random.default_rng(155)
    perm = rng.permutation(w.num_blocks)
    n = min(pairs, w.num_blocks // 2)
    lines = []
    if op == "copy_blocks":
        mapping = torch.from_numpy(np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int64)).cuda()
        ms = _time_events(lambda: pa.copy_blocks(kc, vc, mapping), iters)
        moved = n * block_bytes * 2 * 2  # K and V, read + write
        t = float(np.median(ms)) * 1e-3
        line_cpu = None
        if cpu is not None:  # the oracle's block copy on host copies of the same pool
            import oracle
            orc = oracle.get()
            okc, ovc = w.k_cache.copy(), w.v_cache.copy()
            m = mapping.cpu().numpy()
            dt, runs = _time_oracle(lambda: orc.copy_blocks(okc, ovc, m), cpu.cpu_repeats,
                                    cpu.cpu_seconds / 4)
            line_cpu = {"value": round(moved / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                        "kind": "oracle", "cpu": _cpu_model(),
                        "sample": f"the same {n} block pairs on host copies of the pool; "
                                  f"median of {runs} runs = {dt * 1e3:.2f} ms"}
        lines.append({"op": "copy_blocks", "pairs": n, "block_bytes": block_bytes,
                      "bytes_per_call": moved, "us_median": round(t * 1e6, 2),
                      "roofline": {"bound": "hbm", "achieved": round(moved / t / 1e9, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(moved / t / 1e9 / HBM_PEAK_GBS, 4)},
                      "cpu_baseline": line_cpu})
    else:
        hk = torch.empty((n,) + tuple(kc.shape[1:]), dtype=torch.float16).pin_memory()
        hv = torch.empty_like(hk).pin_memory()
        out_map = torch.from_numpy(np.stack([perm[:n], np.arange(n)], 1).astype(np.int64))
        in_map = torch.from_numpy(np.stack([np.arange(n), perm[n:2 * n]], 1).astype(np.int64))

        def out_():
            pa.swap_blocks(kc, hk, out_map)
            pa.swap_blocks(vc, hv, out_map)

        def in_():
            pa.swap_blocks(hk, kc, in_map)
            pa.swap_blocks(hv, vc, in_map)

        orc = None
        if cpu is not None:  # the oracle's block swap between host arrays of the same shapes
            import oracle
            orc = oracle.get()
            hpool_k, hpool_v = w.k_cache.copy(), w.v_cache.copy()
            hbuf_k = np.zeros((n,) + w.k_cache.shape[1:], dtype=np.float16)
            hbuf_v = np.zeros_like(hbuf_k)
            om, im = out_map.numpy(), in_map.numpy()
            oracle_fns = {"swap_out": lambda: (orc.swap_blocks(hpool_k, hbuf_k, om),
                                               orc.swap_blocks(hpool_v, hbuf_v, om)),
                          "swap_in": lambda: (orc.swap_blocks(hbuf_k, hpool_k, im),
                                              orc.swap_blocks(hbuf_v, hpool_v, im))}
        for name, fn in (("swap_out", out_), ("swap_in", in_)):
            ms = _time_events(fn, iters)
            moved = n * block_bytes * 2
            t = float(np.median(ms)) * 1e-3
            line_cpu = None
            if orc is not None:
                dt, runs = _time_oracle(oracle_fns[name], cpu.cpu_repeats, cpu.cpu_seconds / 4)
                line_cpu = {"value": round(moved / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                            "kind": "oracle", "cpu": _cpu_model(),
                            "sample": f"the same {n} blocks of K and of V between host arrays; "
                                      f"median of {runs} runs = {dt * 1e3:.2f} ms"}
            lines.append({"op": name, "pairs": n, "block_bytes": block_bytes,
                          "bytes_per_call": moved, "us_median": round(t * 1e6, 2),
                          "roofline": {"bound": "pcie", "achieved": round(moved / t / 1e9, 2),
                                       "peak": PCIE5_X16_GBS, "unit": "GB/s",
                                       "frac": round(moved / t / 1e9 / PCIE5_X16_GBS, 4)},
                          "cpu_baseline": line_cpu})
    for ln in lines:
        print(json.dumps(ln), flush=True)


MFMA_F16_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak


def bench_cascade(iters, warmup, cpu=None, fp8=False):
    """Shared-prefix step (config 3) with the prefix read once per 64
    sequences: pa_decode_cascade_append (the new tokens are written by the
    prefix pass's launch); the same step as two calls (reshape_and_cache +
    pa_decode_cascade) is reported beside it.  FP8 caches: the _fp8 forms."""
    import numpy as np
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import (DESCRIPTIONS, fp8_pools, make_workload,
                                                  split_shared_prefix)
    w = make_workload(3, poison=False)
    prefix, plen, st, sl = split_shared_prefix(w, 32)

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    f8 = fp8_pools(w) if fp8 else None
    kc, vc = (up(f8.k_cache), up(f8.v_cache)) if fp8 else (up(w.k_cache), up(w.v_cache))
    q = up(w.q)
    key, val, slots = up(w.key), up(w.value), up(w.slot_mapping)
    pt, stt, slt = up(prefix), up(st), up(sl)
    out = torch.empty_like(q)
    P = 0
    ws = torch.empty(pa.decode_cascade_workspace_size(w.num_seqs, w.num_heads, w.head_dim,
                                                      w.block_size, plen, st.shape[1], P),
                     dtype=torch.uint8, device="cuda")
    scale = float(w.scale)
    stream = torch.cuda.current_stream()

    def reshape():
        if fp8:
            pa.reshape_and_cache_fp8(key, val, kc, vc, slots, f8.k_scale, f8.v_scale)
        else:
            pa.reshape_and_cache(key, val, kc, vc, slots)

    def decode():
        if fp8:
            pa.decode_cascade_fp8(out, q, kc, vc, pt, plen, stt, slt, scale, f8.k_scale,
                                  f8.v_scale, P, ws)
        else:
            pa.decode_cascade(out, q, kc, vc, pt, plen, stt, slt, scale, P, ws)

    def step():
        if fp8:
            pa.decode_cascade_append_fp8(out, q, key, val, kc, vc, slots, pt, plen, stt, slt,
                                         scale, f8.k_scale, f8.v_scale, P, ws)
        else:
            pa.decode_cascade_append(out, q, key, val, kc, vc, slots, pt, plen, stt, slt, scale,
                                     P, ws)
    for _ in range(warmup):
        reshape()
        decode()
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(iters)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        reshape()
        e[1].record(stream)
        decode()
        e[2].record(stream)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / iters
    dec_events = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    rc = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    # the roofline's duration: `iters` decode calls back to back between two events
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(iters):
        decode()
    d1.record(stream)
    torch.cuda.synchronize()
    dec = d0.elapsed_time(d1) / iters
    # the step as two calls (reshape_and_cache + decode) back to back
    d0.record(stream)
    for _ in range(iters):
        reshape()
        decode()
    d1.record(stream)
    torch.cuda.synchronize()
    step_two = d0.elapsed_time(d1) / iters
    # the step in one call back to back
    d0.record(stream)
    for _ in range(iters):
        step()
    d1.record(stream)
    torch.cuda.synchronize()
    step_gpu = d0.elapsed_time(d1) / iters
    eb = 1 if fp8 else 2  # bytes per cache element
    uniq, logical = w.unique_kv_bytes() * eb // 2, w.kv_bytes() * eb // 2
    line_cpu = None
    if cpu is not None:  # the oracle's decode over the full tables, whole workload
        import oracle
        orc = oracle.get()
        if fp8:
            okc, ovc = f8.k_cache.copy(), f8.v_cache.copy()
            orc.reshape_and_cache_fp8(w.key, w.value, okc, ovc, w.slot_mapping, f8.k_scale,
                                      f8.v_scale)

            def run():
                return orc.decode_fp8(w.q, okc, ovc, w.block_tables, w.context_lens, scale,
                                      f8.k_scale, f8.v_scale)
        else:
            okc, ovc = w.k_cache.copy(), w.v_cache.copy()
            orc.reshape_and_cache(w.key, w.value, okc, ovc, w.slot_mapping)

            def run():
                return orc.decode(w.q, okc, ovc, w.block_tables, w.context_lens, scale)
        dt, runs = _time_oracle(run, cpu.cpu_repeats, cpu.cpu_seconds)
        line_cpu = {"value": round(uniq / dt / 1e9, 4), "unit": "GB/s (unique K/V bytes)",
                    "cores": orc.threads_used, "kind": "oracle",
                    "sample": f"the whole workload ({w.num_seqs} seqs x {w.num_heads} heads over "
                              f"the full tables); fp64 oracle decode, median of {runs} runs = "
                              f"{dt:.3f} s wall on {orc.threads_used} threads; "
                              f"{w.num_seqs / dt:.1f} tokens/s/layer"}
    print(json.dumps({
        "op": "cascade", "workload": f"config3: {DESCRIPTIONS[3]}", "partition_size": P,
        "kv_dtype": "fp8-e4m3" if fp8 else "fp16",
        "t_decode_us_mean": round(dec * 1e3, 2),
        "t_decode_us_events_mean": round(dec_events * 1e3, 2),
        "t_reshape_us_mean": round(rc * 1e3, 2),
        "wall_ms_per_step": round(step_ms, 4), "ms_per_step": round(step_gpu, 6),
        "step": "pa_decode_cascade_append" + ("_fp8" if fp8 else ""),
        "ms_per_step_two_calls": round(step_two, 6),
        "decode_tokens_per_s_per_layer": round(w.num_seqs / (step_gpu * 1e-3), 1),
        "kv_bytes_logical": logical, "kv_bytes_unique": uniq,
        "roofline": {"bound": "hbm", "achieved": round(uniq / (dec * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(uniq / (dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "bytes": "unique K/V bytes",
                     "kernel": ("pa_decode_cascade_fp8" if fp8 else "pa_decode_cascade")
                               + " (prefix pass + partition kernel): HIP events around calls "
                               "back to back",
                     **_traffic_fields(("fp8_" if fp8 else "") + "cascade_config3_B16_P0")},
        "logical_kv_gbs": round(logical / (dec * 1e-3) / 1e9, 1),
        "cpu_baseline": line_cpu}), flush=True)


def bench_multi_query(iters, warmup, cpu=None, fp8=False):
    """A chunked-prefill batch: 16 sequences of 2048 positions whose last 512
    are this step's new tokens (32 heads x 128, B = 16); fp16 or FP8 caches
    (the matrix-core products are fp16 either way)."""
    import numpy as np
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import fp8_pools, make_multi_query
    S, ctx, n = 16, 2048, 512
    w, qh, qs = make_multi_query([ctx] * S, [n] * S, 32, 128, 16, seed=155, poison=False)

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    f8 = fp8_pools(w) if fp8 else None
    kc, vc = (up(f8.k_cache), up(f8.v_cache)) if fp8 else (up(w.k_cache), up(w.v_cache))
    q = up(qh)
    bt, cl, qst = up(w.block_tables), up(w.context_lens), up(qs)
    out = torch.empty_like(q)
    scale = float(w.scale)

    def call():
        if fp8:
            pa.multi_query_fp8(out, q, kc, vc, bt, cl, qst, n, scale, f8.k_scale, f8.v_scale)
        else:
            pa.multi_query(out, q, kc, vc, bt, cl, qst, n, scale)
    # at least 100 untimed calls (~35 ms): the matrix-core clock settles over the first ~20 ms
    ms = _time_events(call, iters, max(warmup, 100))
    t = float(np.median(ms)) * 1e-3
    H, D = w.num_heads, w.head_dim
    visible = sum(ctx - n + i + 1 for i in range(n)) * S          # (row, key) pairs per head
    flops = 4.0 * D * visible * H                                   # q.k and p.v
    kv_unique = S * ctx * H * D * 2 * (1 if fp8 else 2)
    line_cpu = None
    if cpu is not None:  # the oracle's prefill on the first 2 of the 16 sequences
        import oracle
        orc = oracle.get()
        ns = 2
        sq = qh[qs[0]:qs[ns]]
        if fp8:
            def run():
                return orc.prefill_fp8(sq, f8.k_cache, f8.v_cache, w.block_tables[:ns],
                                       w.context_lens[:ns], qs[:ns + 1], scale, f8.k_scale,
                                       f8.v_scale)
        else:
            def run():
                return orc.prefill(sq, w.k_cache, w.v_cache, w.block_tables[:ns],
                                   w.context_lens[:ns], qs[:ns + 1], scale)
        dt, runs = _time_oracle(run, cpu.cpu_repeats, cpu.cpu_seconds)
        sflops = flops * ns / S
        line_cpu = {"value": round(sflops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": orc.threads_used,
                    "kind": "oracle",
                    "sample": f"{ns} of {S} sequences ({ns * n} query rows x {H} heads); fp64 "
                              f"oracle {'FP8 ' if fp8 else ''}prefill, median of {runs} runs = "
                              f"{dt:.3f} s wall on "
                              f"{orc.threads_used} threads; {ns * n / dt:.1f} query rows/s"}
    print(json.dumps({
        "op": "multi_query", "workload": f"{S} seqs x {ctx} positions, last {n} new, 32 heads x 128",
        "kv_dtype": "fp8-e4m3" if fp8 else "fp16",
        "rows": S * n, "us_median": round(t * 1e6, 2),
        "query_tokens_per_s": round(S * n / t, 1),
        "roofline": {"bound": "mfma", "achieved": round(flops / t / 1e12, 2),
                     "peak": MFMA_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / t / 1e12 / MFMA_F16_TFLOPS, 4),
                     **_traffic_fields(("fp8_" if fp8 else "") + "multi_query_16x2048_last512")},
        "kv_unique_gbs": round(kv_unique / t / 1e9, 1), "cpu_baseline": line_cpu}), flush=True)


READ_PROBE = os.path.join(ROOT, "_build", "read_probe")
READ_PEAK = os.path.join(ROOT, "profiles", "read_peak.json")


def probe_read():
    if not os.path.exists(READ_PROBE):
        print(f"{READ_PROBE} is missing: run __graft_entry__.build() first", file=sys.stderr)
        return 1
    r = subprocess.run([READ_PROBE], capture_output=True, text=True, timeout=600)
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    return r.returncode


def _measured_peak():
    """Best streaming-read rate of read_probe.hip on this GPU type, as
    committed in profiles/read_peak.json (None if absent)."""
    try:
        return float(json.load(open(READ_PEAK))["best_read_gbs"])
    except (OSError, KeyError, ValueError):
        return None


def _device_info(torch):
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_oracle(fn, repeats, seconds):
    """Median wall time of fn() over at least `repeats` runs, repeated until
    `seconds` of wall time are spent (capped at 1000 runs)."""
    import numpy as np
    times = []
    while len(times) < max(1, repeats) or (sum(times) < seconds and len(times) < 1000):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times)


def cpu_baseline(w, sample_tokens, repeats, seconds, f8=None):
    """Time the oracle (as it stands) on a bounded, deterministic sample of
    (sequence, head) pairs of the same workload (the whole workload when it
    is under the cap); GB/s over the sampled K/V bytes, median of the runs
    (at least `repeats`, and more until `seconds` of wall time are spent)."""
    import numpy as np
    import oracle
    from paged_kv_cache_155_amd.workloads import kv_bytes_per_token
    orc = oracle.get()
    if f8 is None:
        kc, vc = w.k_cache.copy(), w.v_cache.copy()
        orc.reshape_and_cache(w.key, w.value, kc, vc, w.slot_mapping)

        def run(pairs):
            orc.decode_pairs(pairs, w.q, kc, vc, w.block_tables, w.context_lens, float(w.scale))
    else:  # the FP8 caches as the GPU holds them, the oracle's FP8 decode
        kc, vc = f8.k_cache.copy(), f8.v_cache.copy()
        orc.reshape_and_cache_fp8(w.key, w.value, kc, vc, w.slot_mapping, f8.k_scale, f8.v_scale)

        def run(pairs):
            orc.decode_fp8(w.q, kc, vc, w.block_tables, w.context_lens, float(w.scale),
                           f8.k_scale, f8.v_scale, pairs=pairs)
    S, H = w.num_seqs, w.num_heads
    pairs = [(s, h) for s in range(S) for h in range(H)]
    rng = np.random.default_rng(155)
    order = rng.permutation(len(pairs))
    chosen, tok = [], 0
    for i in order:
        if tok >= sample_tokens:
            break
        s, h = pairs[i]
        chosen.append((s, h))
        tok += int(w.context_lens[s])
    dt, runs = _time_oracle(lambda: run(chosen), repeats, seconds)
    threads = orc.threads_used
    # one core, on every 16th pair of the same sample
    one = chosen[::16]
    one_tok = sum(int(w.context_lens[s]) for s, _ in one)
    orc.set_threads(1)
    try:
        dt1, runs1 = _time_oracle(lambda: run(one), repeats, seconds / 4)
    finally:
        orc.set_threads(0)
    nbytes = tok * kv_bytes_per_token(1, w.head_dim) // (2 if f8 is not None else 1)
    one_bytes = one_tok * kv_bytes_per_token(1, w.head_dim) // (2 if f8 is not None else 1)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "value_1core": round(one_bytes / dt1 / 1e9, 4),
            "cpu": _cpu_model(),
            "sample": f"{len(chosen)} of {len(pairs)} (sequence, head) pairs (seeded permutation), "
                      f"{tok} token-heads = {nbytes} K/V bytes; fp64 oracle "
                      f"{'FP8 ' if f8 is not None else ''}decode, median of "
                      f"{runs} runs = {dt:.3f} s wall on {threads} threads; "
                      f"value_1core: every 16th of those pairs on 1 thread, median of {runs1} "
                      f"runs = {dt1:.3f} s; "
                      f"tokens/s/layer-equivalent {len(chosen) / H / dt:.1f}"}


def _decode_calls(w, fp8, P):
    """Upload one workload and return the step's two callables:
    write() = reshape_and_cache(_fp8) of the step's new tokens, attend() =
    decode(_fp8) over the paged K/V.  Inputs stay resident in HBM."""
    import numpy as np
    import torch
    import paged_kv_cache_155_amd as pa

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if fp8:
        from paged_kv_cache_155_amd.workloads import fp8_pools
        f8 = fp8_pools(w)
        kc, vc = up(f8.k_cache), up(f8.v_cache)
        ks, vs = float(f8.k_scale), float(f8.v_scale)
    else:
        f8 = None
        kc, vc = up(w.k_cache), up(w.v_cache)
    q = up(w.q)
    bt, cl = up(w.block_tables), up(w.context_lens)
    key, val, slots = up(w.key), up(w.value), up(w.slot_mapping)
    out = torch.empty_like(q)
    need = pa.decode_workspace_size(w.num_seqs, w.num_heads, w.head_dim, w.block_size,
                                    w.max_blocks_per_seq, P)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    scale = float(w.scale)

    def write():
        if fp8:
            pa.reshape_and_cache_fp8(key, val, kc, vc, slots, ks, vs)
        else:
            pa.reshape_and_cache(key, val, kc, vc, slots)

    def attend():
        if fp8:
            pa.decode_fp8(out, q, kc, vc, bt, cl, scale, ks, vs, partition_size=P, workspace=ws)
        else:
            pa.decode(out, q, kc, vc, bt, cl, scale, partition_size=P, workspace=ws)
    return write, attend, f8


def _cascade_calls(w, fp8):
    """Config 3 through the shared-prefix entry points: write() + attend() is
    reshape_and_cache + pa_decode_cascade; fused() is the same step as one
    pa_decode_cascade_append call."""
    import numpy as np
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import fp8_pools, split_shared_prefix
    prefix, plen, st, sl = split_shared_prefix(w, 512 // w.block_size)

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    f8 = fp8_pools(w) if fp8 else None
    kc, vc = (up(f8.k_cache), up(f8.v_cache)) if fp8 else (up(w.k_cache), up(w.v_cache))
    q = up(w.q)
    key, val, slots = up(w.key), up(w.value), up(w.slot_mapping)
    pt, stt, slt = up(prefix), up(st), up(sl)
    out = torch.empty_like(q)
    P = 0
    ws = torch.empty(pa.decode_cascade_workspace_size(w.num_seqs, w.num_heads, w.head_dim,
                                                      w.block_size, plen, st.shape[1], P),
                     dtype=torch.uint8, device="cuda")
    scale = float(w.scale)

    def write():
        if fp8:
            pa.reshape_and_cache_fp8(key, val, kc, vc, slots, f8.k_scale, f8.v_scale)
        else:
            pa.reshape_and_cache(key, val, kc, vc, slots)

    def attend():
        if fp8:
            pa.decode_cascade_fp8(out, q, kc, vc, pt, plen, stt, slt, scale, f8.k_scale,
                                  f8.v_scale, P, ws)
        else:
            pa.decode_cascade(out, q, kc, vc, pt, plen, stt, slt, scale, P, ws)

    def fused():
        if fp8:
            pa.decode_cascade_append_fp8(out, q, key, val, kc, vc, slots, pt, plen, stt, slt,
                                         scale, f8.k_scale, f8.v_scale, P, ws)
        else:
            pa.decode_cascade_append(out, q, key, val, kc, vc, slots, pt, plen, stt, slt, scale,
                                     P, ws)
    return write, attend, fused, f8


def _b2b_ms(fn, n):
    """Mean ms of n calls of fn back to back between two HIP events on the
    current stream (the one the library launches on)."""
    import torch
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def measure(write, attend, K, W, flush_iters, scratch, fused=None):
    """Timings of one workload's step (write + attend):
      t_step   K steps back to back (HIP events around the K steps);
      t_decode K attend() calls back to back;
      flushed  attend() after a 1 GiB write that evicts the L2s and the MALL,
               HIP events around each call (median, p10, p90);
      t_reshape mean of write() between events."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()

    def step():
        write()
        attend()
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_step = _b2b_ms(step, K)
    wall = time.perf_counter() - wall0
    t_dec = _b2b_ms(attend, K)
    t_fused = _b2b_ms(fused, K) if fused is not None else None
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for e in ev:
        e[0].record(stream)
        write()
        e[1].record(stream)
        attend()
        e[2].record(stream)
    torch.cuda.synchronize()
    t_rc = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    t_dec_events = [e[1].elapsed_time(e[2]) for e in ev]
    fl = []
    if flush_iters:
        fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(flush_iters)]
        for i, (a, b) in enumerate(fe):
            scratch.fill_(i & 0xFF)
            a.record(stream)
            attend()
            b.record(stream)
        torch.cuda.synchronize()
        fl = [a.elapsed_time(b) for a, b in fe]
    r = {"t_step_ms": t_step, "t_decode_ms": t_dec, "t_reshape_ms": t_rc,
         "t_decode_events_ms": t_dec_events, "t_decode_flushed_ms": fl, "wall_s": wall}
    if t_fused is not None:
        r["t_fused_step_ms"] = t_fused
    return r


SUITE = [  # (label, config, block size, call); partition size = the workload's own
    ("config2_B16", 2, 16, "decode"),  # headline: the largest single-GPU workload
    ("config0_B16", 0, None, "decode"),
    ("config1_B16", 1, None, "decode"),
    ("config2_B32", 2, 32, "decode"),
    ("config3_B16", 3, None, "decode"),
    ("config3_B16_cascade", 3, None, "cascade"),
    ("config4_B16", 4, None, "decode"),
]
TARGET_FRAC = 0.70  # of the 8 TB/s HBM peak, on configs 1-4


def _entry(label, cfg, w, call, fp8, r):
    """One per_config record: times in us, rates on the workload's bytes."""
    import numpy as np
    eb = 1 if fp8 else 2
    logical = w.kv_bytes() * eb // 2
    uniq = w.unique_kv_bytes() * eb // 2
    t_dec = r["t_decode_ms"] * 1e-3
    step = r.get("t_fused_step_ms", r["t_step_ms"]) * 1e-3
    fl = r["t_decode_flushed_ms"]
    e = {"label": label, "config": cfg, "call": ("pa_decode_cascade" if call == "cascade"
                                                 else "pa_decode") + ("_fp8" if fp8 else ""),
         "block_size": w.block_size, "partition_size": 0 if call == "cascade" else w.partition_size,
         "num_seqs": w.num_seqs, "num_heads": w.num_heads, "head_dim": w.head_dim,
         "kv_bytes_logical": logical, "kv_bytes_unique": uniq,
         "t_decode_us": round(t_dec * 1e6, 2),
         "t_decode_us_events_median": round(float(np.median(r["t_decode_events_ms"])) * 1e3, 2),
         "t_reshape_us": round(r["t_reshape_ms"] * 1e3, 2),
         "t_step_us": round(step * 1e6, 2),
         "step": ("pa_decode_cascade_append" + ("_fp8" if fp8 else "")) if call == "cascade"
                 else "reshape_and_cache + pa_decode" + (" (fp8)" if fp8 else ""),
         "decode_tokens_per_s_per_layer": round(w.num_seqs / step, 1),
         "kv_gbs_unique": round(uniq / t_dec / 1e9, 1),
         "frac": round(uniq / t_dec / 1e9 / HBM_PEAK_GBS, 4)}
    if "t_fused_step_ms" in r:
        e["t_step_two_calls_us"] = round(r["t_step_ms"] * 1e3, 2)
    if uniq != logical:
        e["kv_gbs_logical"] = round(logical / t_dec / 1e9, 1)
    if fl:
        tf = float(np.median(fl)) * 1e-3
        e["flushed"] = {"t_decode_us_median": round(tf * 1e6, 2),
                        "t_decode_us_p10_p90": [round(float(np.percentile(fl, 10)) * 1e3, 2),
                                                round(float(np.percentile(fl, 90)) * 1e3, 2)],
                        "frac": round(uniq / tf / 1e9 / HBM_PEAK_GBS, 4)}
    if cfg != 0:
        e["meets_target"] = bool(e["frac"] >= TARGET_FRAC)
    e.update(_traffic_fields(("fp8_" if fp8 else "")
                             + (f"cascade_config3_B16_P0" if call == "cascade"
                                else f"config{cfg}_B{w.block_size}_P{w.partition_size}")))
    return e


def _workload_bytes(key):
    """(algorithmic K/V bytes, unique K/V bytes) of the workload a traffic key
    names (config{c}_B{b}_P{p}, cascade_config3_B16_P0,
    multi_query_16x2048_last512; fp8_ prefix: one byte per element)."""
    from paged_kv_cache_155_amd.workloads import make_workload
    fp8 = key.startswith("fp8_")
    k = key[4:] if fp8 else key
    eb = 1 if fp8 else 2
    if k.startswith("multi_query_16x2048"):
        n = 16 * 2048 * 32 * 128 * 2 * eb
        return n, n
    if k.startswith("cascade_config3"):
        w = make_workload(3, poison=False)
    else:
        cfg = int(k[len("config"):].split("_")[0])
        bsz = int(k.split("_B")[1].split("_")[0])
        w = make_workload(cfg, block_size=bsz, poison=False)
    return w.kv_bytes() * eb // 2, w.unique_kv_bytes() * eb // 2


def ingest_traffic(key, fetch_csv, write_csv):
    """profiles/traffic.json[key] from rocprofv3 --pmc FETCH_SIZE and
    WRITE_SIZE csvs of one workload: the median per dispatch of each library
    kernel (the step's reshape_and_cache excluded), summed over the kernels
    of one call and scaled to bytes by the calibration entry."""
    import csv
    import statistics
    from collections import defaultdict
    tj = json.load(open(TRAFFIC_JSON))
    cal = tj["_calibration"]

    def per_kernel(path, counter):
        vals = defaultdict(list)
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if r["Counter_Name"] != counter or "pa::" not in name or "reshape_and_cache" in name:
                continue
            name = name.replace("void ", "").replace("pa::(anonymous namespace)::", "")
            vals[name.split("(pa::")[0]].append(float(r["Counter_Value"]))
        return {k: statistics.median(v) for k, v in vals.items()}
    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    rd = sum(f.values()) * 1024 * cal["fetch_scale"]
    wr = sum(w.values()) * 1024 * cal["write_scale"]
    alg, uniq = _workload_bytes(key)
    tj[key] = {"kernel_code_sha": kernel_code_sha(), "bytes_per_launch": int(round(rd + wr)),
               "read_bytes": int(round(rd)), "write_bytes": int(round(wr)),
               "read_over_unique": round(rd / uniq, 4),
               "fetch_size_kib": f, "write_size_kib": w,
               "algorithmic_kv_bytes": alg, "unique_kv_bytes": uniq}
    json.dump(tj, open(TRAFFIC_JSON, "w"), indent=1)
    print(json.dumps({key: tj[key]}))


def main():
    a = _args()
    if a.ingest_traffic:
        ingest_traffic(*a.ingest_traffic)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}): "
              "this library is a single-GPU kernel; sharding is described, not built.",
              file=sys.stderr)
        sys.exit(2)
    if a.probe == "read":  # a child process of its own; nothing here touches the GPU
        sys.exit(probe_read())
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import DESCRIPTIONS, make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pa.load()
    if a.probe == "copy":
        probe_copy(a.probe_mib)
        return
    if a.op == "cascade":
        bench_cascade(a.steps, a.warmup, None if a.no_cpu_baseline else a,
                      fp8=a.kv_dtype == "fp8")
        return
    if a.op == "multi_query":
        bench_multi_query(a.steps, a.warmup, None if a.no_cpu_baseline else a,
                          fp8=a.kv_dtype == "fp8")
        return
    if a.op != "step":
        bench_blocks(a.op, a.pairs, a.steps, None if a.no_cpu_baseline else a)
        return

    fp8 = a.kv_dtype == "fp8"
    K, W = a.steps, a.warmup
    flush_iters = 0 if a.no_flush else max(K, 10)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if flush_iters else None
    if a.config is None:  # the suite: config 2 (B 16) headline + every config
        suite = SUITE
    else:
        bs = a.block_size
        suite = [(f"config{a.config}_B{bs or 'd'}" + ("_cascade" if a.call == "cascade" else ""),
                  a.config, bs, a.call)]
    entries, head = [], None
    for label, cfg, bs, call in suite:
        w = make_workload(cfg, block_size=bs, poison=False,
                          partition_size=a.partition_size if a.config is not None else None)
        print(f"[bench] {label}: S={w.num_seqs} H={w.num_heads} D={w.head_dim} "
              f"B={w.block_size} P={w.partition_size} call={call}", file=sys.stderr, flush=True)
        if call == "cascade":
            write, attend, fused, f8 = _cascade_calls(w, fp8)
            r = measure(write, attend, K, W, flush_iters, scratch,
                        fused=fused if a.config is None else None)
        else:
            write, attend, f8 = _decode_calls(w, fp8, w.partition_size)
            r = measure(write, attend, K, W, flush_iters, scratch)
        e = _entry(label, cfg, w, call, fp8, r)
        entries.append(e)
        if head is None:
            head = (w, f8, r, e, cfg)
        else:
            del w
        del write, attend, f8
        torch.cuda.empty_cache()

    w, f8, r, e, cfg = head
    ms_step = r["t_step_ms"]
    t_dec = r["t_decode_ms"]
    kvb = e["kv_bytes_logical"]
    uniq = e["kv_bytes_unique"]
    achieved = uniq / (t_dec * 1e-3) / 1e9
    value = kvb / (ms_step * 1e-3) / 1e9
    mp = _measured_peak()
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3" if fp8 else "f16",
        "data": "synthetic",
        "config": {
            "workload": f"config{cfg}: {DESCRIPTIONS[cfg]}",
            "num_seqs": w.num_seqs, "num_heads": w.num_heads, "head_dim": w.head_dim,
            "block_size": w.block_size, "partition_size": w.partition_size,
            "num_blocks": w.num_blocks, "kv_dtype": a.kv_dtype, "kv_bytes_per_step": kvb,
            "unique_kv_bytes": uniq,
            "decode_tokens_per_s_per_layer": round(w.num_seqs / (ms_step * 1e-3), 1),
            "decode_only_tokens_per_s_per_layer": round(w.num_seqs / (t_dec * 1e-3), 1),
            "t_decode_us_mean": round(t_dec * 1e3, 2),
            "t_reshape_us_mean": round(r["t_reshape_ms"] * 1e3, 2),
            "wall_s_timed": round(r["wall_s"], 4), "accumulate": "f32",
            "timing": "value and ms_per_step: K steps (reshape_and_cache + decode) back to back "
                      "between two HIP events; roofline: K decode calls back to back",
            "device": _device_info(torch),
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes": "unique K/V bytes",
                     "measured_peak": mp,
                     "frac_of_measured": round(achieved / mp, 4) if mp else None,
                     "traffic": e["traffic"], "traffic_source": e["traffic_source"],
                     "kernel": e["call"] + (" (shared-prefix pass + partition kernel)"
                                            if "cascade" in e["call"]
                                            else " (partition kernel + reduce kernel)")
                               + ": HIP events around K calls back to back"},
        "per_config": entries,
        "cpu_baseline": None,
    }
    if "flushed" in e:
        line["roofline"]["flushed"] = e["flushed"]
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_sample_tokens, a.cpu_repeats, a.cpu_seconds,
                                            f8 if fp8 else None)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
