"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

Headline workload (one "step"): a decode step of a Qwen2.5-1.5B-shaped attention
stack. Batch 8, 12 query / 2 KV heads, head_dim 128, bf16 KV, 16-token blocks; each of
the model's 28 layers has its own pool of 4096 blocks, and per layer the step stores
the 8 new tokens through slot_mapping and then attends them plus the cached prefix
(pa_decode_step, one launch per layer; the same step as pa_store_kv + pa_decode is
timed beside it). Contexts are seeded U{128..3200} after the store. The 28
layer steps are captured once in a HIP graph and replayed, so the timed region holds
only GPU work; inputs are resident in HBM. Using 28 distinct pools (~380 MB of KV
touched per step) keeps the decode reads from being served by the 256 MB MALL.

Prints one JSON line: value = algorithmic KV + query/output bytes moved per step /
step time (GB/s), with seqs/s, the decode kernel's roofline (HIP-event timed average
launch over a graph of decode launches only), the CPU oracle's rate on a bounded sample
and, unless --no-extra, the same figures for the 256-sequence decode, the FP8 and INT8
decodes and the varlen prefill.
"""
import argparse
import json
import math
import os
import resource
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV GB/s (% of HBM peak) + decode seqs/sec per step"
# HBM bytes per launch of the headline decode kernel, read with rocprofv3 FETCH_SIZE /
# WRITE_SIZE (calibrated against a copy) and recorded in this profile summary together
# with a hash of the decode sources they were taken with.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_qwen_28layer.md")
DECODE_SOURCES = ["paged_kv_cache_95_amd/csrc/decode.hip", "paged_kv_cache_95_amd/csrc/common.h",
                  "paged_kv_cache_95_amd/csrc/internal.h"]
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
LAYERS = 28


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- bytes

def decode_bytes(lens, hq, hkv, d, e_kv, e_q=2, fp8_scales=False):
    """Algorithmic bytes of one decode call: each context token's K and V row of every
    KV head once, plus (FP8) their two fp32 scales, q and out once, the used block ids."""
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(lens.sum()) * hkv * d * 2 * e_kv
    sc = int(lens.sum()) * hkv * 2 * 4 if fp8_scales else 0
    qo = len(lens) * hq * d * e_q * 2
    ids = int(sum(-(-int(L) // 16) for L in lens)) * 4 + 4 * len(lens)
    return kv + sc + qo + ids


def store_bytes(T, hkv, d, e_src, e_pool, fp8_scales=False):
    return T * hkv * d * 2 * (e_src + e_pool) + 8 * T + (T * hkv * 2 * 4 if fp8_scales else 0)


def prefill_flops(n, P, hq, d):
    """Causal pairs only: row i of a chunk on prefix P sees P + i + 1 keys; 2 matmuls."""
    pairs = sum(int(ni) * int(pi) + int(ni) * (int(ni) + 1) // 2 for ni, pi in zip(n, P))
    return 4 * d * hq * pairs


def decode_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """Counter-measured HBM bytes per launch of the headline decode kernel, or None when
    the profile is missing or was taken with other decode sources."""
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch=(\d+) decode_sources_sha256=([0-9a-f]{64})", text)
    if not m or m.group(2) != decode_sources_sha256():
        return None
    return int(m.group(1))


# ----------------------------------------------------------------------------- timing

def time_graph(torch, graph, reps):
    """Average ms per replay measured with HIP events on the replay stream."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        graph.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    fn()                                   # eager run first (allocations, warm caches)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# ----------------------------------------------------------------------------- workloads

def qwen_layers(torch, pa, W, dev, split_tokens):
    case = W.make(2)
    B, hq, hkv, D = case.num_seqs, case.Hq, case.Hkv, case.D
    bt = torch.from_numpy(case.block_tables).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    maxctx = int(case.block_tables.shape[1] * 16)          # 3200: the table's capacity
    layers = []
    for l in range(LAYERS):
        pool = pa.KVPool.empty(case.num_blocks, hkv, D, "bf16", dev)
        W.fill_device_normal_(pool.k, 20000 + 2 * l)
        W.fill_device_normal_(pool.v, 20001 + 2 * l)
        q = W.fill_device_normal_(torch.empty((B, hq, D), dtype=torch.bfloat16, device=dev),
                                  30000 + l)
        kn = W.fill_device_normal_(torch.empty((B, hkv, D), dtype=torch.bfloat16, device=dev),
                                   40000 + l)
        vn = W.fill_device_normal_(torch.empty((B, hkv, D), dtype=torch.bfloat16, device=dev),
                                   50000 + l)
        out = torch.empty((B, hq, D), dtype=torch.bfloat16, device=dev)
        layers.append((pool, q, kn, vn, out))
    ws = pa.decode_workspace(B, hq, hkv, D, maxctx, split_tokens, device=dev)

    def store_all():
        for pool, q, kn, vn, out in layers:
            pa.store_kv(pool, kn, vn, slots)

    def decode_all():
        for pool, q, kn, vn, out in layers:
            pa.decode(q, pool, bt, ctx, case.scale, max_context_len=maxctx,
                      split_tokens=split_tokens, out=out, workspace=ws)

    def step():
        # the library's decode step: store the new rows and attend, one call per layer
        for pool, q, kn, vn, out in layers:
            pa.decode_step(q, pool, kn, vn, slots, bt, ctx, case.scale, max_context_len=maxctx,
                           split_tokens=split_tokens, out=out, workspace=ws)

    def step_two_calls():
        for pool, q, kn, vn, out in layers:
            pa.store_kv(pool, kn, vn, slots)
            pa.decode(q, pool, bt, ctx, case.scale, max_context_len=maxctx,
                      split_tokens=split_tokens, out=out, workspace=ws)

    return case, step, step_two_calls, decode_all, store_all


def cpu_baseline(case, budget_s=12.0):
    """The oracle (store + decode of one layer of the headline workload, 8 sequences)
    timed on the host, repeated until about budget_s of work; cores = process CPU time
    / wall time over the run (what the oracle actually used)."""
    import workloads as W
    from oracle import ref
    kp = W.host_pool(case, "k", poison_unused=False).astype(np.float64)
    vp = W.host_pool(case, "v", poison_unused=False).astype(np.float64)
    reps = 0
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    while True:
        k2 = ref.store_ref(kp, case.k_new.astype(np.float64), case.slot_mapping)
        v2 = ref.store_ref(vp, case.v_new.astype(np.float64), case.slot_mapping)
        ref.decode_ref(case.q, k2, v2, case.block_tables, case.context_lens, case.scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    per = el / reps
    by = decode_bytes(case.context_lens, case.Hq, case.Hkv, case.D, 2) + \
        store_bytes(case.num_seqs, case.Hkv, case.D, 2, 2)
    return {"value": round(by / per / 1e9, 4), "unit": "GB/s", "cores": round(cpu / el, 2),
            "kind": "oracle", "seconds_per_layer_step": round(per, 4),
            "seqs_per_s": round(case.num_seqs / per, 2),
            "sample": f"store + decode of one layer of the headline workload (8 sequences, "
                      f"{int(case.context_lens.sum())} context tokens), repeated {reps}x "
                      f"({el:.1f} s); fp64 numpy oracle, host cores of the GPU box "
                      f"(affinity {len(os.sched_getaffinity(0))})"}


def extra_large_decode(torch, pa, W, dev, reps=20, split_tokens=0):
    case = W.make(4)
    pool = pa.KVPool.empty(case.num_blocks, case.Hkv, case.D, "bf16", dev)
    W.fill_device_normal_(pool.k, 41)
    W.fill_device_normal_(pool.v, 42)
    bt = torch.from_numpy(case.block_tables).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    q = torch.from_numpy(case.q).to(torch.bfloat16).to(dev)
    kn = torch.from_numpy(case.k_new).to(torch.bfloat16).to(dev)
    vn = torch.from_numpy(case.v_new).to(torch.bfloat16).to(dev)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    out = torch.empty_like(q)
    maxctx = case.max_context_len
    ws = pa.decode_workspace(case.num_seqs, case.Hq, case.Hkv, case.D, maxctx, split_tokens,
                             device=dev)
    g = capture(torch, lambda: pa.decode(q, pool, bt, ctx, case.scale, max_context_len=maxctx,
                                         split_tokens=split_tokens, out=out, workspace=ws))
    gs = capture(torch, lambda: pa.store_kv(pool, kn, vn, slots))
    for _ in range(3):
        g.replay()
    ms = time_graph(torch, g, reps)
    ms_store = time_graph(torch, gs, reps)
    by = decode_bytes(case.context_lens, case.Hq, case.Hkv, case.D, 2)
    del pool
    return {"workload": "256-sequence decode, 32/8 heads, D 128, bf16, contexts log-uniform "
                        "1K-32K (9.6 GB of KV per call, larger than the MALL)",
            "decode_ms": round(ms, 4), "store_ms": round(ms_store, 4),
            "kv_bytes": by, "gbs": round(by / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * by / ms / 1e6 / HBM_PEAK_GBS, 1),
            "seqs_per_s": round(case.num_seqs / ((ms + ms_store) / 1e3), 1)}


def extra_fp8_decode(torch, pa, W, dev, reps=30, copies=2, split_tokens=0, dtype="fp8"):
    """Two copies of the 64 x 8192 FP8 (or INT8) multi-slot pool (277 MB each) alternate,
    so a call does not find its pool in the MALL left by the previous one."""
    case = W.make(5)
    ctx_len = case.extra["ctx"]
    B, hkv, D = case.num_seqs, case.Hkv, case.D
    pos = np.arange(ctx_len - 1)
    slots_prefix = torch.from_numpy(np.concatenate(
        [case.block_tables[s, pos // 16].astype(np.int64) * 16 + pos % 16 for s in range(B)])).to(dev)
    src = torch.empty((B * (ctx_len - 1), hkv, D), dtype=torch.bfloat16, device=dev)
    pools = []
    for c in range(copies):
        pool = pa.KVPool.empty(case.num_blocks, hkv, D, dtype, dev)
        W.fill_device_normal_(src, case.seed * 1000 + 1 + 10 * c)
        srcv = src.clone()
        W.fill_device_normal_(srcv, case.seed * 1000 + 2 + 10 * c)
        pa.store_kv(pool, src, srcv, slots_prefix)
        pools.append(pool)
    del src, srcv
    bt = torch.from_numpy(case.block_tables).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    q = torch.from_numpy(case.q).to(torch.bfloat16).to(dev)
    kn = torch.from_numpy(case.k_new).to(torch.bfloat16).to(dev)
    vn = torch.from_numpy(case.v_new).to(torch.bfloat16).to(dev)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    out = torch.empty_like(q)
    ws = pa.decode_workspace(B, case.Hq, hkv, D, ctx_len, split_tokens, device=dev)

    def dec():
        for p in pools:
            pa.decode(q, p, bt, ctx, case.scale, max_context_len=ctx_len,
                      split_tokens=split_tokens, out=out, workspace=ws)

    def sto():
        for p in pools:
            pa.store_kv(p, kn, vn, slots)

    g, gs = capture(torch, dec), capture(torch, sto)
    ms = time_graph(torch, g, reps) / copies
    ms_store = time_graph(torch, gs, reps) / copies
    by = decode_bytes(case.context_lens, case.Hq, hkv, D, 1, fp8_scales=True)
    name = "FP8 e4m3" if dtype == "fp8" else "INT8"
    return {"workload": f"64 x 8192 {name} decode, 12/2 heads, D 128, per-token-head fp32 "
                        "scales, multi-slot layout viewed as 16-token blocks",
            "decode_ms": round(ms, 4), "store_ms": round(ms_store, 4), "kv_bytes": by,
            "gbs": round(by / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * by / ms / 1e6 / HBM_PEAK_GBS, 1),
            "seqs_per_s": round(B / ((ms + ms_store) / 1e3), 1)}


def extra_prefill(torch, pa, W, dev, reps=30, split_tokens=0):
    case = W.make(3)
    pool = pa.KVPool.empty(case.num_blocks, case.Hkv, case.D, "bf16", dev)
    W.fill_device_normal_(pool.k, 31)
    W.fill_device_normal_(pool.v, 32)
    bf = torch.bfloat16
    q = torch.from_numpy(case.q).to(bf).to(dev)
    kn = torch.from_numpy(case.k_new).to(bf).to(dev)
    vn = torch.from_numpy(case.v_new).to(bf).to(dev)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    cu = torch.from_numpy(case.cu_seqlens).to(dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    out = torch.empty_like(q)
    ws = pa.varlen_prefill_workspace(q.shape[0], case.Hq, case.D, case.max_context_len,
                                     split_tokens, device=dev)

    def run():
        pa.varlen_prefill(q, cu, pool, bt, ctx, case.scale, max_q_len=case.max_q_len,
                          max_context_len=case.max_context_len, split_tokens=split_tokens,
                          out=out, workspace=ws)

    g = capture(torch, run)
    gs = capture(torch, lambda: pa.store_kv(pool, kn, vn, slots))
    ms = time_graph(torch, g, reps)
    ms_store = time_graph(torch, gs, reps)
    fl = prefill_flops(case.extra["n"], case.extra["P"], case.Hq, case.D)
    tf = fl / ms / 1e9
    return {"workload": "varlen mixed step: 16 chunks of 1-512 new tokens (4 of length 1) on "
                        "cached prefixes of 0-2048, 12/2 heads, D 128, bf16",
            "prefill_ms": round(ms, 4), "store_ms": round(ms_store, 4),
            "tokens": int(case.cu_seqlens[-1]), "causal_gflop": round(fl / 1e9, 2),
            "tflops": round(tf, 1), "mfma_util_pct": round(100 * tf / BF16_MFMA_PEAK_TFLOPS, 2)}


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards by "
              "sequence or KV head with no exchange, so run one process per GPU instead.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_95_amd as pa
    import workloads as W
    pa.lib()
    dev = torch.device("cuda:0")

    log("setup: 28 layer pools of the qwen-shaped decode")
    case, step, step_two_calls, decode_all, store_all = qwen_layers(torch, pa, W, dev,
                                                                    args.split_tokens)
    g_step = capture(torch, step)
    g_two = capture(torch, step_two_calls)
    g_dec = capture(torch, decode_all)
    g_sto = capture(torch, store_all)
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    ms_events = time_graph(torch, g_step, args.steps)
    wall = time.perf_counter() - t0
    ms_step = ms_events
    # the same step as separate store and decode calls, and each of them alone
    two_ms = time_graph(torch, g_two, max(args.steps, 10))
    dec_ms = time_graph(torch, g_dec, max(args.steps, 10)) / LAYERS
    sto_ms = time_graph(torch, g_sto, max(args.steps, 10)) / LAYERS
    launch_ms = ms_step / LAYERS     # the step is one launch per layer

    B, hq, hkv, D = case.num_seqs, case.Hq, case.Hkv, case.D
    dby = decode_bytes(case.context_lens, hq, hkv, D, 2)
    sby = store_bytes(B, hkv, D, 2, 2)
    step_bytes = LAYERS * (dby + sby)
    gbs = step_bytes / ms_step / 1e6
    # a one-off 256 MiB device copy: its HBM counter readings calibrate FETCH/WRITE_SIZE
    a = torch.empty(1 << 27, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b

    res = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen2.5-1.5b-shaped paged decode step: 28 layers x "
                               "(store 8 new tokens + decode), one 4096-block pool per layer",
                   "batch": B, "q_heads": hq, "kv_heads": hkv, "head_dim": D, "block_size": 16,
                   "pool_blocks": case.num_blocks, "layers": LAYERS,
                   "context_lens": case.context_lens.tolist(),
                   "split_tokens": args.split_tokens or pa.default_split_tokens(B, hkv, 3200),
                   "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(B / (ms_step / 1e3), 1),
        "wall_s_timed_region": round(wall, 4),
        "per_layer": {"step_ms": round(launch_ms, 5), "two_call_step_ms": round(two_ms / LAYERS, 5),
                      "decode_ms": round(dec_ms, 5), "store_ms": round(sto_ms, 5),
                      "decode_bytes": dby, "store_bytes": sby},
        "two_call_step": {"ms_per_step": round(two_ms, 5),
                          "value": round(step_bytes / two_ms / 1e6, 2),
                          "note": "same step as pa_store_kv + pa_decode per layer"},
        "roofline": {"kernel": "decode_fused_kernel<bf16, D128, G6> (decode step, store folded in)",
                     "bound": "hbm",
                     "achieved": round((dby + sby) / launch_ms / 1e6, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s",
                     "frac": round((dby + sby) / launch_ms / 1e6 / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(),
                     "per_launch_bytes": dby + sby, "per_launch_us": round(launch_ms * 1e3, 2),
                     "note": "achieved = algorithmic bytes of one step launch (decode + store) / "
                             "its average duration (HIP events around the timed graph of 28 "
                             "one-launch layer steps); traffic = HBM bytes per launch from "
                             "rocprofv3 FETCH_SIZE x2 + WRITE_SIZE (copy-calibrated), null if "
                             "the decode sources changed since"},
    }
    if not args.no_extra:
        log("extra: large decode")
        res["extra"] = {"large_decode": extra_large_decode(torch, pa, W, dev)}
        torch.cuda.empty_cache()
        log("extra: fp8 decode")
        res["extra"]["fp8_decode"] = extra_fp8_decode(torch, pa, W, dev)
        torch.cuda.empty_cache()
        log("extra: int8 decode")
        res["extra"]["int8_decode"] = extra_fp8_decode(torch, pa, W, dev, dtype="int8")
        torch.cuda.empty_cache()
        log("extra: varlen prefill")
        res["extra"]["varlen_prefill"] = extra_prefill(torch, pa, W, dev)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
