"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
                    [--only NAME]

Headline workload (one "step"): the large decode batch. 256 sequences, 32 query / 8 KV
heads, head_dim 128, bf16 KV in 16-token blocks, contexts log-uniform in [1024, 32768]
(seeded; 2.69M context tokens, 11.0 GB of KV, far more than the 256 MB MALL). A step
stores each sequence's new K/V row through slot_mapping and then attends the whole
context (pa_decode_step: a store launch, the persistent split-K decode kernel and the
log-sum-exp merge). The step is captured once in a HIP graph and replayed, so the
timed region holds GPU work only; every input is resident in HBM before it starts.

Prints one JSON line: value = algorithmic bytes of the step (KV read once, q and out,
block ids, the stored rows) / step time, in GB/s; seqs/s; the decode kernel's roofline
(HIP events around a graph of decode calls); the CPU oracle's rate on a bounded sample
of the same workload; and, unless --no-extra, the same figures (each with its own
roofline) for the Qwen2.5-1.5B-shaped 28-layer decode step, the FP8 and INT8 64 x 8192
decodes, the varlen prefill step and a plain device copy (achievable bandwidth).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV GB/s (% of HBM peak) + decode seqs/sec per step"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, datasheet
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, datasheet
LAYERS = 28                      # Qwen2.5-1.5B's layer count (public model config)
PROFILES = os.path.join(ROOT, "profiles")
# sources whose text decides a recorded kernel's traffic (api.cpp: split policy and
# workspace layout)
DECODE_SOURCES = ["paged_kv_cache_95_amd/csrc/decode.hip", "paged_kv_cache_95_amd/csrc/common.h",
                  "paged_kv_cache_95_amd/csrc/internal.h", "paged_kv_cache_95_amd/csrc/api.cpp"]
PREFILL_SOURCES = ["paged_kv_cache_95_amd/csrc/prefill.hip",
                   "paged_kv_cache_95_amd/csrc/common.h", "paged_kv_cache_95_amd/csrc/internal.h",
                   "paged_kv_cache_95_amd/csrc/api.cpp"]
WORKLOADS = ("large_decode", "qwen_step", "fp8_decode", "int8_decode", "varlen_prefill", "copy")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- bytes

def decode_bytes(lens, hq, hkv, d, e_kv, e_q=2, scales=False):
    """Algorithmic bytes of one decode call: each context token's K and V row of every
    KV head once, plus (FP8 / INT8) their two fp32 scales, q and out once, the used
    block ids and the context lengths."""
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(lens.sum()) * hkv * d * 2 * e_kv
    sc = int(lens.sum()) * hkv * 2 * 4 if scales else 0
    qo = len(lens) * hq * d * e_q * 2
    ids = int(sum(-(-int(L) // 16) for L in lens)) * 4 + 4 * len(lens)
    return kv + sc + qo + ids


def store_bytes(T, hkv, d, e_src, e_pool, scales=False):
    """Algorithmic bytes of storing T new tokens: source rows read, pool rows written,
    the int64 slots, and (FP8 / INT8) the two fp32 scales per row."""
    return T * hkv * d * 2 * (e_src + e_pool) + 8 * T + (T * hkv * 2 * 4 if scales else 0)


def prefill_flops(n, P, hq, d):
    """Causal pairs only: row i of a chunk on prefix P sees P + i + 1 keys; 2 products."""
    pairs = sum(int(ni) * int(pi) + int(ni) * (int(ni) + 1) // 2 for ni, pi in zip(n, P))
    return 4 * d * hq * pairs


# ----------------------------------------------------------------------------- recorded counters

def sources_sha256(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded(profile, kernel, sources):
    """key=value figures a profile summary records for `kernel` on a line
    `record: kernel=<kernel> ... sources_sha256=<hash>`, or {} when the summary is missing
    or was taken with other kernel sources (counters of an older kernel do not count)."""
    try:
        text = open(os.path.join(PROFILES, profile)).read()
    except OSError:
        return {}
    for line in text.splitlines():
        if not line.startswith("record: ") or f" kernel={kernel} " not in line + " ":
            continue
        kv = dict(re.findall(r"(\w+)=(\S+)", line))
        if kv.get("sources_sha256") != sources_sha256(sources):
            return {}
        return kv
    return {}


def roofline(kernel, bound, alg, launch_ms, peak, unit, rec, note):
    """The roofline block for one kernel: achieved = algorithmic work per launch /
    average launch duration (HIP events), traffic = counter-measured HBM bytes per launch
    recorded in the kernel's profile summary (null when none matches the sources)."""
    per_s = alg / (launch_ms / 1e3)
    achieved = per_s / (1e9 if unit == "GB/s" else 1e12)
    traffic = int(rec["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in rec else None
    out = {"kernel": kernel, "bound": bound, "achieved": round(achieved, 1), "peak": peak,
           "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
           "per_launch_work": alg, "per_launch_us": round(launch_ms * 1e3, 2), "note": note}
    if traffic is not None:
        out["traffic_over_algorithmic"] = round(traffic / alg, 4) if unit == "GB/s" else None
    return out


# ----------------------------------------------------------------------------- timing

def time_graph(torch, graph, reps):
    """Average ms per replay, HIP events recorded on the stream the replays run on."""
    stream = torch.cuda.current_stream()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record(stream)
    for _ in range(reps):
        graph.replay()
    e.record(stream)
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


SETTLE_S = 0.25


def settle(torch, graph, seconds=None):
    """Replay until `seconds` of GPU work have run, so that the timed replays see the
    GPU's steady clocks rather than its ramp from idle (short timed windows right after
    setup read several percent slow otherwise)."""
    seconds = SETTLE_S if seconds is None else seconds
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            graph.replay()
        torch.cuda.synchronize()


# ----------------------------------------------------------------------------- headline

def large_decode(torch, pa, W, dev, steps, warmup):
    """The 256-sequence decode step (store + decode), and the decode call alone."""
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
    ws = pa.decode_workspace(case.num_seqs, case.Hq, case.Hkv, case.D, maxctx, device=dev)

    def step():
        pa.decode_step(q, pool, kn, vn, slots, bt, ctx, case.scale, max_context_len=maxctx,
                       out=out, workspace=ws)

    def dec():
        pa.decode(q, pool, bt, ctx, case.scale, max_context_len=maxctx, out=out, workspace=ws)

    g_step, g_dec = capture(torch, step), capture(torch, dec)
    settle(torch, g_step)
    for _ in range(warmup):
        g_step.replay()
    torch.cuda.synchronize()
    log(f"timing {steps} steps of the 256-sequence decode")
    t0 = time.perf_counter()
    ms = time_graph(torch, g_step, steps)
    wall = time.perf_counter() - t0
    dec_ms = time_graph(torch, g_dec, max(steps, 5))
    dby = decode_bytes(case.context_lens, case.Hq, case.Hkv, case.D, 2)
    sby = store_bytes(case.num_seqs, case.Hkv, case.D, 2, 2)
    kern = "decode_compact_kernel<bf16, 128, 4, bf16>"
    rec = recorded("decode_large_256seq.md", kern.replace(" ", ""), DECODE_SOURCES)
    res = {"case": case, "ms_step": ms, "wall": wall, "decode_ms": dec_ms,
           "decode_bytes": dby, "store_bytes": sby,
           "roofline": roofline(
               kern, "hbm", dby, dec_ms, HBM_PEAK_GBS, "GB/s", rec,
               "achieved = algorithmic decode bytes / the decode call's average time (HIP "
               "events over a graph of decode calls; the call is this persistent split "
               "kernel plus the small log-sum-exp merge launch, ~1% of the call); traffic "
               "= rocprofv3 FETCH_SIZE + WRITE_SIZE of this kernel per launch, scaled by a "
               "device copy's readings")}
    del pool
    return res


# ----------------------------------------------------------------------------- extras

def qwen_step(torch, pa, W, dev, reps):
    """Qwen2.5-1.5B-shaped decode step: 28 layers, each with its own 4096-block pool
    (~380 MB of KV touched per step, more than the MALL), one pa_decode_step per layer."""
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
        mk = lambda shape, seed: W.fill_device_normal_(
            torch.empty(shape, dtype=torch.bfloat16, device=dev), seed)
        layers.append((pool, mk((B, hq, D), 30000 + l), mk((B, hkv, D), 40000 + l),
                       mk((B, hkv, D), 50000 + l), torch.empty((B, hq, D), dtype=torch.bfloat16,
                                                               device=dev)))
    ws = pa.decode_workspace(B, hq, hkv, D, maxctx, device=dev)

    def step():
        for pool, q, kn, vn, out in layers:
            pa.decode_step(q, pool, kn, vn, slots, bt, ctx, case.scale, max_context_len=maxctx,
                           out=out, workspace=ws)

    def two_calls():
        for pool, q, kn, vn, out in layers:
            pa.store_kv(pool, kn, vn, slots)
            pa.decode(q, pool, bt, ctx, case.scale, max_context_len=maxctx, out=out,
                      workspace=ws)

    g, g2 = capture(torch, step), capture(torch, two_calls)
    settle(torch, g)
    ms = time_graph(torch, g, reps)
    ms2 = time_graph(torch, g2, reps)
    dby = decode_bytes(case.context_lens, hq, hkv, D, 2)
    sby = store_bytes(B, hkv, D, 2, 2)
    kern = "decode_fused_kernel<bf16, 128, 6, bf16, step>"
    rec = recorded("decode_qwen_28layer.md", kern.replace(" ", ""), DECODE_SOURCES)
    del layers
    return {"workload": "Qwen2.5-1.5B-shaped decode step: 28 layers x (store 8 new tokens + "
                        "decode), 8 sequences, 12/2 heads, D 128, bf16, contexts U{128..3200}, "
                        "one 4096-block pool per layer, one pa_decode_step launch per layer",
            "ms_per_step": round(ms, 5), "per_layer_us": round(ms / LAYERS * 1e3, 2),
            "two_call_per_layer_us": round(ms2 / LAYERS * 1e3, 2),
            "gbs": round(LAYERS * (dby + sby) / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * LAYERS * (dby + sby) / ms / 1e6 / HBM_PEAK_GBS, 2),
            "seqs_per_s_per_layer": round(B / (ms / LAYERS / 1e3), 1),
            "roofline": roofline(kern, "hbm", dby + sby, ms / LAYERS, HBM_PEAK_GBS, "GB/s", rec,
                                 "one launch per layer (store folded in); achieved = its "
                                 "algorithmic bytes / the graph's time per layer")}


def quant_decode(torch, pa, W, dev, reps, dtype, copies=2):
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
    ws = pa.decode_workspace(B, case.Hq, hkv, D, ctx_len, device=dev)

    def dec():
        for p in pools:
            pa.decode(q, p, bt, ctx, case.scale, max_context_len=ctx_len, out=out, workspace=ws)

    def sto():
        for p in pools:
            pa.store_kv(p, kn, vn, slots)

    g, gs = capture(torch, dec), capture(torch, sto)
    settle(torch, g)
    ms = time_graph(torch, g, reps) / copies
    ms_store = time_graph(torch, gs, reps) / copies
    by = decode_bytes(case.context_lens, case.Hq, hkv, D, 1, scales=True)
    name = "FP8 e4m3" if dtype == "fp8" else "INT8"
    kern = f"decode_fused_kernel<{dtype}, 128, 6, bf16>"
    rec = recorded(f"decode_{dtype}_64x8192.md", kern.replace(" ", ""), DECODE_SOURCES)
    del pools
    return {"workload": f"64 x 8192 {name} decode, 12/2 heads, D 128, per-token-head fp32 "
                        "scales, multi-slot layout viewed as 16-token blocks (277 MB per call)",
            "decode_ms": round(ms, 4), "store_ms": round(ms_store, 4), "kv_bytes": by,
            "gbs": round(by / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * by / ms / 1e6 / HBM_PEAK_GBS, 1),
            "seqs_per_s": round(B / ((ms + ms_store) / 1e3), 1),
            "roofline": roofline(kern, "hbm", by, ms, HBM_PEAK_GBS, "GB/s", rec,
                                 "single-launch decode; achieved = algorithmic bytes / the "
                                 "graph's time per call (two pools alternate)")}


def varlen_prefill(torch, pa, W, dev, reps):
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
                                     device=dev)

    def run():
        pa.varlen_prefill(q, cu, pool, bt, ctx, case.scale, max_q_len=case.max_q_len,
                          max_context_len=case.max_context_len, out=out, workspace=ws)

    g = capture(torch, run)
    gs = capture(torch, lambda: pa.store_kv(pool, kn, vn, slots))
    settle(torch, g)
    ms = time_graph(torch, g, reps)
    ms_store = time_graph(torch, gs, reps)
    fl = prefill_flops(case.extra["n"], case.extra["P"], case.Hq, case.D)
    rec = recorded("prefill_varlen_mixed.md", "prefill_kernel", PREFILL_SOURCES)
    rl = roofline("prefill call (plan + prefill_kernel + merge)", "mfma", fl, ms,
                  BF16_MFMA_PEAK_TFLOPS, "TFLOP/s", rec,
                  "achieved = causal flops (4 D Hq per visible (query, key) pair) / the "
                  "whole call's average time; traffic = HBM bytes of the call's kernels")
    if "mfma_busy_pct" in rec:
        rl["mfma_busy_pct_counter"] = float(rec["mfma_busy_pct"])
        rl["mfma_busy_note"] = ("prefill_kernel: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x "
                                "1024 SIMDs), rocprofv3 counters")
    del pool
    return {"workload": "varlen mixed step: 16 chunks of 1-512 new tokens (4 of length 1) on "
                        "cached prefixes of 0-2048, 12/2 heads, D 128, bf16",
            "prefill_ms": round(ms, 4), "store_ms": round(ms_store, 4),
            "tokens": int(case.cu_seqlens[-1]), "causal_gflop": round(fl / 1e9, 2),
            "tflops": round(fl / ms / 1e9, 1),
            "mfma_util_pct": round(100 * fl / ms / 1e9 / BF16_MFMA_PEAK_TFLOPS, 2),
            "roofline": rl}


def copy_probe(torch, dev, reps=20):
    """A plain 1 GiB device-to-device copy: the bandwidth a simple streaming kernel
    reaches on this GPU (read + write bytes / time), reported beside the HBM peak."""
    a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    g = capture(torch, lambda: b.copy_(a))
    settle(torch, g)
    ms = time_graph(torch, g, reps)
    by = 2 * a.numel() * a.element_size()
    del a, b
    return {"workload": "torch copy of 1 GiB (read + write)", "ms": round(ms, 4),
            "gbs": round(by / ms / 1e6, 1), "pct_hbm_peak": round(100 * by / ms / 1e6 / HBM_PEAK_GBS, 1)}


# ----------------------------------------------------------------------------- CPU baseline

def _oracle_worker(args):
    """One host process: the oracle's store + decode of its sequences, one at a time
    (values drawn once per process, outside the timed region; BLAS single-threaded)."""
    seqs, lens, seed, Hq, Hkv, D, scale = args
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    from oracle import ref
    rng = np.random.default_rng(seed)
    nblk_max = -(-int(max(lens)) // 16)
    kp = rng.standard_normal((nblk_max, 16, Hkv, D))
    vp = rng.standard_normal((nblk_max, 16, Hkv, D))
    q = rng.standard_normal((1, Hq, D))
    kn = rng.standard_normal((1, Hkv, D))
    vn = rng.standard_normal((1, Hkv, D))
    timed, cpu = 0.0, 0.0
    for L in lens:
        nblk = -(-int(L) // 16)
        bt = np.arange(nblk, dtype=np.int32)[None]
        k, v = kp[:nblk], vp[:nblk]
        c0, t0 = time.process_time(), time.perf_counter()
        k2 = ref.store_ref(k, kn, [int(L) - 1])
        v2 = ref.store_ref(v, vn, [int(L) - 1])
        ref.decode_ref(q, k2, v2, bt, np.array([int(L)]), scale)
        timed += time.perf_counter() - t0
        cpu += time.process_time() - c0
    return len(lens), timed, cpu


def cpu_baseline(nsample=256, max_workers=16):
    """The oracle (store + decode) on the headline workload's
    sequences, spread over the host's cores (one single-threaded process per core).
    Runs before the GPU is touched, so the worker processes are plain forks."""
    import multiprocessing as mp
    import workloads as W
    case = W.make(4)
    pick = np.sort(np.random.default_rng(99).choice(case.num_seqs, nsample, replace=False))
    lens = case.context_lens[pick]
    cores = max(1, min(len(os.sched_getaffinity(0)), max_workers))
    shares = [lens[i::cores].tolist() for i in range(cores)]
    jobs = [(pick[i::cores].tolist(), shares[i], 1000 + i, case.Hq, case.Hkv, case.D, case.scale)
            for i in range(cores) if shares[i]]
    with mp.get_context("fork").Pool(len(jobs)) as pool:
        res = pool.map(_oracle_worker, jobs)
    # each process's rate while it computed, summed: the host's aggregate rate
    rate = 0.0
    for (n, timed, cpu), (_, share, *_r) in zip(res, jobs):
        by = decode_bytes(share, case.Hq, case.Hkv, case.D, 2) + \
            store_bytes(len(share), case.Hkv, case.D, 2, 2)
        rate += by / timed
    cpu_total = sum(r[2] for r in res)
    timed_total = sum(r[1] for r in res)
    secs = max(r[1] for r in res)
    seqs_per_s = sum(r[0] / r[1] for r in res)
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": len(jobs),
            "kind": "oracle", "blas_threads_per_process": 1,
            "cpu_seconds": round(cpu_total, 2), "seqs_per_s": round(seqs_per_s, 2),
            "cpu_over_wall_per_process": round(cpu_total / timed_total, 3),
            "sample": f"store + decode of {nsample} seeded sequences of the headline workload "
                      f"({int(lens.sum())} context tokens, lengths {int(lens.min())}.."
                      f"{int(lens.max())}); fp64 numpy oracle, {len(jobs)} single-threaded "
                      f"processes on the host cores of the GPU box (affinity "
                      f"{len(os.sched_getaffinity(0))}), {secs:.1f} s each at most; value = "
                      "the sum of the processes' algorithmic-byte rates"}


# ----------------------------------------------------------------------------- main

def main():
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", choices=WORKLOADS, default=None,
                    help="run one workload (for profiling); prints its figures only")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed replays before each timing (steady clocks)")
    args = ap.parse_args()
    SETTLE_S = args.settle
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this build runs on a "
              "single GPU; the path shards by sequence or KV head with no exchange, so one "
              "process per GPU would run the same kernels on its share.", file=sys.stderr)
        sys.exit(2)

    base = None
    if not args.no_cpu_baseline and args.only is None:
        log("cpu baseline (oracle) on the host cores")
        base = cpu_baseline()

    import torch
    import paged_kv_cache_95_amd as pa
    import workloads as W
    pa.lib()
    dev = torch.device("cuda:0")
    reps = max(args.steps, 10)

    if args.only is not None:
        fn = {"qwen_step": lambda: qwen_step(torch, pa, W, dev, reps),
              "fp8_decode": lambda: quant_decode(torch, pa, W, dev, reps, "fp8"),
              "int8_decode": lambda: quant_decode(torch, pa, W, dev, reps, "int8"),
              "varlen_prefill": lambda: varlen_prefill(torch, pa, W, dev, reps),
              "copy": lambda: copy_probe(torch, dev, reps)}.get(args.only)
        if fn is None:
            r = large_decode(torch, pa, W, dev, args.steps, args.warmup)
            r = {k: v for k, v in r.items() if k != "case"}
        else:
            r = fn()
        # a 256 MiB device copy: its HBM counter readings calibrate FETCH/WRITE_SIZE
        a = torch.empty(1 << 27, dtype=torch.int16, device=dev)
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, **r}), flush=True)
        return

    hl = large_decode(torch, pa, W, dev, args.steps, args.warmup)
    case = hl["case"]
    torch.cuda.empty_cache()
    step_bytes = hl["decode_bytes"] + hl["store_bytes"]
    gbs = step_bytes / hl["ms_step"] / 1e6
    lens = case.context_lens
    res = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(hl["ms_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "large decode step: 256 sequences, 32/8 heads, head_dim 128, "
                               "bf16 KV in 16-token blocks, contexts log-uniform 1K-32K "
                               "(seeded), store of each sequence's new token + decode",
                   "batch": case.num_seqs, "q_heads": case.Hq, "kv_heads": case.Hkv,
                   "head_dim": case.D, "block_size": 16, "pool_blocks": case.num_blocks,
                   "context_tokens": int(lens.sum()), "context_min": int(lens.min()),
                   "context_max": int(lens.max()),
                   "split_tokens": pa.default_split_tokens(case.num_seqs, case.Hkv,
                                                           case.max_context_len),
                   "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(case.num_seqs / (hl["ms_step"] / 1e3), 1),
        "wall_s_timed_region": round(hl["wall"], 4),
        "step_bytes": step_bytes,
        "decode_call_ms": round(hl["decode_ms"], 5),
        "roofline": hl["roofline"],
    }
    if base is not None:
        res["cpu_baseline"] = base
    if not args.no_extra:
        res["extra"] = {}
        for name, fn in (("qwen_step", lambda: qwen_step(torch, pa, W, dev, reps)),
                         ("fp8_decode", lambda: quant_decode(torch, pa, W, dev, reps, "fp8")),
                         ("int8_decode", lambda: quant_decode(torch, pa, W, dev, reps, "int8")),
                         ("varlen_prefill", lambda: varlen_prefill(torch, pa, W, dev, reps)),
                         ("copy", lambda: copy_probe(torch, dev))):
            log(f"extra: {name}")
            res["extra"][name] = fn()
            torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
