"""Block manager output driving the kernels: sequences that share prefix blocks, and a
forked sequence after copy-on-write, attend exactly their own tokens (decode against
the oracle); pa_copy_blocks copies K, V and scales."""
import numpy as np
import pytest
import torch

import paged_kv_cache_95_amd as pa
import workloads as W
from oracle import ref

from _harness import TOL, max_err

pytestmark = pytest.mark.gpu

HKV, HQ, D, VOCAB, MAXPOS = 2, 12, 128, 50, 96


def _kv_table(seed):
    """K / V value of (token id, position): identical prefixes give identical rows."""
    rng = np.random.default_rng(seed)
    k = W.round_to_bf16(rng.standard_normal((VOCAB, MAXPOS, HKV, D)).astype(np.float32))
    v = W.round_to_bf16(rng.standard_normal((VOCAB, MAXPOS, HKV, D)).astype(np.float32))
    return k, v


def _store(pool, kt, vt, tokens, positions, slots, dev):
    k = np.stack([kt[tokens[p], p] for p in positions])
    v = np.stack([vt[tokens[p], p] for p in positions])
    pa.store_kv(pool, torch.from_numpy(k).to(torch.bfloat16).to(dev),
                torch.from_numpy(v).to(torch.bfloat16).to(dev),
                torch.from_numpy(np.asarray(slots, np.int64)).to(dev))


def _check_decode(bm, pool, kt, vt, seqs, tokens_of, dev, seed):
    q = W.round_to_bf16(np.random.default_rng(seed).standard_normal(
        (len(seqs), HQ, D)).astype(np.float32))
    bt, cl = bm.block_tables(seqs, MAXPOS // 16 + 1)
    out = pa.decode(torch.from_numpy(q).to(torch.bfloat16).to(dev), pool,
                    torch.from_numpy(bt).to(dev), torch.from_numpy(cl).to(dev),
                    1 / np.sqrt(D), split_tokens=16)
    torch.cuda.synchronize()
    # oracle: dense attention over each sequence's own tokens, one sequence per pool
    exp = np.zeros((len(seqs), HQ, D))
    for i, s in enumerate(seqs):
        t = tokens_of[s]
        K = np.stack([kt[t[p], p] for p in range(len(t))])[None]    # [1, L, Hkv, D]
        V = np.stack([vt[t[p], p] for p in range(len(t))])[None]
        table = np.arange(-(-len(t) // 16), dtype=np.int32)[None]
        Kp = np.zeros((table.shape[1], 16, HKV, D))
        Vp = np.zeros_like(Kp)
        Kp.reshape(-1, HKV, D)[:len(t)] = K[0]
        Vp.reshape(-1, HKV, D)[:len(t)] = V[0]
        exp[i] = ref.decode_ref(q[i:i + 1], Kp, Vp, table, np.array([len(t)], np.int32),
                                1 / np.sqrt(D))[0][0]
    err = max_err(out, exp)
    print(f"block-manager decode max_abs_err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_shared_prefix_blocks_feed_decode(dev):
    kt, vt = _kv_table(1)
    rng = np.random.default_rng(2)
    bm = pa.BlockManager(64)
    pool = pa.KVPool.empty(64, HKV, D, "bf16", dev)
    pool.k.fill_(float("nan"))
    pool.v.fill_(float("nan"))
    base = list(rng.integers(0, VOCAB, 70))
    tokens_of = {1: base[:50], 2: base[:40] + list(rng.integers(0, VOCAB, 5)), 3: base[:66]}
    for s, t in tokens_of.items():
        cached = bm.add_sequence(s, t)
        assert cached == {1: 0, 2: 32, 3: 48}[s]
        # compute (store) only what the prefix cache does not already hold
        _store(pool, kt, vt, t, range(cached, len(t)), bm.slots(s, cached, len(t) - cached), dev)
    bt, _ = bm.block_tables([1, 2, 3], 6)
    assert bt[0, 0] == bt[1, 0] == bt[2, 0] and bt[0, 2] == bt[2, 2] != bt[1, 2]
    _check_decode(bm, pool, kt, vt, [1, 2, 3], tokens_of, dev, 3)


def test_fork_copy_on_write_feeds_decode(dev):
    kt, vt = _kv_table(4)
    rng = np.random.default_rng(5)
    bm = pa.BlockManager(32)
    pool = pa.KVPool.empty(32, HKV, D, "bf16", dev)
    pool.k.fill_(float("nan"))
    pool.v.fill_(float("nan"))
    t1 = list(rng.integers(0, VOCAB, 37))
    bm.add_sequence(1, t1)
    _store(pool, kt, vt, t1, range(37), bm.slots(1, 0, 37), dev)
    bm.fork(1, 2)
    tokens_of = {1: list(t1), 2: list(t1)}
    for step in range(20):                       # both grow; the first append COWs
        for s in (2, 1):
            tok = int(rng.integers(0, VOCAB))
            slot, cs, cd = bm.append(s, tok)
            if cs >= 0:
                pa.copy_blocks(pool, torch.tensor([cs], dtype=torch.int32, device=dev),
                               torch.tensor([cd], dtype=torch.int32, device=dev))
            tokens_of[s].append(tok)
            _store(pool, kt, vt, tokens_of[s], [len(tokens_of[s]) - 1], [slot], dev)
    bt, _ = bm.block_tables([1, 2], 4)
    assert bt[0, 0] == bt[1, 0] and bt[0, 1] == bt[1, 1] and bt[0, 2] != bt[1, 2]
    _check_decode(bm, pool, kt, vt, [1, 2], tokens_of, dev, 6)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "int8"])
def test_copy_blocks(dev, dtype):
    pool = pa.KVPool.empty(10, 2, 64, dtype, dev)
    for t in (pool.k, pool.v):
        t.view(torch.uint8).copy_(torch.randint(0, 256, t.view(torch.uint8).shape,
                                                dtype=torch.uint8, device=dev))
    if pool.k_scale is not None:
        pool.k_scale.copy_(torch.rand_like(pool.k_scale))
        pool.v_scale.copy_(torch.rand_like(pool.v_scale))
    before = [t.clone() for t in (pool.k, pool.v, pool.k_scale, pool.v_scale) if t is not None]
    src = torch.tensor([1, 2, 7, 99], dtype=torch.int32, device=dev)   # 99: skipped
    dst = torch.tensor([5, 6, 0, 3], dtype=torch.int32, device=dev)
    pa.copy_blocks(pool, src, dst)
    torch.cuda.synchronize()
    after = [t for t in (pool.k, pool.v, pool.k_scale, pool.v_scale) if t is not None]
    for b0, a in zip(before, after):
        exp = b0.clone()
        exp[[5, 6, 0]] = b0[[1, 2, 7]]
        assert torch.equal(a.view(torch.uint8), exp.view(torch.uint8))
