"""Seeded synthetic inputs for paged GQA attention, shared by tests and the benchmark.

This module holds no attention arithmetic: it draws random values, lays out block
tables the way an engine's block manager would (a global pool of 16-token blocks,
handed out from a seeded permutation), and writes the slot_mapping an engine would
pass for the new tokens. Both the HIP path and the CPU oracle consume what it returns;
the oracle re-derives every slot from the block tables itself.

Values are drawn as float32 N(0, 1) and rounded to the storage dtype (bf16 by
round-to-nearest-even); the rounded values are the ground truth. Large pools (the
256-sequence decode and the FP8 decode) are filled on the device with a seeded torch
generator instead; see fill_device_normal_().

Configurations (sizes as named in the project brief):
  1 tiny decode        B=1, L=37, Hq=2, Hkv=1, D=64, fp32, pool of 8 blocks,
                       block table = permutation(8), scale 1/8; all 37 tokens stored.
  2 qwen decode        B=8, Hq=12, Hkv=2, D=128, bf16 pool of 4096 blocks, L_s ~ U{128..3200}
                       counted after the new token is stored; one new token per sequence.
  3 varlen mixed       16 sequences; 4 of them (seeded positions) are 1-token chunks, the
                       rest n_s ~ U{2..512}; cached prefix P_s ~ U{0..2048}; Hq=12, Hkv=2,
                       D=128, bf16, pool 4096 blocks.
  4 large decode       B=256, Hq=32, Hkv=8, D=128, bf16, L_s = floor(exp(U(ln 1024, ln 32768))),
                       pool = sum ceil(L_s/16) blocks, permuted.
  5 fp8 decode         B=64, L=8192 each, Hq=12, Hkv=2, D=128; bf16 source quantised into an
                       FP8 pool by the store; multi-slot layout [64, 8192, Hkv, D] viewed as
                       16-token blocks, block_tables[s][j] = s*512 + j (a permuted twin
                       placement is available).
"""
from dataclasses import dataclass, field
import math

import numpy as np

BLOCK_SIZE = 16


def round_to_bf16(x):
    """float32 -> nearest bfloat16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x):
    """Raw bits (uint16) of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def normal(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype in ("bf16", "fp8", "int8"):   # quantised pools are fed from a bf16 source
        x = round_to_bf16(x)
    return x


@dataclass
class Case:
    name: str
    seed: int
    kind: str                      # "decode" or "varlen"
    Hq: int
    Hkv: int
    D: int
    kv_dtype: str                  # "f32", "bf16", "fp8", "int8"
    q_dtype: str                   # "f32", "bf16"
    num_blocks: int
    block_tables: np.ndarray       # int32 [B, max_blocks_per_seq]; unused entries -1
    context_lens: np.ndarray       # int32 [B]
    q: np.ndarray                  # float32 values [T_q, Hq, D]
    k_new: np.ndarray              # float32 values [T_new, Hkv, D] (src dtype exact)
    v_new: np.ndarray
    new_seq: np.ndarray            # int64 [T_new] sequence of each new token
    new_pos: np.ndarray            # int64 [T_new] logical position of each new token
    slot_mapping: np.ndarray       # int64 [T_new]
    cu_seqlens: np.ndarray = None  # int32 [B+1] for varlen
    scale: float = 0.0
    block_size: int = BLOCK_SIZE
    pool_fill: str = "random"      # "random" (host), "nan", or "device"
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self):
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self):
        return int(self.context_lens.max())

    @property
    def max_q_len(self):
        if self.cu_seqlens is None:
            return 1
        return int(np.max(np.diff(self.cu_seqlens))) if self.num_seqs else 0

    @property
    def src_dtype(self):
        return "bf16" if self.kv_dtype in ("fp8", "int8") else self.kv_dtype


def _tables_from_perm(perm, lens, max_blocks, bs=BLOCK_SIZE):
    """Consecutive slices of a permutation of physical blocks become each sequence's
    block table (what a block manager handing out free blocks produces)."""
    B = len(lens)
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for s, L in enumerate(lens):
        nb = -(-int(L) // bs)
        bt[s, :nb] = perm[off:off + nb]
        off += nb
    return bt, off


def _slots(bt, seqs, pos, bs=BLOCK_SIZE):
    """slot_mapping an engine passes for new tokens at (sequence, position)."""
    return np.array([int(bt[s, p // bs]) * bs + p % bs for s, p in zip(seqs, pos)],
                    dtype=np.int64)


def tiny_decode(seed=1):
    rng = np.random.default_rng(seed)
    L, Hq, Hkv, D, nb = 37, 2, 1, 64, 8
    bt = rng.permutation(nb).astype(np.int32)[None, :]
    q = normal(rng, (1, Hq, D), "f32")
    k = normal(rng, (L, Hkv, D), "f32")
    v = normal(rng, (L, Hkv, D), "f32")
    seqs = np.zeros(L, dtype=np.int64)
    pos = np.arange(L, dtype=np.int64)
    return Case("tiny_decode", seed, "decode", Hq, Hkv, D, "f32", "f32", nb, bt,
                np.array([L], dtype=np.int32), q, k, v, seqs, pos, _slots(bt, seqs, pos),
                scale=1.0 / math.sqrt(D), pool_fill="nan")


def qwen_decode(seed=2, batch=8, lmin=128, lmax=3200, num_blocks=4096):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = 12, 2, 128
    lens = rng.integers(lmin, lmax + 1, size=batch).astype(np.int32)
    perm = rng.permutation(num_blocks).astype(np.int32)
    max_blocks = -(-lmax // BLOCK_SIZE)
    bt, used = _tables_from_perm(perm, lens, max_blocks)
    assert used <= num_blocks
    q = normal(rng, (batch, Hq, D), "bf16")
    k = normal(rng, (batch, Hkv, D), "bf16")
    v = normal(rng, (batch, Hkv, D), "bf16")
    seqs = np.arange(batch, dtype=np.int64)
    pos = lens.astype(np.int64) - 1
    return Case("qwen_decode", seed, "decode", Hq, Hkv, D, "bf16", "bf16", num_blocks, bt,
                lens, q, k, v, seqs, pos, _slots(bt, seqs, pos),
                scale=1.0 / math.sqrt(D), pool_fill="random")


def varlen_mixed(seed=3, nseq=16, n_decode=4, nmax=512, pmax=2048, num_blocks=4096,
                 Hq=12, Hkv=2, D=128):
    rng = np.random.default_rng(seed)
    n = rng.integers(2, nmax + 1, size=nseq)
    dec = rng.choice(nseq, size=n_decode, replace=False)
    n[dec] = 1
    P = rng.integers(0, pmax + 1, size=nseq)
    lens = (P + n).astype(np.int32)
    perm = rng.permutation(num_blocks).astype(np.int32)
    max_blocks = -(-(pmax + nmax) // BLOCK_SIZE)
    bt, used = _tables_from_perm(perm, lens, max_blocks)
    assert used <= num_blocks
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    T = int(cu[-1])
    q = normal(rng, (T, Hq, D), "bf16")
    k = normal(rng, (T, Hkv, D), "bf16")
    v = normal(rng, (T, Hkv, D), "bf16")
    seqs = np.repeat(np.arange(nseq), n).astype(np.int64)
    pos = np.concatenate([P[s] + np.arange(n[s]) for s in range(nseq)]).astype(np.int64)
    return Case("varlen_mixed", seed, "varlen", Hq, Hkv, D, "bf16", "bf16", num_blocks, bt,
                lens, q, k, v, seqs, pos, _slots(bt, seqs, pos), cu_seqlens=cu,
                scale=1.0 / math.sqrt(D), pool_fill="random",
                extra={"n": n.astype(np.int64), "P": P.astype(np.int64)})


def large_decode(seed=4, batch=256, lmin=1024, lmax=32768):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = 32, 8, 128
    lens = np.floor(np.exp(rng.uniform(math.log(lmin), math.log(lmax), size=batch)))
    lens = np.clip(lens, lmin, lmax).astype(np.int32)
    nblk = int(sum(-(-int(L) // BLOCK_SIZE) for L in lens))
    perm = rng.permutation(nblk).astype(np.int32)
    bt, used = _tables_from_perm(perm, lens, -(-lmax // BLOCK_SIZE))
    q = normal(rng, (batch, Hq, D), "bf16")
    k = normal(rng, (batch, Hkv, D), "bf16")
    v = normal(rng, (batch, Hkv, D), "bf16")
    seqs = np.arange(batch, dtype=np.int64)
    pos = lens.astype(np.int64) - 1
    return Case("large_decode", seed, "decode", Hq, Hkv, D, "bf16", "bf16", nblk, bt,
                lens, q, k, v, seqs, pos, _slots(bt, seqs, pos),
                scale=1.0 / math.sqrt(D), pool_fill="device")


def fp8_decode(seed=5, batch=64, ctx=8192, permuted=False):
    """Multi-slot FP8 pool; setup stores ctx-1 prefix tokens per slot from a bf16 source
    generated on the device (fill_device_normal_ with seed*1000+1 for K, +2 for V), the
    step stores the last token (k_new/v_new here) and attends all ctx tokens."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = 12, 2, 128
    per = ctx // BLOCK_SIZE
    nb = batch * per
    bt = (np.arange(batch)[:, None] * per + np.arange(per)[None, :]).astype(np.int32)
    if permuted:
        perm = rng.permutation(nb).astype(np.int32)
        bt = perm[bt]
    else:
        rng.permutation(nb)   # keep the draw order identical between the twins
    lens = np.full(batch, ctx, dtype=np.int32)
    q = normal(rng, (batch, Hq, D), "bf16")
    k = normal(rng, (batch, Hkv, D), "bf16")
    v = normal(rng, (batch, Hkv, D), "bf16")
    seqs = np.arange(batch, dtype=np.int64)
    pos = lens.astype(np.int64) - 1
    return Case("fp8_decode", seed, "decode", Hq, Hkv, D, "fp8", "bf16", nb, bt, lens,
                q, k, v, seqs, pos, _slots(bt, seqs, pos), scale=1.0 / math.sqrt(D),
                pool_fill="device", extra={"ctx": ctx, "per_slot_blocks": per})


CONFIGS = {1: tiny_decode, 2: qwen_decode, 3: varlen_mixed, 4: large_decode, 5: fp8_decode}


def make(cfg, seed=None, **kw):
    fn = CONFIGS[cfg]
    return fn(seed=cfg if seed is None else seed, **kw)


# ----------------------------------------------------------------------------- small cases

def random_case(seed, kind="decode", B=3, Hq=4, Hkv=2, D=64, kv_dtype="bf16", bs=BLOCK_SIZE,
                lmin=1, lmax=80, nmax=20, num_blocks=None, poison=True):
    """Small random case for tests: random lengths (and chunks for varlen), blocks
    scattered over a pool with spare blocks; pool_fill 'nan' poisons every slot that is
    not part of any sequence's context."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lmin, lmax + 1, size=B).astype(np.int32)
    if kind == "varlen":
        n = np.minimum(rng.integers(0, nmax + 1, size=B), lens)
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    need = int(sum(-(-int(L) // bs) for L in lens))
    nb = num_blocks or need + 5
    perm = rng.permutation(nb).astype(np.int32)
    max_blocks = -(-lmax // bs) + 1
    bt, _ = _tables_from_perm(perm, lens, max_blocks, bs)
    src = "bf16" if kv_dtype in ("fp8", "int8") else kv_dtype
    qd = "f32" if kv_dtype == "f32" else "bf16"
    if kind == "decode":
        q = normal(rng, (B, Hq, D), qd)
        seqs = np.arange(B, dtype=np.int64)
        pos = lens.astype(np.int64) - 1
        cu = None
    else:
        q = normal(rng, (int(cu[-1]), Hq, D), qd)
        seqs = np.repeat(np.arange(B), n).astype(np.int64)
        pos = np.concatenate([lens[s] - n[s] + np.arange(n[s]) for s in range(B)]
                             ).astype(np.int64) if cu[-1] else np.zeros(0, np.int64)
    T = len(seqs)
    k = normal(rng, (T, Hkv, D), src)
    v = normal(rng, (T, Hkv, D), src)
    return Case(f"random_{kind}_{seed}", seed, kind, Hq, Hkv, D, kv_dtype, qd, nb, bt, lens,
                q, k, v, seqs, pos, _slots(bt, seqs, pos, bs), cu_seqlens=cu,
                scale=1.0 / math.sqrt(D), block_size=bs,
                pool_fill="nan" if poison else "random")


# ----------------------------------------------------------------------------- pools

def used_slot_mask(case):
    """Boolean [num_blocks, bs]: True for slots inside some sequence's context."""
    bs = case.block_size
    used = np.zeros((case.num_blocks, bs), dtype=bool)
    for s in range(case.num_seqs):
        L = int(case.context_lens[s])
        for j in range(-(-L // bs)):
            blk = int(case.block_tables[s, j])
            cnt = min(bs, L - j * bs)
            used[blk, :cnt] = True
    return used


def host_pool(case, which, poison_unused=None):
    """float32 values [num_blocks, bs, Hkv, D] of the pool before this step's store:
    N(0,1) in the pool's source dtype (seeded by case.seed and `which` = 'k' or 'v');
    with poison_unused (default: pool_fill == 'nan') every slot outside all contexts
    holds NaN."""
    rng = np.random.default_rng([case.seed, 1 if which == "k" else 2])
    shape = (case.num_blocks, case.block_size, case.Hkv, case.D)
    x = normal(rng, shape, case.src_dtype)
    if poison_unused is None:
        poison_unused = case.pool_fill == "nan"
    if poison_unused:
        x[~used_slot_mask(case)] = np.nan
    return x


def prefix_tokens(case):
    """Context tokens that are not stored in this step, as (seq, pos) arrays, plus a
    bf16 source row for each (K and V, [n, Hkv, D] float32 values). Used to populate
    FP8 pools through the store, so both the GPU and the oracle quantise them."""
    new = set(zip(case.new_seq.tolist(), case.new_pos.tolist()))
    rows = [(s, p) for s in range(case.num_seqs) for p in range(int(case.context_lens[s]))
            if (s, p) not in new]
    seqs = np.array([r[0] for r in rows], dtype=np.int64)
    pos = np.array([r[1] for r in rows], dtype=np.int64)
    rng = np.random.default_rng([case.seed, 7])
    k = normal(rng, (len(rows), case.Hkv, case.D), "bf16")
    v = normal(rng, (len(rows), case.Hkv, case.D), "bf16")
    slots = _slots(case.block_tables, seqs, pos, case.block_size) if len(rows) else \
        np.zeros(0, np.int64)
    return seqs, pos, slots, k, v


def fill_device_normal_(tensor, seed):
    """Fill a torch tensor (any float dtype, on its device) with N(0,1) from a seeded
    generator on that device; values are rounded to the tensor's dtype by torch."""
    import torch
    g = torch.Generator(device=tensor.device)
    g.manual_seed(int(seed))
    flat = tensor.view(-1)
    chunk = 1 << 28
    for a in range(0, flat.numel(), chunk):
        b = min(flat.numel(), a + chunk)
        flat[a:b] = torch.randn(b - a, generator=g, device=tensor.device,
                                dtype=torch.float32).to(tensor.dtype)
    return tensor


def rope_tables(max_position, head_dim, base=1.0e6):
    """cos / sin tables, float32 [max_position, head_dim/2], of the usual rotary schedule
    angle(p, i) = p * base^(-2i/head_dim) (Qwen2.5 uses base 1e6). Any table is a valid
    input to the fused RoPE store; this one is the realistic case."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
