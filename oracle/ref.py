"""Plain fp64 definition of paged GQA attention (oracle; test infrastructure).

What the path computes has a plain definition, so this module writes that definition
out, the "gather then dense attention" way:

* store: every new K/V row goes to the physical slot slot_mapping[t] (koas-w "errors
  and solutions" post, "hand-written Triton kernels": store_kvcache_kernel); a negative
  slot is padding and is skipped (reading taken where the pages are silent).
* slot of logical position j of sequence s: block_table[s][j // bs] * bs + j % bs
  (same post, "KV Cache management": a block_table maps logical blocks of 16 tokens to
  physical blocks of one global pool).
* gather: the first L_s tokens of sequence s are collected through its block table
  (mini-vllm "step14_7 - Batched Forward", per-sequence gather of the KV blocks; same
  as the "PagedAttention (gather)" version of the koas-w post).
* attention: query row at absolute position p attends keys 0..p of its own sequence,
  softmax(scale * q.K^T) V, with query head h reading KV head h // G (contiguous GQA
  groups, the convention of the HF model the post aligns with tensor by tensor).
  Decode: one row per sequence at p = L_s - 1 (context_lens includes the token just
  stored: koas-w post, "errors, type 1"). Varlen: the chunk of sequence s is rows
  cu[s]..cu[s+1]-1 at positions P_s + i with P_s = L_s - n_s (mini-vllm step14_7,
  cu_seqlens segments attention; attention(seq_q, K_full, V_full, start_position)).

All arithmetic is float64. Pool arguments are float64 VALUE arrays
[num_blocks, bs, Hkv, D]; helpers convert raw bf16/fp32 bits and FP8 codes exactly.

Pinned by (tests/test_oracle_*.py): the pure-Python brute force in oracle/brute.py;
closed forms (L = 1 gives v; q = 0 gives the causal prefix mean, including the
hand-computed fixture tests/golden/varlen_prefix_mean_p5.txt on the cu_seqlens
[0,3,4,6] structure of the varlen page; V constant; identical keys; one dominant key);
invariants (block permutation, paged == contiguous, key shift, V shift, GQA == MHA with
repeated KV heads); and merge-of-partials == unsplit.
"""
import numpy as np


# ----------------------------------------------------------------------------- values

def bf16_bits_to_f64(bits):
    """Exact value of raw bfloat16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_f64(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- store

def slot_of(block_table_row, j, bs):
    """Physical slot of logical token position j of one sequence."""
    return int(block_table_row[j // bs]) * bs + (j % bs)


def store_ref(pool, src, slot_mapping):
    """Copy rows src[t] ([T, Hkv, D], any dtype incl. raw bits) into a copy of
    pool ([nb, bs, Hkv, D], same dtype) at slot_mapping[t]; slots < 0 are skipped.
    Bit-level: the array dtype is preserved, nothing is converted."""
    out = pool.copy()
    nb, bs = pool.shape[0], pool.shape[1]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= nb * bs:
            continue
        out[slot // bs, slot % bs] = src[t]
    return out


def store_fp8_ref(codes, scales, src_f32, slot_mapping):
    """FP8 store: each source row (float32 values [T, Hkv, D]) is quantised per
    (token, head) row by oracle.fp8.quantize_rows and written with its scale.
    codes: uint8 [nb, bs, Hkv, D]; scales: float32 [nb, bs, Hkv]. Returns copies."""
    from . import fp8
    c_out, s_out = codes.copy(), scales.copy()
    q_codes, q_scale = fp8.quantize_rows(src_f32)
    nb, bs = codes.shape[0], codes.shape[1]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= nb * bs:
            continue
        c_out[slot // bs, slot % bs] = q_codes[t]
        s_out[slot // bs, slot % bs] = q_scale[t]
    return c_out, s_out


def store_int8_ref(codes, scales, src_f32, slot_mapping):
    """INT8 store: as store_fp8_ref with oracle.int8.quantize_rows. codes: int8
    [nb, bs, Hkv, D]; scales: float32 [nb, bs, Hkv]. Returns copies."""
    from . import int8
    c_out, s_out = codes.copy(), scales.copy()
    q_codes, q_scale = int8.quantize_rows(src_f32)
    nb, bs = codes.shape[0], codes.shape[1]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= nb * bs:
            continue
        c_out[slot // bs, slot % bs] = q_codes[t]
        s_out[slot // bs, slot % bs] = q_scale[t]
    return c_out, s_out


# ----------------------------------------------------------------------------- gather

def gather_seq(pool_vals, block_table_row, length):
    """[length, Hkv, D] float64: the sequence's tokens 0..length-1, read through its
    block table one token at a time (only blocks 0..ceil(length/bs)-1 are touched)."""
    nb, bs, hkv, d = pool_vals.shape
    flat = pool_vals.reshape(nb * bs, hkv, d)
    slots = [slot_of(block_table_row, j, bs) for j in range(length)]
    return flat[np.asarray(slots, dtype=np.int64)].astype(np.float64)


# ----------------------------------------------------------------------------- attention

def attend(q_rows, positions, K, V, scale, keys=None):
    """Dense causal GQA attention of query rows against one sequence's keys.

    q_rows [R, Hq, D], positions [R] (absolute, row r sees keys j <= positions[r]),
    K, V [L, Hkv, D]. keys: optional boolean mask [L] restricting the key set (used for
    split partials). Returns out [R, Hq, D], lse [R, Hq] (natural log of the
    normaliser sum_j exp(s_j)), rowsum [R, Hq] (sum of the softmax weights).
    A row with no visible key gets out = 0, lse = -inf, rowsum = 0."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R, Hq, D = q_rows.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    pos = np.asarray(positions, dtype=np.int64)
    visible = np.arange(L)[None, :] <= pos[:, None]
    if keys is not None:
        visible = visible & np.asarray(keys, dtype=bool)[None, :]
    out = np.zeros((R, Hq, D))
    lse = np.full((R, Hq), -np.inf)
    rowsum = np.zeros((R, Hq))
    for h in range(Hq):
        g = h // G
        s = scale * (q_rows[:, h, :] @ K[:, g, :].T)          # [R, L]
        s = np.where(visible, s, -np.inf)
        m = np.max(s, axis=1)
        any_vis = np.isfinite(m)
        m_safe = np.where(any_vis, m, 0.0)
        w = np.where(visible, np.exp(s - m_safe[:, None]), 0.0)
        den = w.sum(axis=1)
        num = w @ V[:, g, :]
        ok = any_vis & (den > 0)
        out[ok, h, :] = num[ok] / den[ok, None]
        lse[ok, h] = m_safe[ok] + np.log(den[ok])
        rowsum[ok, h] = (w[ok] / den[ok, None]).sum(axis=1)
    return out, lse, rowsum


def decode_ref(q, k_pool, v_pool, block_tables, context_lens, scale):
    """Paged decode: q [B, Hq, D]; pools float64 values [nb, bs, Hkv, D];
    block_tables [B, maxb]; context_lens [B]. Row s sits at position L_s - 1.
    Returns out [B, Hq, D], lse [B, Hq]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for s in range(B):
        L = int(context_lens[s])
        K = gather_seq(k_pool, block_tables[s], L)
        V = gather_seq(v_pool, block_tables[s], L)
        o, l, _ = attend(q[s:s + 1], [L - 1], K, V, scale)
        out[s], lse[s] = o[0], l[0]
    return out, lse


def varlen_ref(q, cu_seqlens, k_pool, v_pool, block_tables, context_lens, scale):
    """Varlen causal prefill: q [T, Hq, D]; chunk s is rows cu[s]..cu[s+1]-1 at
    positions P_s + i, P_s = L_s - n_s. Returns out [T, Hq, D], lse [T, Hq]."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D))
    lse = np.zeros((T, Hq))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        n = b - a
        if n == 0:
            continue
        L = int(context_lens[s])
        if n > L:
            raise ValueError("chunk longer than its context")
        P = L - n
        K = gather_seq(k_pool, block_tables[s], L)
        V = gather_seq(v_pool, block_tables[s], L)
        o, l, _ = attend(q[a:b], P + np.arange(n), K, V, scale)
        out[a:b], lse[a:b] = o, l
    return out, lse


# ----------------------------------------------------------------------------- split-K

def partial_ref(q_rows, positions, K, V, scale, key_lo, key_hi):
    """Partial attention over keys [key_lo, key_hi): (lse [R, Hq], o [R, Hq, D]) with
    o normalised over that key range only (lse = -inf, o = 0 for an empty range)."""
    L = K.shape[0]
    keys = (np.arange(L) >= key_lo) & (np.arange(L) < key_hi)
    o, lse, _ = attend(q_rows, positions, K, V, scale, keys=keys)
    return lse, o


def merge_ref(lses, outs):
    """Log-sum-exp merge of partials: M = max_i lse_i, w_i = exp(lse_i - M),
    out = sum_i w_i o_i / sum_i w_i, LSE = M + log sum_i w_i. Inputs are lists of
    [..., ] lse arrays and [..., D] o arrays; partials with lse = -inf weigh 0."""
    lses = np.stack([np.asarray(x, dtype=np.float64) for x in lses])   # [S, ...]
    outs = np.stack([np.asarray(x, dtype=np.float64) for x in outs])   # [S, ..., D]
    M = np.max(lses, axis=0)
    w = np.exp(lses - M[None])
    den = w.sum(axis=0)
    out = (w[..., None] * outs).sum(axis=0) / den[..., None]
    return out, M + np.log(den)
