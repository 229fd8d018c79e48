"""Brute-force paged attention in pure Python (oracle; test infrastructure).

Structurally different from oracle/ref.py on purpose, so the two pin each other on
tiny inputs: no numpy arithmetic, a block-table lookup per key token, exp of the raw
scores without subtracting a maximum, and math.fsum (exactly rounded sums) for every
reduction. Inputs must be small enough for exp not to overflow (|score| < ~700).

Same definition as oracle/ref.py: key j of sequence s lives at physical slot
block_table[s][j // bs] * bs + j % bs of a [num_blocks, bs, Hkv, D] pool; a row at
absolute position p attends keys 0..p; query head h reads KV head h // (Hq // Hkv).
"""
import math


def _row(pool, bt_row, bs, j, g):
    blk = int(bt_row[j // bs])
    return pool[blk][j % bs][g]


def brute_rows(q_rows, positions, k_pool, v_pool, bt_row, bs, scale):
    """q_rows: nested lists / arrays [R][Hq][D]; pools [nb][bs][Hkv][D] (values).
    Returns out [R][Hq][D] as nested lists of floats."""
    hkv = len(k_pool[0][0])
    out = []
    for r, q in enumerate(q_rows):
        hq = len(q)
        G = hq // hkv
        p = int(positions[r])
        row_out = []
        for h in range(hq):
            g = h // G
            qh = [float(x) for x in q[h]]
            d = len(qh)
            weights = []
            for j in range(p + 1):
                k = _row(k_pool, bt_row, bs, j, g)
                sc = scale * math.fsum(qh[i] * float(k[i]) for i in range(d))
                weights.append(math.exp(sc))
            den = math.fsum(weights)
            o = []
            for i in range(d):
                num = math.fsum(weights[j] * float(_row(v_pool, bt_row, bs, j, g)[i])
                                for j in range(p + 1))
                o.append(num / den)
            row_out.append(o)
        out.append(row_out)
    return out


def brute_decode(q, k_pool, v_pool, block_tables, context_lens, bs, scale):
    return [brute_rows([q[s]], [int(context_lens[s]) - 1], k_pool, v_pool,
                       block_tables[s], bs, scale)[0]
            for s in range(len(context_lens))]


def brute_varlen(q, cu_seqlens, k_pool, v_pool, block_tables, context_lens, bs, scale):
    out = [None] * int(cu_seqlens[-1])
    for s in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        n = b - a
        P = int(context_lens[s]) - n
        rows = brute_rows([q[t] for t in range(a, b)], [P + i for i in range(n)],
                          k_pool, v_pool, block_tables[s], bs, scale)
        for i in range(n):
            out[a + i] = rows[i]
    return out
