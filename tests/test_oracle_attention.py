"""Pins of the oracle's attention, store and merge (CPU only).

Each test fixes something a plausible mistake in oracle/ref.py would break: the brute
force (different structure: per-token lookups, no max subtraction, exact sums) catches
dropped terms, wrong scale, wrong head mapping and index slips; the closed forms and the
hand-computed fixture pin the causal alignment of chunks on a cached prefix and the
cu_seqlens segmentation; the invariants pin the block-table indirection.
"""
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import brute, ref
from oracle import fp8 as ofp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "varlen_prefix_mean_p5.txt")


def pools_after_store(case, poison=None):
    """Oracle-side pools (float64 values) after this step's store."""
    kp = W.host_pool(case, "k", poison).astype(np.float64)
    vp = W.host_pool(case, "v", poison).astype(np.float64)
    kp = ref.store_ref(kp, case.k_new.astype(np.float64), case.slot_mapping)
    vp = ref.store_ref(vp, case.v_new.astype(np.float64), case.slot_mapping)
    return kp, vp


def run_ref(case, kp, vp):
    if case.kind == "decode":
        return ref.decode_ref(case.q, kp, vp, case.block_tables, case.context_lens,
                              case.scale)[0]
    return ref.varlen_ref(case.q, case.cu_seqlens, kp, vp, case.block_tables,
                          case.context_lens, case.scale)[0]


def run_brute(case, kp, vp):
    if case.kind == "decode":
        return np.array(brute.brute_decode(case.q, kp, vp, case.block_tables,
                                           case.context_lens, case.block_size, case.scale))
    out = brute.brute_varlen(case.q, case.cu_seqlens, kp, vp, case.block_tables,
                             case.context_lens, case.block_size, case.scale)
    return np.array(out).reshape(case.q.shape)


# ----------------------------------------------------------------------------- brute force

def test_brute_tiny_decode_config():
    case = W.make(1)
    kp, vp = pools_after_store(case)
    a, b = run_ref(case, kp, vp), run_brute(case, kp, vp)
    assert np.max(np.abs(a - b)) <= 1e-12


@pytest.mark.parametrize("seed,kind,bs,hq,hkv", [
    (11, "decode", 16, 4, 2), (12, "decode", 4, 6, 1), (13, "varlen", 16, 4, 2),
    (14, "varlen", 4, 3, 3), (15, "varlen", 4, 8, 2), (16, "decode", 4, 2, 2)])
def test_brute_random_tiny(seed, kind, bs, hq, hkv):
    case = W.random_case(seed, kind=kind, B=3, Hq=hq, Hkv=hkv, D=8, kv_dtype="f32", bs=bs,
                         lmax=40, nmax=9)
    kp, vp = pools_after_store(case)
    a, b = run_ref(case, kp, vp), run_brute(case, kp, vp)
    assert np.all(np.isfinite(a))
    assert np.max(np.abs(a - b)) <= 1e-12


def test_brute_p5_structure_random_values():
    rng = np.random.default_rng(5)
    cu = np.array([0, 3, 4, 6], dtype=np.int32)
    lens = np.array([5, 4, 2], dtype=np.int32)
    bt = np.array([[3, 0], [5, -1], [1, -1]], dtype=np.int32)
    kp = rng.standard_normal((6, 4, 1, 4))
    vp = rng.standard_normal((6, 4, 1, 4))
    q = rng.standard_normal((6, 2, 4))
    a = ref.varlen_ref(q, cu, kp, vp, bt, lens, 0.7)[0]
    b = np.array(brute.brute_varlen(q, cu, kp, vp, bt, lens, 4, 0.7))
    assert np.max(np.abs(a - b)) <= 1e-12


# ----------------------------------------------------------------------------- closed forms

def _golden_case():
    g = {"table": {}, "v": [], "out": []}
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if not line:
            continue
        key, vals = line[0], line[1:]
        if key == "table":
            g["table"][int(vals[0])] = [int(x) for x in vals[1:]]
        elif key in ("v", "out"):
            g[key].append([float(x) for x in vals])
        elif key in ("cu_seqlens", "context_lens"):
            g[key] = [int(x) for x in vals]
        else:
            g[key] = int(vals[0])
    return g


def test_golden_varlen_prefix_mean_p5():
    g = _golden_case()
    bs, hq, hkv, d, nb = g["block_size"], g["hq"], g["hkv"], g["d"], g["num_blocks"]
    nseq = len(g["context_lens"])
    bt = np.full((nseq, 4), -1, dtype=np.int32)
    for s, row in g["table"].items():
        bt[s, :len(row)] = row
    vp = np.full((nb, bs, hkv, d), np.nan)
    kp = np.full((nb, bs, hkv, d), np.nan)
    rng = np.random.default_rng(0)
    for s, pos, *v in g["v"]:
        s, pos = int(s), int(pos)
        blk = bt[s, pos // bs]
        vp[blk, pos % bs, 0] = v
        kp[blk, pos % bs, 0] = rng.standard_normal(d)
    T = g["cu_seqlens"][-1]
    q = np.zeros((T, hq, d))
    out = ref.varlen_ref(q, g["cu_seqlens"], kp, vp, bt, g["context_lens"], 0.5)[0]
    exp = np.zeros((T, d))
    for t, *o in g["out"]:
        exp[int(t)] = o
    for h in range(hq):
        assert np.max(np.abs(out[:, h] - exp)) <= 1e-12
    br = np.array(brute.brute_varlen(q, g["cu_seqlens"], kp, vp, bt, g["context_lens"],
                                     bs, 0.5))
    assert np.max(np.abs(br[:, 0] - exp)) <= 1e-12


def test_context_of_one_returns_v():
    case = W.random_case(21, B=4, lmin=1, lmax=1, D=16, kv_dtype="f32")
    kp, vp = pools_after_store(case)
    out = run_ref(case, kp, vp)
    G = case.Hq // case.Hkv
    for s in range(case.num_seqs):
        for h in range(case.Hq):
            assert np.array_equal(out[s, h], case.v_new[s, h // G].astype(np.float64))


def test_zero_query_gives_causal_prefix_mean():
    case = W.random_case(22, kind="varlen", B=4, D=8, kv_dtype="f32", lmax=50, nmax=12)
    case.q[:] = 0
    kp, vp = pools_after_store(case)
    out = run_ref(case, kp, vp)
    G = case.Hq // case.Hkv
    for s in range(case.num_seqs):
        a, b = case.cu_seqlens[s], case.cu_seqlens[s + 1]
        L = case.context_lens[s]
        V = ref.gather_seq(vp, case.block_tables[s], L)
        for i in range(b - a):
            p = L - (b - a) + i
            for h in range(case.Hq):
                exp = V[:p + 1, h // G].mean(axis=0)
                assert np.max(np.abs(out[a + i, h] - exp)) <= 1e-12


def test_constant_v_and_rows_sum_to_one():
    case = W.random_case(23, kind="varlen", B=3, D=8, kv_dtype="f32")
    kp, vp = pools_after_store(case)
    vp[:] = 2.5
    out = run_ref(case, kp, vp)
    assert np.max(np.abs(out - 2.5)) <= 1e-13
    s = 1
    L = case.context_lens[s]
    K = ref.gather_seq(kp, case.block_tables[s], L)
    V = ref.gather_seq(vp, case.block_tables[s], L)
    _, _, rs = ref.attend(np.ones((2, case.Hq, 8)), [0, L - 1], K, V, 0.3)
    assert np.max(np.abs(rs - 1.0)) <= 1e-13


def test_identical_keys_give_mean_v():
    case = W.random_case(24, B=3, D=8, kv_dtype="f32")
    kp, vp = pools_after_store(case)
    kp[:] = 0.37
    out = run_ref(case, kp, vp)
    G = case.Hq // case.Hkv
    for s in range(case.num_seqs):
        V = ref.gather_seq(vp, case.block_tables[s], case.context_lens[s])
        for h in range(case.Hq):
            assert np.max(np.abs(out[s, h] - V[:, h // G].mean(0))) <= 1e-12


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(25)
    L, D = 30, 16
    K = rng.standard_normal((L, 1, D))
    V = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((1, 1, D))
    K[17, 0] = 40.0 * q[0, 0] / np.linalg.norm(q[0, 0])   # score gap >> 50
    out, _, _ = ref.attend(q, [L - 1], K, V, 1.0 * np.linalg.norm(q[0, 0]) / 40.0 * 10)
    assert np.max(np.abs(out[0, 0] - V[17, 0])) < 1e-9


# ----------------------------------------------------------------------------- invariants

def test_block_permutation_invariance():
    case = W.random_case(31, kind="varlen", B=3, D=16, kv_dtype="f32")
    kp, vp = pools_after_store(case)
    out = run_ref(case, kp, vp)
    perm = np.random.default_rng(0).permutation(case.num_blocks)
    inv = np.argsort(perm)
    kp2, vp2 = kp[perm], vp[perm]          # new block b holds old block perm[b]
    bt2 = np.where(case.block_tables >= 0, inv[np.maximum(case.block_tables, 0)], -1)
    out2 = ref.varlen_ref(case.q, case.cu_seqlens, kp2, vp2, bt2, case.context_lens,
                          case.scale)[0]
    assert np.array_equal(out, out2)


def test_paged_equals_contiguous():
    rng = np.random.default_rng(32)
    B, Lmax, Hkv, Hq, D, bs = 3, 48, 2, 6, 16, 16
    lens = np.array([48, 17, 1], dtype=np.int32)
    Kc = rng.standard_normal((B, Lmax, Hkv, D))          # contiguous per-slot cache
    Vc = rng.standard_normal((B, Lmax, Hkv, D))
    q = rng.standard_normal((B, Hq, D))
    # contiguous: dense attention over the first L_s tokens of each slot
    exp = np.stack([ref.attend(q[s:s + 1], [lens[s] - 1], Kc[s, :lens[s]], Vc[s, :lens[s]],
                               0.25)[0][0] for s in range(B)])
    # the same caches viewed as 16-token blocks, identity placement, then permuted
    per = Lmax // bs
    kp = Kc.reshape(B * per, bs, Hkv, D)
    vp = Vc.reshape(B * per, bs, Hkv, D)
    bt = (np.arange(B)[:, None] * per + np.arange(per)[None]).astype(np.int32)
    out = ref.decode_ref(q, kp, vp, bt, lens, 0.25)[0]
    assert np.array_equal(out, exp)
    perm = rng.permutation(B * per)
    inv = np.argsort(perm)
    out2 = ref.decode_ref(q, kp[perm], vp[perm], inv[bt], lens, 0.25)[0]
    assert np.array_equal(out2, exp)


def test_key_shift_and_value_shift():
    case = W.random_case(33, kind="varlen", B=3, D=8, kv_dtype="f32")
    kp, vp = pools_after_store(case)
    out = run_ref(case, kp, vp)
    # adding one vector c to every key adds q.c to every score of a row: no change
    c = np.random.default_rng(1).standard_normal(8)
    out_k = run_ref(case, kp + c, vp)
    assert np.max(np.abs(out - out_k)) <= 1e-10
    out_v = run_ref(case, kp, vp + c)
    assert np.max(np.abs(out + c - out_v)) <= 1e-12


def test_gqa_equals_mha_with_repeated_kv_heads():
    case = W.random_case(34, kind="varlen", B=3, Hq=6, Hkv=2, D=8, kv_dtype="f32")
    kp, vp = pools_after_store(case)
    out = run_ref(case, kp, vp)
    G = case.Hq // case.Hkv
    kr, vr = np.repeat(kp, G, axis=2), np.repeat(vp, G, axis=2)   # head h -> kv h // G
    out_mha = ref.varlen_ref(case.q, case.cu_seqlens, kr, vr, case.block_tables,
                             case.context_lens, case.scale)[0]
    assert np.array_equal(out, out_mha)
    # and a different grouping (h % Hkv) gives a different answer on this input
    kt, vt = np.tile(kp, (1, 1, G, 1)), np.tile(vp, (1, 1, G, 1))
    out_bad = ref.varlen_ref(case.q, case.cu_seqlens, kt, vt, case.block_tables,
                             case.context_lens, case.scale)[0]
    assert np.max(np.abs(out_bad - out)) > 1e-3


def test_varlen_sequences_are_isolated():
    case = W.random_case(35, kind="varlen", B=3, D=8, kv_dtype="f32", lmin=10, nmax=8)
    kp, vp = pools_after_store(case)
    out = run_ref(case, kp, vp)
    # perturb everything of sequence 1 (its query rows and its blocks)
    q2 = case.q.copy()
    a, b = case.cu_seqlens[1], case.cu_seqlens[2]
    q2[a:b] += 1.0
    kp2, vp2 = kp.copy(), vp.copy()
    for blk in case.block_tables[1]:
        if blk >= 0:
            kp2[blk] += 3.0
            vp2[blk] -= 2.0
    out2 = ref.varlen_ref(q2, case.cu_seqlens, kp2, vp2, case.block_tables,
                          case.context_lens, case.scale)[0]
    keep = np.ones(len(q2), bool)
    keep[a:b] = False
    assert np.array_equal(out[keep], out2[keep])


def test_decode_equals_varlen_with_chunks_of_one():
    case = W.random_case(36, B=4, D=8, kv_dtype="f32")
    kp, vp = pools_after_store(case)
    dec = run_ref(case, kp, vp)
    cu = np.arange(case.num_seqs + 1, dtype=np.int32)
    var = ref.varlen_ref(case.q, cu, kp, vp, case.block_tables, case.context_lens,
                         case.scale)[0]
    assert np.array_equal(dec, var)


# ----------------------------------------------------------------------------- split merge

@pytest.mark.parametrize("cuts", [[0, 16, 37], [0, 1, 2, 37], [0, 36, 37], [0, 5, 5, 37]])
def test_merge_of_partials_equals_whole(cuts):
    case = W.make(1)
    kp, vp = pools_after_store(case)
    L = int(case.context_lens[0])
    K = ref.gather_seq(kp, case.block_tables[0], L)
    V = ref.gather_seq(vp, case.block_tables[0], L)
    whole, lse, _ = ref.attend(case.q, [L - 1], K, V, case.scale)
    parts = [ref.partial_ref(case.q, [L - 1], K, V, case.scale, a, b)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, l = ref.merge_ref([p[0] for p in parts], [p[1] for p in parts])
    assert np.max(np.abs(o - whole)) <= 1e-12
    assert np.max(np.abs(l - lse)) <= 1e-12
    # lse is log sum exp of the scores (brute definition)
    s = [case.scale * math.fsum(case.q[0, 0, d] * K[j, 0, d] for d in range(case.D))
         for j in range(L)]
    assert abs(lse[0, 0] - math.log(math.fsum(math.exp(x) for x in s))) <= 1e-12


# ----------------------------------------------------------------------------- store + inputs

def test_store_ref_places_rows_and_leaves_rest():
    case = W.random_case(41, kind="varlen", B=3, D=8, kv_dtype="bf16")
    pool = np.arange(case.num_blocks * 16 * case.Hkv * 8, dtype=np.uint16).reshape(
        case.num_blocks, 16, case.Hkv, 8)
    src = W.bf16_bits(case.k_new)
    sm = case.slot_mapping.copy()
    if len(sm) > 1:
        sm[1] = -1                                        # padding entry
    out = ref.store_ref(pool, src, sm)
    touched = np.zeros((case.num_blocks, 16), bool)
    for t, (s, p) in enumerate(zip(case.new_seq, case.new_pos)):
        slot = ref.slot_of(case.block_tables[s], p, 16)
        if sm[t] < 0:
            continue
        assert np.array_equal(out[slot // 16, slot % 16], src[t])
        touched[slot // 16, slot % 16] = True
    assert np.array_equal(out[~touched], pool[~touched])


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_generator_slots_match_block_tables(cfg):
    case = W.make(cfg)
    for t, (s, p) in enumerate(zip(case.new_seq, case.new_pos)):
        assert case.slot_mapping[t] == ref.slot_of(case.block_tables[s], p, 16)
    # distinct slots, inside the pool, and each new token is inside its context
    assert len(set(case.slot_mapping.tolist())) == len(case.slot_mapping)
    assert case.slot_mapping.min() >= 0
    assert case.slot_mapping.max() < case.num_blocks * 16
    assert np.all(case.new_pos < case.context_lens[case.new_seq])
    # blocks are not shared between sequences
    used = [b for s in range(case.num_seqs) for b in
            case.block_tables[s, :-(-int(case.context_lens[s]) // 16)]]
    assert len(set(used)) == len(used)


def test_config_shapes():
    c3 = W.make(3)
    n = np.diff(c3.cu_seqlens)
    assert c3.num_seqs == 16 and (n == 1).sum() == 4 and n.max() <= 512
    assert np.all(c3.context_lens - n <= 2048)
    c2 = W.make(2)
    assert c2.context_lens.min() >= 128 and c2.context_lens.max() <= 3200
    c4 = W.make(4)
    assert c4.num_seqs == 256 and c4.context_lens.min() >= 1024
    assert c4.context_lens.max() <= 32768


def test_fp8_store_ref_quantises_rows():
    case = W.random_case(42, B=3, D=16, kv_dtype="fp8")
    codes = np.zeros((case.num_blocks, 16, case.Hkv, 16), np.uint8)
    scales = np.zeros((case.num_blocks, 16, case.Hkv), np.float32)
    c2, s2 = ref.store_fp8_ref(codes, scales, case.k_new, case.slot_mapping)
    qc, qs = ofp8.quantize_rows(case.k_new)
    for t, slot in enumerate(case.slot_mapping):
        assert np.array_equal(c2[slot // 16, slot % 16], qc[t])
        assert np.array_equal(s2[slot // 16, slot % 16], qs[t])
