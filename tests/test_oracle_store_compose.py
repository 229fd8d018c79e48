"""Pins of the oracle's quantised and fused stores that do not reuse their own code
paths: rows are read back one token at a time through the block table (the brute
force's lookup, not the slot arithmetic of the store), and the fused RoPE store is
checked against angles whose rotation is exact (identity, quarter and half turns), so
the order rotate -> round / quantise -> store and the unrotated v are fixed by closed
forms."""
import numpy as np
import pytest

import workloads as W
from oracle import brute, fp8, int8, ref, rope


def _readback(pool, case, t, g):
    """Row of new token t, head g, found through its sequence's block table."""
    s, p = int(case.new_seq[t]), int(case.new_pos[t])
    return brute._row(pool, case.block_tables[s], 16, p, g)


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_quantised_store_places_each_row_at_its_token(kind):
    case = W.random_case(91, kind="varlen", B=4, Hq=4, Hkv=2, D=16, kv_dtype=kind, nmax=40)
    nb, hkv, D = case.num_blocks, case.Hkv, case.D
    dt = np.int8 if kind == "int8" else np.uint8
    codes0 = np.full((nb, 16, hkv, D), 0x55, dt)
    scales0 = np.full((nb, 16, hkv), -7.0, np.float32)
    x = case.k_new * np.random.default_rng(1).uniform(0.01, 100, (len(case.k_new), hkv, 1))
    x = x.astype(np.float32)
    sm = case.slot_mapping.copy()
    sm[2] = -1                                    # padding: nothing stored
    sm[3] = nb * 16 + 5                           # past the pool: nothing stored
    store = ref.store_int8_ref if kind == "int8" else ref.store_fp8_ref
    quant = int8.quantize_rows if kind == "int8" else fp8.quantize_rows
    c2, s2 = store(codes0, scales0, x, sm)
    touched = np.zeros((nb, 16), bool)
    for t in range(len(sm)):
        s, p = int(case.new_seq[t]), int(case.new_pos[t])
        blk = int(case.block_tables[s][p // 16])
        if t in (2, 3):
            assert np.array_equal(c2[blk, p % 16], codes0[blk, p % 16])
            continue
        touched[blk, p % 16] = True
        for g in range(hkv):
            qc, qs = quant(x[t, g][None])
            assert np.array_equal(_readback(c2, case, t, g), qc[0])
            assert _readback(s2, case, t, g) == qs[0]
    assert np.array_equal(c2[~touched], codes0[~touched])
    assert np.array_equal(s2[~touched], scales0[~touched])


def _turn_tables(D, P=3):
    """Position 0: identity; 1: quarter turn; 2: half turn (all exact)."""
    c = np.zeros((P, D // 2), np.float32)
    s = np.zeros((P, D // 2), np.float32)
    c[0], s[0] = 1.0, 0.0
    c[1], s[1] = 0.0, 1.0
    c[2], s[2] = -1.0, 0.0
    return c, s


def _closed_form(x, p):
    h = x.shape[-1] // 2
    if p == 0:
        return x
    if p == 1:
        return np.concatenate([-x[..., h:], x[..., :h]], axis=-1)
    return -x


@pytest.mark.parametrize("kind", ["bf16", "f32", "fp8", "int8"])
def test_rope_store_composition_closed_forms(kind):
    """k is rotated, then rounded / quantised, then stored; v is stored as it is; q is
    rotated for every token, padding included."""
    rng = np.random.default_rng(92)
    T, hq, hkv, D, nb = 9, 4, 2, 16, 4
    q = rng.standard_normal((T, hq, D)).astype(np.float32)
    k = rng.standard_normal((T, hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, hkv, D)).astype(np.float32)
    if kind != "f32":
        q, k, v = W.round_to_bf16(q), W.round_to_bf16(k), W.round_to_bf16(v)
    pos = np.arange(T, dtype=np.int64) % 3
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[4] = -1
    cos, sin = _turn_tables(D)
    if kind in ("bf16", "f32"):
        pk0 = np.full((nb, 16, hkv, D), 7.0)
        pv0 = np.full((nb, 16, hkv, D), 9.0)
        q_rot, pk, pv, _ = rope.rope_store_ref(kind, pk0, pv0, None, q, k, v, pos, cos, sin, slots)
    else:
        dt = np.int8 if kind == "int8" else np.uint8
        pk0 = np.zeros((nb, 16, hkv, D), dt)
        pv0 = np.zeros((nb, 16, hkv, D), dt)
        sc = (np.zeros((nb, 16, hkv), np.float32), np.zeros((nb, 16, hkv), np.float32))
        q_rot, pk, pv, (sk, sv) = rope.rope_store_ref(kind, pk0, pv0, sc, q, k, v, pos, cos,
                                                      sin, slots)
    quant = {"fp8": fp8.quantize_rows, "int8": int8.quantize_rows}.get(kind)
    for t in range(T):
        p = int(pos[t])
        assert np.array_equal(q_rot[t], _closed_form(q[t], p))       # padding too
        sl = int(slots[t])
        if sl < 0:
            continue
        kr = _closed_form(k[t], p)
        if quant is None:
            assert np.array_equal(pk[sl // 16, sl % 16], kr.astype(np.float64))
            assert np.array_equal(pv[sl // 16, sl % 16], v[t].astype(np.float64))
        else:
            ck, skk = quant(kr)
            cv, svv = quant(v[t])
            assert np.array_equal(pk[sl // 16, sl % 16], ck)
            assert np.array_equal(sk[sl // 16, sl % 16], skk)
            assert np.array_equal(pv[sl // 16, sl % 16], cv)
            assert np.array_equal(sv[sl // 16, sl % 16], svv)
    written = {int(x) for x in slots if x >= 0}
    for sl in range(nb * 16):
        if sl not in written:
            assert np.array_equal(pk[sl // 16, sl % 16], pk0[sl // 16, sl % 16])


def test_rope_store_bf16_rounds_after_rotating():
    """General angles: the stored k is the bf16 value nearest the exact rotation of k
    (within half a bf16 ulp of the float32 result, which is itself within 2^-23 of
    exact), so neither the unrotated k nor a rotation of an already rounded value
    passes."""
    rng = np.random.default_rng(93)
    T, hq, hkv, D, nb = 16, 2, 2, 64, 2
    q = W.round_to_bf16(rng.standard_normal((T, hq, D)).astype(np.float32))
    k = W.round_to_bf16(rng.standard_normal((T, hkv, D)).astype(np.float32))
    v = W.round_to_bf16(rng.standard_normal((T, hkv, D)).astype(np.float32))
    cos, sin = W.rope_tables(64, D)
    pos = rng.integers(1, 64, T)
    slots = np.arange(T, dtype=np.int64)
    _, pk, pv, _ = rope.rope_store_ref("bf16", np.zeros((nb, 16, hkv, D)),
                                       np.zeros((nb, 16, hkv, D)), None, q, k, v, pos, cos,
                                       sin, slots)
    h = D // 2
    c = cos[pos][:, None, :].astype(np.float64)
    s = sin[pos][:, None, :].astype(np.float64)
    a, b = k[..., :h].astype(np.float64), k[..., h:].astype(np.float64)
    exact = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    got = pk.reshape(nb * 16, hkv, D)[:T]
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    assert np.all(np.abs(got - exact) <= 0.5 * ulp + 2.0 ** -22 * np.abs(exact) + 1e-30)
    assert np.array_equal(W.round_to_bf16(got.astype(np.float32)), got.astype(np.float32))
    assert not np.array_equal(got, k.astype(np.float64))
    assert np.array_equal(pv.reshape(nb * 16, hkv, D)[:T], v.astype(np.float64))
