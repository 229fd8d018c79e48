"""pa_rope_store_kv on the GPU against oracle.rope: rotated q and the stored (rotated) k
and v are bit-exact for bf16 / fp32 / FP8 / INT8 pools; then a decode on the rotated q
matches the oracle's attention over the rotated cache."""
import numpy as np
import pytest
import torch

import paged_kv_cache_95_amd as pa
import workloads as W
from oracle import ref, rope

from _harness import TOL, Setup, max_err

pytestmark = pytest.mark.gpu

_TD = {"bf16": torch.bfloat16, "f32": torch.float32}


def _inputs(seed, T, Hq, Hkv, D, src, nb, maxp):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, Hq, D)).astype(np.float32) * 3
    k = rng.standard_normal((T, Hkv, D)).astype(np.float32) * 3
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    if src == "bf16":
        q, k, v = W.round_to_bf16(q), W.round_to_bf16(k), W.round_to_bf16(v)
    pos = rng.integers(0, maxp, T).astype(np.int64)
    pos[0] = 0                                          # identity row
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[3::7] = -1                                    # padding: nothing stored
    return q, k, v, pos, slots


@pytest.mark.parametrize("src,kind,D,Hq,Hkv", [
    ("bf16", "bf16", 128, 12, 2), ("bf16", "bf16", 64, 8, 8), ("f32", "f32", 64, 4, 2),
    ("bf16", "fp8", 128, 12, 2), ("bf16", "int8", 64, 6, 3), ("f32", "fp8", 64, 4, 1)])
def test_rope_store_bitexact(dev, src, kind, D, Hq, Hkv):
    T, nb, maxp = 70, 12, 4096
    q, k, v, pos, slots = _inputs(D + Hq, T, Hq, Hkv, D, src, nb, maxp)
    cos, sin = W.rope_tables(maxp, D)
    shape = (nb, 16, Hkv, D)
    td = _TD[src]
    if kind in ("bf16", "f32"):
        init = np.random.default_rng(9).standard_normal(shape).astype(np.float32)
        init = W.round_to_bf16(init) if kind == "bf16" else init
        pool = pa.KVPool(torch.from_numpy(init).to(td).to(dev),
                         torch.from_numpy(-init).to(td).to(dev))
        ref_k, ref_v, sc = init.astype(np.float64), -init.astype(np.float64), None
    else:
        pool = pa.KVPool.empty(nb, Hkv, D, kind, dev)
        fill = 0x55 if kind == "fp8" else -55
        for t in (pool.k, pool.v):
            t.fill_(fill)
        for t in (pool.k_scale, pool.v_scale):
            t.fill_(-3.0)
        ref_k = np.full(shape, fill, np.uint8 if kind == "fp8" else np.int8)
        ref_v = ref_k.copy()
        sc = (np.full(shape[:3], -3.0, np.float32), np.full(shape[:3], -3.0, np.float32))
    to = lambda a: torch.from_numpy(a).to(td).to(dev)
    q_out = pa.rope_store_kv(pool, to(q), to(k), to(v), torch.from_numpy(pos).to(dev),
                             torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev),
                             torch.from_numpy(slots).to(dev))
    torch.cuda.synchronize()
    q_rot, pk, pv, psc = rope.rope_store_ref(kind, ref_k, ref_v, sc, q, k, v, pos, cos, sin,
                                             slots)
    expect_q = rope.bf16_round(q_rot) if src == "bf16" else q_rot
    assert np.array_equal(q_out.float().cpu().numpy().view(np.uint32), expect_q.view(np.uint32))
    if kind in ("bf16", "f32"):
        for got, exp in ((pool.k, pk), (pool.v, pv)):
            assert np.array_equal(got.float().cpu().numpy().view(np.uint32),
                                  exp.astype(np.float32).view(np.uint32))
    else:
        assert np.array_equal(pool.k.cpu().numpy(), pk)
        assert np.array_equal(pool.v.cpu().numpy(), pv)
        assert np.array_equal(pool.k_scale.cpu().numpy().view(np.uint32), psc[0].view(np.uint32))
        assert np.array_equal(pool.v_scale.cpu().numpy().view(np.uint32), psc[1].view(np.uint32))


def test_in_place_and_strided_q(dev):
    T, Hq, Hkv, D, nb, maxp = 33, 6, 2, 128, 8, 512
    q, k, v, pos, slots = _inputs(5, T, Hq, Hkv, D, "bf16", nb, maxp)
    cos, sin = W.rope_tables(maxp, D)
    qbuf = torch.zeros((T, Hq + 2, D), dtype=torch.bfloat16, device=dev)
    qbuf[:, 1:Hq + 1] = torch.from_numpy(q).to(torch.bfloat16)
    qv = qbuf[:, 1:Hq + 1]                               # strided view, rotated in place
    pool = pa.KVPool.empty(nb, Hkv, D, "bf16", dev)
    out = pa.rope_store_kv(pool, qv, torch.from_numpy(k).to(torch.bfloat16).to(dev),
                           torch.from_numpy(v).to(torch.bfloat16).to(dev),
                           torch.from_numpy(pos).to(dev), torch.from_numpy(cos).to(dev),
                           torch.from_numpy(sin).to(dev), torch.from_numpy(slots).to(dev),
                           q_out=qv)
    torch.cuda.synchronize()
    assert out.data_ptr() == qv.data_ptr()
    expect = rope.bf16_round(rope.rotate(q, pos, cos, sin))
    assert np.array_equal(qbuf[:, 1:Hq + 1].float().cpu().numpy(), expect)
    assert not qbuf[:, 0].any() and not qbuf[:, Hq + 1].any()   # neighbours untouched


def test_rotated_decode_matches_oracle(dev):
    """The step as the pages' engine runs it: rotate q and k of the new token and store
    k and v (one launch), then decode with the rotated q."""
    case = W.random_case(71, B=6, Hq=12, Hkv=2, D=128, lmin=1, lmax=900)
    s = Setup(case, dev, store_new=False)
    cos, sin = W.rope_tables(1024, 128)
    pos = case.new_pos.astype(np.int64)
    q_rot = pa.rope_store_kv(s.pool, s.q, s.k_new, s.v_new, torch.from_numpy(pos).to(dev),
                             torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev),
                             s.slots)
    out = pa.decode(q_rot, s.pool, s.bt, s.ctx, case.scale, max_context_len=case.max_context_len)
    torch.cuda.synchronize()
    kp = W.host_pool(case, "k", True).astype(np.float64)
    vp = W.host_pool(case, "v", True).astype(np.float64)
    k_rot = rope.bf16_round(rope.rotate(case.k_new, pos, cos, sin)).astype(np.float64)
    rk = ref.store_ref(kp, k_rot, case.slot_mapping)
    rv = ref.store_ref(vp, case.v_new.astype(np.float64), case.slot_mapping)
    qr = rope.bf16_round(rope.rotate(case.q, pos, cos, sin))
    expect = ref.decode_ref(qr, rk, rv, case.block_tables, case.context_lens, case.scale)[0]
    err = max_err(out, expect)
    print(f"rotated decode max_abs_err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    # and the unrotated query is measurably not what was asked for
    assert max_err(pa.decode(s.q, s.pool, s.bt, s.ctx, case.scale,
                             max_context_len=case.max_context_len), expect) > TOL["bf16"]
