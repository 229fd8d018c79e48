"""pa_decode_step (store this step's rows, then attend) on the GPU: bit-identical to
pa_store_kv followed by pa_decode on every path (store folded into the single decode
launch, FP8 quantise-on-store launch, persistent schedule, unaligned rows, padding
slots), within tolerance of the oracle, and stable under graph replay."""
import numpy as np
import pytest
import torch

import paged_kv_cache_95_amd as pa
import workloads as W

from _harness import TOL, Setup, max_err

pytestmark = pytest.mark.gpu

_BITS = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.uint8: torch.uint8}


def same_bits(x, y):
    """Bitwise equality (NaN-poisoned slots compare equal to themselves)."""
    return torch.equal(x.view(_BITS[x.dtype]), y.view(_BITS[y.dtype]))


def same_pools(p, r):
    ok = same_bits(p.k, r.k) and same_bits(p.v, r.v)
    if p.k_scale is not None:
        ok = ok and same_bits(p.k_scale, r.k_scale) and same_bits(p.v_scale, r.v_scale)
    return ok


def run_both(case, dev, split, k_new=None, v_new=None, slots=None):
    """(decode_step output, its setup, store+decode output, its setup) on twin pools."""
    a = Setup(case, dev, store_new=False)
    b = Setup(case, dev, store_new=False)
    kn = a.k_new if k_new is None else k_new
    vn = a.v_new if v_new is None else v_new
    sl = a.slots if slots is None else slots
    out_a = pa.decode_step(a.q, a.pool, kn, vn, sl, a.bt, a.ctx, case.scale,
                           max_context_len=case.max_context_len, split_tokens=split)
    pa.store_kv(b.pool, kn, vn, sl)
    out_b = pa.decode(b.q, b.pool, b.bt, b.ctx, case.scale,
                      max_context_len=case.max_context_len, split_tokens=split)
    torch.cuda.synchronize()
    return out_a, a, out_b, b


CASES = {
    "bf16 folded": (dict(seed=61, B=8, Hq=12, Hkv=2, D=128, kv_dtype="bf16", lmax=2000), 32),
    "bf16 folded one group": (dict(seed=65, B=5, Hq=8, Hkv=2, D=64, kv_dtype="bf16", lmax=100), 16),
    "f32 folded": (dict(seed=62, B=3, Hq=4, Hkv=2, D=64, kv_dtype="f32", lmax=300), 16),
    "fp8 store launch": (dict(seed=63, B=5, Hq=12, Hkv=2, D=128, kv_dtype="fp8", lmax=900), 32),
    "bf16 persistent": (dict(seed=64, B=40, Hq=16, Hkv=4, D=128, kv_dtype="bf16", lmax=3000), 16),
}


@pytest.mark.parametrize("name", list(CASES))
def test_step_equals_store_then_decode(dev, name):
    kw, split = CASES[name]
    case = W.random_case(**kw)
    out_a, a, out_b, b = run_both(case, dev, split)
    assert torch.equal(out_a, out_b)
    assert same_pools(a.pool, b.pool)
    err = max_err(out_a, a.oracle())
    print(f"{name}: max_abs_err={err:.3e}", flush=True)
    assert err <= TOL[case.kv_dtype]


def test_unaligned_rows_take_the_store_launch(dev):
    case = W.random_case(66, B=6, Hq=12, Hkv=2, D=128, lmax=700)
    a0 = Setup(case, dev, store_new=False)
    # rows shifted by one element: not 16-byte aligned, same values
    kb = torch.zeros((6, 2, 129), dtype=torch.bfloat16, device=dev)
    vb = torch.zeros_like(kb)
    kb[:, :, 1:] = a0.k_new
    vb[:, :, 1:] = a0.v_new
    out_a, a, out_b, b = run_both(case, dev, 32, k_new=kb[:, :, 1:], v_new=vb[:, :, 1:])
    assert torch.equal(out_a, out_b)
    assert same_pools(a.pool, b.pool)
    assert max_err(out_a, a.oracle()) <= TOL["bf16"]


def test_padding_slots_store_nothing(dev):
    """Sequences with slot -1 store nothing and attend the pool as it is; the others
    store and use their new row."""
    case = W.random_case(67, B=8, Hq=12, Hkv=2, D=128, lmax=1500)
    sl = torch.from_numpy(case.slot_mapping.copy()).to(dev)
    sl[::3] = -1
    out_a, a, out_b, b = run_both(case, dev, 32, slots=sl)
    assert torch.equal(out_a, out_b)
    assert same_pools(a.pool, b.pool)


def test_step_graph_replay(dev):
    case = W.random_case(68, B=6, Hq=12, Hkv=2, D=128, lmin=50, lmax=2500)
    s = Setup(case, dev, store_new=False)
    ws = pa.decode_workspace(6, 12, 2, 128, 2500, 32, device=dev)
    out = torch.empty_like(s.q)

    def step():
        pa.decode_step(s.q, s.pool, s.k_new, s.v_new, s.slots, s.bt, s.ctx, case.scale,
                       max_context_len=2500, split_tokens=32, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    assert max_err(eager, s.oracle()) <= TOL["bf16"]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.zero_()
        junk = torch.randn(1000, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        del junk
