"""The PA_DEBUG_CHECKS build (libpa_debug.so) on the GPU: calls whose device-side
metadata breaks the contract are reported, not silently skipped.

Each case runs one call with deliberately bad metadata (a block id outside the pool
inside a context, a context length of 0 or past the bound, a slot past the pool, a
decode-step slot that is not the new token's, a varlen chunk longer than its context,
a decreasing cu_seqlens, a RoPE position past the table). Every kernel still runs in
bounds and exits normally: the release kernels skip or clamp such values, which is
exactly why a debug build is needed to see them. The next call then fails with
PA_ERR_DEVICE_DATA without launching, pa_debug_take_violation names the violation and
where it happened, and after taking it calls succeed again. A clean call records
nothing, and results of the debug build equal the release build's bit for bit."""
import numpy as np
import pytest
import torch

import paged_kv_cache_95_amd as pa
import workloads as W

from _harness import TOL, Setup, max_err

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_lib(dev):
    release = pa.lib()
    out = torch.empty(1, device=dev)                  # the stream exists
    del out
    pa.use_library(pa.DEBUG_LIB_PATH)
    try:
        assert pa.debug_checks()
        pa.take_violation()                           # nothing left from elsewhere
        yield
        pa.take_violation()
    finally:
        pa.use_library_handle(release)
    assert not pa.debug_checks()


def decode_case(seed=3, **kw):
    args = dict(B=4, Hq=12, Hkv=2, D=128, lmin=40, lmax=300)
    args.update(kw)
    return W.random_case(seed, **args)


def expect_violation(name, where=None):
    """The next call is refused; the violation is then taken and cleared."""
    got = pa.take_violation()
    assert got[0] == name, got
    if where is not None:
        assert got[2] == where, got
    assert pa.take_violation() == (None, 0, 0)


def test_clean_calls_record_nothing_and_match_release(dev, debug_lib):
    s = Setup(decode_case(), dev)
    out = s.gpu()
    assert pa.take_violation() == (None, 0, 0)
    assert max_err(out, s.oracle()) <= TOL["bf16"]
    prev = pa.use_library(pa.LIB_PATH)
    try:
        out_release = s.gpu()
    finally:
        pa.use_library_handle(prev)
    assert torch.equal(out, out_release)


def test_block_id_outside_the_pool(dev, debug_lib):
    case = decode_case()
    s = Setup(case, dev)
    bt = case.block_tables.copy()
    j = int(case.context_lens[2] - 1) // 16          # the last block of sequence 2
    bt[2, j] = case.num_blocks + 7
    pa.decode(s.q, s.pool, torch.from_numpy(bt).to(dev), s.ctx, case.scale,
              max_context_len=case.max_context_len)
    with pytest.raises(pa.PaError) as e:              # refused, nothing launched
        s.gpu()
    assert e.value.status == pa.PA_ERR_DEVICE_DATA
    expect_violation("block_id", (2 << 28) | j)
    s.gpu()                                           # taken: calls run again
    assert pa.take_violation() == (None, 0, 0)
    bt[2, j] = -3                                     # negative ids too
    pa.decode(s.q, s.pool, torch.from_numpy(bt).to(dev), s.ctx, case.scale,
              max_context_len=case.max_context_len)
    expect_violation("block_id", (2 << 28) | j)


@pytest.mark.parametrize("bad", [0, -4, "past"])
def test_context_length_out_of_range(dev, debug_lib, bad):
    case = decode_case()
    s = Setup(case, dev)
    ctx = case.context_lens.copy()
    ctx[1] = case.max_context_len + 16 if bad == "past" else bad
    pa.decode(s.q, s.pool, s.bt, torch.from_numpy(ctx).to(dev), case.scale,
              max_context_len=case.max_context_len)
    expect_violation("context_len", 1)


def test_store_slot_past_the_pool(dev, debug_lib):
    case = decode_case()
    s = Setup(case, dev, store_new=False)
    sl = case.slot_mapping.copy()
    sl[3] = case.num_blocks * 16 + 2
    sl[0] = -1                                        # padding: legal
    pa.store_kv(s.pool, s.k_new, s.v_new, torch.from_numpy(sl).to(dev))
    expect_violation("slot", 3)


def test_store_slot_named_twice(dev, debug_lib):
    case = decode_case()
    s = Setup(case, dev, store_new=False)
    sl = case.slot_mapping.copy()
    sl[0] = sl[1] = -1                                # padding twice: legal
    pa.store_kv(s.pool, s.k_new, s.v_new, torch.from_numpy(sl).to(dev))
    assert pa.take_violation()[1] == 0
    sl[3] = sl[2]                                     # two rows into one slot: they race
    pa.store_kv(s.pool, s.k_new, s.v_new, torch.from_numpy(sl).to(dev))
    name, code, where = pa.take_violation()
    assert name == "dup_slot" and where in (2, 3), (name, code, where)


def test_decode_step_slot_not_the_new_tokens(dev, debug_lib):
    case = decode_case()
    s = Setup(case, dev, store_new=False)
    sl = case.slot_mapping.copy()
    sl[1] = sl[1] - 1 if sl[1] % 16 else sl[1] + 1    # a slot in the pool, the wrong one
    pa.decode_step(s.q, s.pool, s.k_new, s.v_new, torch.from_numpy(sl).to(dev), s.bt, s.ctx,
                   case.scale, max_context_len=case.max_context_len)
    expect_violation("step_slot", 1)
    # the right slots (and -1 padding) are clean
    sl = case.slot_mapping.copy()
    sl[2] = -1
    pa.decode_step(s.q, s.pool, s.k_new, s.v_new, torch.from_numpy(sl).to(dev), s.bt, s.ctx,
                   case.scale, max_context_len=case.max_context_len)
    assert pa.take_violation() == (None, 0, 0)


def test_varlen_chunk_longer_than_context_and_bad_cu_seqlens(dev, debug_lib):
    case = W.random_case(5, kind="varlen", B=4, Hq=6, Hkv=2, D=128, lmin=10, lmax=200, nmax=40)
    s = Setup(case, dev)
    n = np.diff(case.cu_seqlens)
    b = int(np.argmax(n))
    ctx = case.context_lens.copy()
    ctx[b] = n[b] - 1                                 # chunk longer than its context
    pa.varlen_prefill(s.q, s.cu, s.pool, s.bt, torch.from_numpy(ctx).to(dev), case.scale,
                      max_q_len=case.max_q_len, max_context_len=case.max_context_len)
    expect_violation("chunk", b)
    cu = case.cu_seqlens.copy()
    cu[2] = cu[1] - 1                                 # decreasing boundary
    pa.varlen_prefill(s.q, torch.from_numpy(cu).to(dev), s.pool, s.bt, s.ctx, case.scale,
                      max_q_len=case.max_q_len, max_context_len=case.max_context_len)
    got = pa.take_violation()
    assert got[0] == "cu_seqlens" and got[2] in (1, 2), got
    s.gpu()
    assert pa.take_violation() == (None, 0, 0)


def test_rope_position_past_the_table(dev, debug_lib):
    case = decode_case()
    s = Setup(case, dev, store_new=False)
    cos, sin = W.rope_tables(400, case.D)
    pos = case.new_pos.copy()
    pos[2] = 400
    pa.rope_store_kv(s.pool, s.q, s.k_new, s.v_new, torch.from_numpy(pos).to(dev),
                     torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev), s.slots)
    expect_violation("position", 2)
