"""The Python binding rejects mismatched tensor arguments before any launch (CPU only).

The kernels index block_tables, context_lens, q and out with the sizes the call
states (B sequences, the pool's head_dim), so a too-short table, a head_dim that is
not the pool's, an output of another shape or dtype, or tensors on different devices
would make them read or write outside those buffers. Each case below must raise
ValueError in the binding. CPU tensors reach the device check last, so a call whose
shapes are all right still raises (nothing is ever handed to the library here)."""
import pytest
import torch

import paged_kv_cache_95_amd as pa

B, HQ, HKV, D = 4, 6, 2, 128
bf = torch.bfloat16


def pool(d=D):
    return pa.KVPool.empty(8, HKV, d, "bf16", "cpu")


def args():
    return dict(q=torch.zeros((B, HQ, D), dtype=bf),
                block_tables=torch.zeros((B, 3), dtype=torch.int32),
                context_lens=torch.ones(B, dtype=torch.int32))


def decode(**over):
    a = {**args(), **over}
    p = a.pop("pool", pool())
    return pa.decode(a.pop("q"), p, a.pop("block_tables"), a.pop("context_lens"), 0.1, **a)


def step(**over):
    a = {**args(), "k_new": torch.zeros((B, HKV, D), dtype=bf),
         "v_new": torch.zeros((B, HKV, D), dtype=bf),
         "slot_mapping": torch.zeros(B, dtype=torch.int64), **over}
    p = a.pop("pool", pool())
    return pa.decode_step(a.pop("q"), p, a.pop("k_new"), a.pop("v_new"), a.pop("slot_mapping"),
                          a.pop("block_tables"), a.pop("context_lens"), 0.1, **a)


def prefill(**over):
    a = {**args(), "cu_seqlens": torch.tensor([0, 1, 2, 3, 4], dtype=torch.int32), **over}
    p = a.pop("pool", pool())
    return pa.varlen_prefill(a.pop("q"), a.pop("cu_seqlens"), p, a.pop("block_tables"),
                             a.pop("context_lens"), 0.1, **a)


BAD = {   # name: (arguments, what the error must name)
    "short block_tables": (dict(block_tables=torch.zeros((B - 1, 3), dtype=torch.int32)),
                           "block_tables has 3 rows"),
    "short context_lens": (dict(context_lens=torch.ones(B - 1, dtype=torch.int32)),
                           "context_lens has 3 entries"),
    "head_dim not the pool's": (dict(pool=pool(64)), "head_dim"),
    "q head_dim not the pool's": (dict(q=torch.zeros((B, HQ, 64), dtype=bf)), "head_dim"),
    "out of another shape": (dict(out=torch.zeros((B, HQ + 1, D), dtype=bf)), "q's shape"),
    "out of another token count": (dict(out=torch.zeros((B + 1, HQ, D), dtype=bf)), "q's shape"),
    "out of another dtype": (dict(out=torch.zeros((B, HQ, D), dtype=torch.float32)), "q's dtype"),
    "tensors on two devices": (dict(context_lens=torch.ones(B, dtype=torch.int32, device="meta")),
                               "one CUDA device"),
    "host tensors": ({}, "one CUDA device"),
}


@pytest.mark.parametrize("call", [decode, step, prefill], ids=["decode", "decode_step", "prefill"])
@pytest.mark.parametrize("name", list(BAD))
def test_mismatch_raises_before_launch(call, name):
    kw, what = BAD[name]
    with pytest.raises(ValueError, match=what):
        call(**kw)


def test_decode_step_row_shapes():
    with pytest.raises(ValueError, match="k_new/v_new shape"):
        step(k_new=torch.zeros((B - 1, HKV, D), dtype=bf))
    with pytest.raises(ValueError, match="slot_mapping"):
        step(slot_mapping=torch.zeros(B + 1, dtype=torch.int64))


def test_prefill_short_cu_seqlens_rows():
    # 5 sequences by cu_seqlens, 4 table rows
    with pytest.raises(ValueError, match="block_tables has 4 rows for 5"):
        prefill(cu_seqlens=torch.tensor([0, 1, 2, 3, 4, 4], dtype=torch.int32))


def test_store_and_pool_devices():
    p = pool()
    k = torch.zeros((3, HKV, D), dtype=bf)
    with pytest.raises(ValueError, match="one CUDA device"):
        pa.store_kv(p, k, k, torch.zeros(3, dtype=torch.int64))      # host tensors
    with pytest.raises(ValueError, match="one device"):
        pa.KVPool(torch.zeros((8, 16, HKV, D), dtype=bf),
                  torch.zeros((8, 16, HKV, D), dtype=bf, device="meta"))
