"""pa_decode_noalloc (the decode call whose scratch is the library's per-GPU array, for
callers that cannot allocate) against pa_decode with a caller workspace: bit-identical
outputs on consecutive calls, the second smaller than the first, on both schedules
(single launch and persistent split + merge) and on a quantised pool; a call needing
more scratch than the array holds is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_95_amd as pa
import workloads as W

from _harness import TOL, Setup, max_err

pytestmark = pytest.mark.gpu


def noalloc_abi(s, split, out):
    """The entry point called straight through the C ABI."""
    c = s.case
    q = s.q
    qs, os_ = (q.stride(0), q.stride(1)), (out.stride(0), out.stride(1))
    st = pa.lib().pa_decode_noalloc(
        ctypes.c_void_p(out.data_ptr()), os_[0], os_[1], ctypes.c_void_p(q.data_ptr()), qs[0],
        qs[1], pa._DTYPE_CODE[q.dtype], c.num_seqs, c.Hq, s.pool.struct,
        ctypes.c_void_p(s.bt.data_ptr()), c.max_blocks_per_seq,
        ctypes.c_void_p(s.ctx.data_ptr()), c.max_context_len, float(c.scale), int(split),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


# (first call, second call): the second is smaller (fewer sequences, shorter contexts)
CASES = {
    "single launch, bf16 G6": (dict(seed=81, B=8, Hq=12, Hkv=2, D=128, lmin=200, lmax=3000), 32,
                               dict(seed=82, B=3, Hq=12, Hkv=2, D=128, lmin=1, lmax=700), 32),
    "persistent, bf16 G4": (dict(seed=83, B=64, Hq=16, Hkv=4, D=128, lmin=100, lmax=4000), 64,
                            dict(seed=84, B=40, Hq=16, Hkv=4, D=128, lmin=1, lmax=2000), 64),
    "fp8 pool": (dict(seed=85, B=6, Hq=12, Hkv=2, D=128, kv_dtype="fp8", lmin=50, lmax=2000), 0,
                 dict(seed=86, B=2, Hq=12, Hkv=2, D=128, kv_dtype="fp8", lmin=1, lmax=300), 0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_workspace_decode(dev, name):
    kw1, split1, kw2, split2 = CASES[name]
    for kw, split in ((kw1, split1), (kw2, split2)):
        case = W.random_case(**kw)
        s = Setup(case, dev)
        assert pa.decode_workspace_bytes(case.num_seqs, case.Hq, case.Hkv, case.D,
                                         case.max_context_len, split) <= pa.NOALLOC_SCRATCH_BYTES
        ref_out = s.gpu(split_tokens=split)
        out = torch.full_like(ref_out, float("nan"))
        assert noalloc_abi(s, split, out) == pa.PA_OK
        torch.cuda.synchronize()
        print(f"{name} seed {kw['seed']}: B={case.num_seqs} max_ctx={case.max_context_len}",
              flush=True)
        assert torch.equal(out, ref_out)
        assert max_err(out, s.oracle()) <= TOL[case.kv_dtype]
        # the binding's wrapper of the same entry point
        out2 = pa.decode_noalloc(s.q, s.pool, s.bt, s.ctx, case.scale,
                                 max_context_len=case.max_context_len, split_tokens=split)
        assert torch.equal(out2, ref_out)


def test_noalloc_refuses_oversized_calls(dev):
    """256 sequences of up to 32768 tokens at split 32 need ~1 GiB of partials: refused
    on the host, nothing launched, the output untouched."""
    B, Hq, Hkv, D, maxctx = 256, 32, 8, 128, 32768
    need = pa.decode_workspace_bytes(B, Hq, Hkv, D, maxctx, 32)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    pool = pa.KVPool.empty(4, Hkv, D, "bf16", dev)
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, maxctx // 16), dtype=torch.int32, device=dev)
    ctx = torch.ones(B, dtype=torch.int32, device=dev)
    out = torch.full_like(q, 3.0)
    with pytest.raises(pa.PaError) as e:
        pa.decode_noalloc(q, pool, bt, ctx, 0.1, max_context_len=maxctx, split_tokens=32,
                          out=out)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
