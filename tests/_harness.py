"""Shared helpers for the GPU parity tests: build device pools from a workloads.Case,
run the HIP path through the binding, and run the oracle on the same inputs.

The oracle side never sees a value produced by the HIP path: bf16/fp32 pools start from
the generator's values and get the new rows via oracle.ref.store_ref; FP8 / INT8 pools
are filled by oracle.ref.store_fp8_ref / store_int8_ref from the same bf16 source the
GPU store consumes.
"""
import numpy as np
import torch

import paged_kv_cache_95_amd as pa
import workloads as W
from oracle import fp8 as ofp8
from oracle import int8 as oint8
from oracle import ref

# INT8 pools run the FP8 arithmetic (codes exact in bf16, probabilities rounded once
# to bf16 for P.V), so they take the FP8 bound.
TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 3e-2, "int8": 3e-2}
NAN_CODE = 0x7F  # e4m3fn NaN pattern, used to poison unused FP8 slots


def to_dev(x, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype).to(dev)


class Setup:
    """Device and oracle state of one case after this step's store (the oracle side
    always includes it; store_new=False leaves the device store to the test)."""

    def __init__(self, case, dev, poison=True, split_tokens=0, store_new=True):
        self.case, self.dev = case, dev
        self.split_tokens = split_tokens
        c = case
        td = {"f32": torch.float32, "bf16": torch.bfloat16}[c.src_dtype]
        self.bt = torch.from_numpy(c.block_tables).to(dev)
        self.ctx = torch.from_numpy(c.context_lens).to(dev)
        self.q = to_dev(c.q, td, dev)
        self.k_new = to_dev(c.k_new, td, dev)
        self.v_new = to_dev(c.v_new, td, dev)
        self.slots = torch.from_numpy(c.slot_mapping).to(dev)
        self.cu = torch.from_numpy(c.cu_seqlens).to(dev) if c.cu_seqlens is not None else None
        if c.kv_dtype in ("fp8", "int8"):
            self._setup_quant(poison)
        else:
            kp = W.host_pool(c, "k", poison)
            vp = W.host_pool(c, "v", poison)
            self.pool = pa.KVPool(to_dev(kp, td, dev), to_dev(vp, td, dev))
            self.ref_k = ref.store_ref(kp.astype(np.float64), c.k_new.astype(np.float64),
                                       c.slot_mapping)
            self.ref_v = ref.store_ref(vp.astype(np.float64), c.v_new.astype(np.float64),
                                       c.slot_mapping)
        if store_new:   # else the caller stores this step's rows (e.g. decode_step)
            pa.store_kv(self.pool, self.k_new, self.v_new, self.slots)

    def _setup_quant(self, poison):
        c, dev = self.case, self.dev
        int8 = c.kv_dtype == "int8"
        shape = (c.num_blocks, c.block_size, c.Hkv, c.D)
        # unused slots: NaN codes for FP8; INT8 has none, so a garbage code with a NaN
        # scale (the scales carry the poison there)
        fill = (-77 if int8 else NAN_CODE) if poison else 0
        codes_k = np.full(shape, fill, np.int8 if int8 else np.uint8)
        codes_v = np.full(shape, fill, np.int8 if int8 else np.uint8)
        sk = np.full(shape[:3], np.nan if poison else 0, np.float32)
        sv = sk.copy()
        self.pool = pa.KVPool(torch.from_numpy(codes_k).to(dev), torch.from_numpy(codes_v).to(dev),
                              torch.from_numpy(sk).to(dev), torch.from_numpy(sv).to(dev))
        # prefix rows: one bf16 source row per (seq, pos), stored by both sides
        _, _, pslots, pk, pv = W.prefix_tokens(c)
        if len(pslots):
            pa.store_kv(self.pool, to_dev(pk, torch.bfloat16, dev), to_dev(pv, torch.bfloat16, dev),
                        torch.from_numpy(pslots).to(dev))
        all_slots = np.concatenate([pslots, c.slot_mapping])
        store = ref.store_int8_ref if int8 else ref.store_fp8_ref
        ck, sk2 = store(codes_k, sk, np.concatenate([pk, c.k_new]), all_slots)
        cv, sv2 = store(codes_v, sv, np.concatenate([pv, c.v_new]), all_slots)
        self.ref_codes = (ck, sk2, cv, sv2)
        self.ref_k = self._dequant(ck, sk2, int8)
        self.ref_v = self._dequant(cv, sv2, int8)

    @staticmethod
    def _dequant(codes, scales, int8=False):
        if int8:
            return oint8.dequantize(codes, scales)
        return ofp8.decode(codes) * scales.astype(np.float64)[..., None]

    # ------------------------------------------------------------------ runs
    def gpu(self, **kw):
        c = self.case
        if c.kind == "decode":
            return pa.decode(self.q, self.pool, self.bt, self.ctx, c.scale,
                             max_context_len=kw.pop("max_context_len", c.max_context_len),
                             split_tokens=kw.pop("split_tokens", self.split_tokens), **kw)
        return pa.varlen_prefill(self.q, self.cu, self.pool, self.bt, self.ctx, c.scale,
                                 max_q_len=kw.pop("max_q_len", c.max_q_len),
                                 max_context_len=kw.pop("max_context_len", c.max_context_len),
                                 split_tokens=kw.pop("split_tokens", self.split_tokens), **kw)

    def oracle(self, seqs=None):
        c = self.case
        if c.kind == "decode":
            if seqs is None:
                return ref.decode_ref(c.q, self.ref_k, self.ref_v, c.block_tables,
                                      c.context_lens, c.scale)[0]
            return ref.decode_ref(c.q[seqs], self.ref_k, self.ref_v, c.block_tables[seqs],
                                  c.context_lens[seqs], c.scale)[0]
        return ref.varlen_ref(c.q, c.cu_seqlens, self.ref_k, self.ref_v, c.block_tables,
                              c.context_lens, c.scale)[0]


def bf16_rounding_excess(expect):
    """Per element, how far bf16's own rounding of the exact value can exceed 2^-7, the
    half spacing of bf16 on [2, 4): 0 below magnitude 4, 2^-7 on [4, 8), 2^-7 * 3 on
    [8, 16), ... A bf16 output cannot be closer to an exact value of magnitude >= 4
    than half the spacing there (2^-6 and up), more than the 1e-2 bar, so that part
    is allowed on top of the bar; below 4 the bar applies unchanged."""
    e = np.abs(np.asarray(expect, np.float64))
    _, x = np.frexp(e)                       # e = m * 2^x, m in [0.5, 1)
    half = np.ldexp(1.0, x - 9)              # half the bf16 spacing at e
    return np.maximum(half - 2.0 ** -7, 0.0) * (e > 0)


def max_err(gpu_out, expect):
    """Max abs error of a GPU output against the oracle. For bf16 outputs the part of
    each element's error that bf16 rounding forces above magnitude 4 is subtracted
    (bf16_rounding_excess), so the result compares with the bars as written."""
    g = gpu_out.float().cpu().numpy().astype(np.float64)
    assert g.shape == expect.shape, (g.shape, expect.shape)
    assert np.all(np.isfinite(g)), "non-finite output"
    if not g.size:
        return 0.0
    err = np.abs(g - expect)
    if gpu_out.dtype == torch.bfloat16:
        err = np.maximum(err - bf16_rounding_excess(expect), 0.0)
    return float(np.max(err))
