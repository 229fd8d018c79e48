"""Paged GQA attention over a block-table KV cache for AMD MI355X (gfx950).

Thin Python binding of libpa.so (C ABI declared in include/pa.h). It only marshals
arguments: checks dtypes, devices and shapes of torch tensors, passes their data
pointers, element strides and torch's current HIP stream, and raises on a non-zero
status. Every step of the computation runs in the HIP kernels of the library; there
is no fallback. PyTorch is used for device memory and streams only.

    pool = KVPool.empty(num_blocks, kv_heads, head_dim, "bf16", device)
    store_kv(pool, k_new, v_new, slot_mapping)
    out = decode(q, pool, block_tables, context_lens, scale)
    out = varlen_prefill(q, cu_seqlens, pool, block_tables, context_lens, scale)
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")
# the same library built with PA_DEBUG_CHECKS (device-data contract checks; see pa.h)
DEBUG_LIB_PATH = os.path.join(_HERE, "libpa_debug.so")

PA_F32, PA_BF16, PA_FP8_E4M3, PA_INT8 = 0, 1, 2, 3
PA_OK = 0
PA_ERR_DEVICE_DATA = -5
BLOCK_SIZE = 16
# contract violations a PA_DEBUG_CHECKS build records (pa.h)
VIOLATIONS = {1: "context_len", 2: "block_id", 3: "slot", 4: "chunk", 5: "cu_seqlens",
              6: "step_slot", 7: "position", 8: "dup_slot"}
# bytes of the per-GPU scratch array behind decode_noalloc (PA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

_DTYPE_CODE = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8_E4M3,
               torch.int8: PA_INT8}
_NAME_CODE = {"f32": PA_F32, "bf16": PA_BF16, "fp8": PA_FP8_E4M3, "int8": PA_INT8}
_NAME_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8,
               "int8": torch.int8}
_QUANT = (PA_FP8_E4M3, PA_INT8)


class PaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


class _Pool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_lib = None

# name -> (restype, argtypes); mirrors include/pa.h
_P, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_debug_checks": (_I32, []),
    "pa_debug_take_violation": (ctypes.c_int, [_P, _P, _P]),
    "pa_decode_default_split_tokens": (_I32, [_I32, _I32, _I32]),
    "pa_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "pa_store_kv": (ctypes.c_int, [ctypes.POINTER(_Pool), _P, _P, _I32, _I64, _I64, _I64, _I64,
                                   _I64, _P, _P]),
    "pa_decode": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _I64, _I32, _I32, _I32,
                                 ctypes.POINTER(_Pool), _P, _I32, _P, _I32, _F, _I32, _P, _SZ,
                                 _P]),
    "pa_rope_store_kv": (ctypes.c_int, [ctypes.POINTER(_Pool), _P, _I64, _I64, _I32, _P, _I64,
                                        _I64, _P, _P, _I32, _I64, _I64, _I64, _I64, _I64, _P,
                                        _P, _P, _I32, _P, _P]),
    "pa_copy_blocks": (ctypes.c_int, [ctypes.POINTER(_Pool), _P, _P, _I32, _P]),
    "pa_bm_create": (_P, [_I64, _I32, _I32]),
    "pa_bm_destroy": (None, [_P]),
    "pa_bm_num_free_blocks": (_I64, [_P]),
    "pa_bm_add_sequence": (ctypes.c_int, [_P, _I64, _P, _I64, _P]),
    "pa_bm_append_token": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P]),
    "pa_bm_fork": (ctypes.c_int, [_P, _I64, _I64]),
    "pa_bm_free_sequence": (ctypes.c_int, [_P, _I64]),
    "pa_bm_context_len": (_I64, [_P, _I64]),
    "pa_bm_block_tables": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P]),
    "pa_bm_slots": (ctypes.c_int, [_P, _I64, _I64, _I64, _P]),
    "pa_bm_block_refcount": (_I32, [_P, _I32]),
    "pa_decode_step": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _I64, _I32, _I32, _I32,
                                      ctypes.POINTER(_Pool), _P, _P, _I32, _I64, _I64, _I64,
                                      _I64, _P, _P, _I32, _P, _I32, _F, _I32, _P, _SZ, _P]),
    "pa_decode_noalloc": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _I64, _I32, _I32, _I32,
                                         ctypes.POINTER(_Pool), _P, _I32, _P, _I32, _F, _I32,
                                         _P]),
    "pa_varlen_prefill_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32]),
    "pa_varlen_prefill": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _I64, _I32, _P, _I32, _I64,
                                         _I32, _I32, ctypes.POINTER(_Pool), _P, _I32, _P, _I32,
                                         _F, _I32, _P, _SZ, _P]),
}


def _load(path):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m paged_kv_cache_95_amd.build`")
    l = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(l, name)
        fn.restype = res
        fn.argtypes = args
    return l


def lib():
    """Load libpa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def use_library(path):
    """Make every call of this module go through the library at `path` (e.g.
    DEBUG_LIB_PATH) from now on; returns the one used so far, to restore it with
    use_library_handle()."""
    global _lib
    prev = lib()
    _lib = _load(path)
    return prev


def use_library_handle(handle):
    global _lib
    _lib = handle


def debug_checks():
    """True when the loaded library is the PA_DEBUG_CHECKS build."""
    return bool(lib().pa_debug_checks())


def take_violation():
    """Wait for the current stream, then return and clear the GPU's recorded contract
    violation as (name, code, where); (None, 0, 0) when there is none."""
    code, where = ctypes.c_int32(0), ctypes.c_int64(0)
    _check(lib().pa_debug_take_violation(_stream(), ctypes.byref(code), ctypes.byref(where)),
           "pa_debug_take_violation")
    return VIOLATIONS.get(code.value), int(code.value), int(where.value)


def status_string(status):
    return lib().pa_status_string(int(status)).decode()


def default_split_tokens(num_seqs, kv_heads, max_context_len):
    """Split length decode() uses for split_tokens=0 at this call shape."""
    return int(lib().pa_decode_default_split_tokens(num_seqs, kv_heads, max_context_len))


def _check(status, what):
    if status != PA_OK:
        raise PaError(status, what)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


class KVPool:
    """One layer's paged KV cache: k, v [num_blocks, 16, kv_heads, head_dim] (bf16,
    fp32, uint8 e4m3fn codes or int8 codes) and, for FP8 / INT8, fp32 k_scale/v_scale
    [num_blocks, 16, kv_heads]. Tensors are owned by the caller (this object)."""

    def __init__(self, k, v, k_scale=None, v_scale=None, dtype=None):
        _need(k.shape == v.shape and k.dim() == 4, "k/v pools must be 4-D and equal")
        _need(k.is_contiguous() and v.is_contiguous(), "pools must be dense")
        self.k, self.v, self.k_scale, self.v_scale = k, v, k_scale, v_scale
        self.dtype = _DTYPE_CODE[k.dtype] if dtype is None else _NAME_CODE[dtype]
        if self.dtype in _QUANT:
            _need(k_scale is not None and v_scale is not None, "FP8/INT8 pool needs scales")
            _need(k_scale.dtype == torch.float32 and k_scale.shape == k.shape[:3]
                  and k_scale.is_contiguous() and v_scale.is_contiguous()
                  and v_scale.shape == k.shape[:3], "scales must be fp32 [nb, bs, Hkv]")
        _need(all(t.device == k.device for t in (v, k_scale, v_scale) if t is not None),
              "pool tensors must be on one device")
        self.num_blocks, self.block_size, self.kv_heads, self.head_dim = k.shape
        self._struct = _Pool(k.data_ptr(), v.data_ptr(),
                             k_scale.data_ptr() if k_scale is not None else 0,
                             v_scale.data_ptr() if v_scale is not None else 0,
                             self.num_blocks, self.block_size, self.kv_heads, self.head_dim,
                             self.dtype)

    @classmethod
    def empty(cls, num_blocks, kv_heads, head_dim, dtype, device, block_size=BLOCK_SIZE):
        shape = (num_blocks, block_size, kv_heads, head_dim)
        td = _NAME_TORCH[dtype]
        k = torch.empty(shape, dtype=td, device=device)
        v = torch.empty(shape, dtype=td, device=device)
        ks = vs = None
        if dtype in ("fp8", "int8"):
            ks = torch.empty(shape[:3], dtype=torch.float32, device=device)
            vs = torch.empty(shape[:3], dtype=torch.float32, device=device)
        return cls(k, v, ks, vs, dtype=dtype)

    @property
    def struct(self):
        return ctypes.byref(self._struct)


def _rows3(x, name):
    """Element strides (token, head) of a [T, H, D] view with unit inner stride."""
    _need(x.dim() == 3, f"{name} must be [tokens, heads, head_dim]")
    _need(x.stride(2) == 1, f"{name} needs a unit innermost stride")
    return x.stride(0), x.stride(1)


def store_kv(pool, k, v, slot_mapping):
    """Write new rows k, v [T, kv_heads, head_dim] (any token/head strides) into the
    pool at slot_mapping [T] (int64; negative = skip). FP8 pools quantise on store."""
    ks = _rows3(k, "k")
    vs = _rows3(v, "v")
    _need(k.shape == v.shape and k.shape[1:] == (pool.kv_heads, pool.head_dim), "k/v shape")
    _need(k.dtype == v.dtype, "k/v dtype")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1
          and slot_mapping.shape[0] == k.shape[0] and slot_mapping.is_contiguous(),
          "slot_mapping must be contiguous int64 [T]")
    _one_device(k, v, slot_mapping, pool.k)
    _check(lib().pa_store_kv(pool.struct, _ptr(k), _ptr(v), _DTYPE_CODE[k.dtype], k.shape[0],
                             ks[0], ks[1], vs[0], vs[1], _ptr(slot_mapping), _stream()),
           "pa_store_kv")


def rope_store_kv(pool, q, k, v, positions, cos_table, sin_table, slot_mapping, q_out=None):
    """Rotary position embedding of q [T, Hq, D] and k [T, kv_heads, D] by the table rows
    positions [T] (int64) of cos_table / sin_table (fp32 [max_position, D/2]; pair i
    with i + D/2), fused with the store of the rotated k and of v at slot_mapping [T].
    Returns the rotated q (q_out, which may be q itself for an in-place rotation)."""
    qs, ks, vs = _rows3(q, "q"), _rows3(k, "k"), _rows3(v, "v")
    T = q.shape[0]
    _need(k.shape == v.shape and k.shape == (T, pool.kv_heads, pool.head_dim), "k/v shape")
    _need(q.shape[2] == pool.head_dim and q.dtype == k.dtype == v.dtype, "q/k/v dtype or shape")
    for t, name in ((positions, "positions"), (slot_mapping, "slot_mapping")):
        _need(t.dtype == torch.int64 and t.dim() == 1 and t.shape[0] == T and t.is_contiguous(),
              f"{name} must be contiguous int64 [T]")
    half = pool.head_dim // 2
    for t, name in ((cos_table, "cos_table"), (sin_table, "sin_table")):
        _need(t.dtype == torch.float32 and t.dim() == 2 and t.shape[1] == half
              and t.is_contiguous(), f"{name} must be contiguous fp32 [max_position, D/2]")
    _need(cos_table.shape == sin_table.shape, "cos/sin tables differ in shape")
    if q_out is None:
        q_out = torch.empty((T,) + tuple(q.shape[1:]), dtype=q.dtype, device=q.device)
    qo = _rows3(q_out, "q_out")
    _need(tuple(q_out.shape) == tuple(q.shape) and q_out.dtype == q.dtype,
          "q_out must have q's shape and dtype")
    _one_device(q, q_out, k, v, positions, cos_table, sin_table, slot_mapping, pool.k)
    _check(lib().pa_rope_store_kv(pool.struct, _ptr(q), qs[0], qs[1], q.shape[1], _ptr(q_out),
                                  qo[0], qo[1], _ptr(k), _ptr(v), _DTYPE_CODE[k.dtype], T, ks[0],
                                  ks[1], vs[0], vs[1], _ptr(positions), _ptr(cos_table),
                                  _ptr(sin_table), cos_table.shape[0], _ptr(slot_mapping),
                                  _stream()),
           "pa_rope_store_kv")
    return q_out


def copy_blocks(pool, src_blocks, dst_blocks):
    """Device copy of pool blocks src_blocks[i] -> dst_blocks[i] (int32 device tensors),
    K, V and (FP8 / INT8) scales: the copy-on-write of BlockManager.append()."""
    for t in (src_blocks, dst_blocks):
        _need(t.dtype == torch.int32 and t.dim() == 1 and t.is_contiguous(),
              "block lists must be contiguous int32 [n]")
    _need(src_blocks.shape == dst_blocks.shape, "src/dst lengths differ")
    _one_device(src_blocks, dst_blocks, pool.k)
    _check(lib().pa_copy_blocks(pool.struct, _ptr(src_blocks), _ptr(dst_blocks),
                                src_blocks.shape[0], _stream()), "pa_copy_blocks")


class BlockManager:
    """Host block manager of one pool (C++ in libpa.so): sequences, their block tables,
    prefix sharing of full blocks and copy-on-write (policy documented in pa.h)."""

    def __init__(self, num_blocks, block_size=BLOCK_SIZE, prefix_caching=True):
        self._h = lib().pa_bm_create(num_blocks, block_size, 1 if prefix_caching else 0)
        if not self._h:
            raise ValueError("invalid block manager arguments")
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.pa_bm_destroy(h)
            self._h = None

    @property
    def num_free(self):
        return int(lib().pa_bm_num_free_blocks(self._h))

    def add_sequence(self, seq_id, token_ids):
        """Register a sequence with its prompt; returns the number of leading tokens
        whose blocks were reused from the prefix cache."""
        t = np.ascontiguousarray(token_ids, dtype=np.int32)
        cached = ctypes.c_int64(0)
        _check(lib().pa_bm_add_sequence(self._h, seq_id, t.ctypes.data_as(ctypes.c_void_p),
                                        t.size, ctypes.byref(cached)), "pa_bm_add_sequence")
        return int(cached.value)

    def append(self, seq_id, token_id):
        """Extend by one token: (slot, copy_src, copy_dst), copy_* = -1 unless the last
        block had to be copied (copy-on-write)."""
        slot, cs, cd = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().pa_bm_append_token(self._h, seq_id, int(token_id), ctypes.byref(slot),
                                        ctypes.byref(cs), ctypes.byref(cd)), "pa_bm_append_token")
        return int(slot.value), int(cs.value), int(cd.value)

    def fork(self, parent_id, child_id):
        _check(lib().pa_bm_fork(self._h, parent_id, child_id), "pa_bm_fork")

    def free(self, seq_id):
        _check(lib().pa_bm_free_sequence(self._h, seq_id), "pa_bm_free_sequence")

    def context_len(self, seq_id):
        return int(lib().pa_bm_context_len(self._h, seq_id))

    def block_tables(self, seq_ids, max_blocks_per_seq):
        """(block_tables int32 [n, max_blocks] -1 padded, context_lens int32 [n])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        bt = np.empty((ids.size, max_blocks_per_seq), dtype=np.int32)
        cl = np.empty(ids.size, dtype=np.int32)
        _check(lib().pa_bm_block_tables(self._h, ids.ctypes.data_as(ctypes.c_void_p), ids.size,
                                        max_blocks_per_seq, bt.ctypes.data_as(ctypes.c_void_p),
                                        cl.ctypes.data_as(ctypes.c_void_p)), "pa_bm_block_tables")
        return bt, cl

    def slots(self, seq_id, first_pos, count):
        out = np.empty(count, dtype=np.int64)
        _check(lib().pa_bm_slots(self._h, seq_id, first_pos, count,
                                 out.ctypes.data_as(ctypes.c_void_p)), "pa_bm_slots")
        return out

    def refcount(self, block):
        return int(lib().pa_bm_block_refcount(self._h, block))


def decode_workspace_bytes(num_seqs, q_heads, kv_heads, head_dim, max_context_len,
                           split_tokens=0):
    return int(lib().pa_decode_workspace_bytes(num_seqs, q_heads, kv_heads, head_dim,
                                               max_context_len, split_tokens))


def decode_workspace(num_seqs, q_heads, kv_heads, head_dim, max_context_len, split_tokens=0,
                     device="cuda"):
    """A workspace for decode() calls of these sizes (and split length), zero-filled as
    pa_decode requires before first use (its arrival counters); calls leave it reusable."""
    need = decode_workspace_bytes(num_seqs, q_heads, kv_heads, head_dim, max_context_len,
                                  split_tokens)
    return torch.zeros(max(need, 1), dtype=torch.uint8, device=device)


def _meta(block_tables, context_lens, num_seqs):
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.is_contiguous(), "block_tables must be contiguous int32 [B, maxb]")
    _need(context_lens.dtype == torch.int32 and context_lens.dim() == 1
          and context_lens.is_contiguous(), "context_lens must be contiguous int32 [B]")
    _need(block_tables.shape[0] >= num_seqs,
          f"block_tables has {block_tables.shape[0]} rows for {num_seqs} sequences")
    _need(context_lens.shape[0] >= num_seqs,
          f"context_lens has {context_lens.shape[0]} entries for {num_seqs} sequences")


def _rows_like(q, out, pool, name="out"):
    """q [N, Hq, head_dim] of the pool's head_dim; out of q's shape and dtype."""
    _need(q.dim() == 3 and q.shape[2] == pool.head_dim,
          f"q must be [tokens, q_heads, {pool.head_dim}] (the pool's head_dim)")
    _need(tuple(out.shape) == tuple(q.shape), f"{name} must have q's shape {tuple(q.shape)}")
    _need(out.dtype == q.dtype, f"{name} must have q's dtype {q.dtype}")


def _one_device(*tensors):
    """Every tensor argument of a kernel call lives on the same GPU (and so does the
    pool): the kernels take raw device pointers."""
    devs = {t.device for t in tensors if t is not None}
    _need(len(devs) == 1 and next(iter(devs)).type == "cuda",
          f"all tensors must be on one CUDA device (got {sorted(map(str, devs))})")


def decode(q, pool, block_tables, context_lens, scale, max_context_len=None, split_tokens=0,
           out=None, workspace=None):
    """Paged decode: q [B, Hq, D] (strided views allowed) -> out [B, Hq, D].
    max_context_len: host-side bound of context_lens (default: the block table's
    capacity; no device sync). workspace: optional preallocated uint8 tensor, zero-filled
    before its first use (decode_workspace()); reusing one keeps the call allocation-free."""
    qs = _rows3(q, "q")
    B, Hq, D = q.shape
    _meta(block_tables, context_lens, B)
    if max_context_len is None:
        max_context_len = block_tables.shape[1] * pool.block_size
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    os_ = _rows3(out, "out")
    _rows_like(q, out, pool)
    _one_device(q, out, block_tables, context_lens, workspace, pool.k)
    need = decode_workspace_bytes(B, Hq, pool.kv_heads, D, max_context_len, split_tokens)
    if need and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_decode(_ptr(out), os_[0], os_[1], _ptr(q), qs[0], qs[1], _DTYPE_CODE[q.dtype],
                           B, Hq, pool.struct, _ptr(block_tables), block_tables.shape[1],
                           _ptr(context_lens), int(max_context_len), float(scale),
                           int(split_tokens), _ptr(workspace), wbytes, _stream()),
           "pa_decode")
    return out


def decode_noalloc(q, pool, block_tables, context_lens, scale, max_context_len=None,
                   split_tokens=0, out=None):
    """decode() without a workspace: the library's per-GPU scratch array holds the split
    partials, so the call allocates nothing on the device (pass `out` to keep this
    function from allocating it). Calls that could overlap on one GPU must not be made.
    Raises PaError (PA_ERR_WORKSPACE) when the call needs more than
    NOALLOC_SCRATCH_BYTES of workspace."""
    qs = _rows3(q, "q")
    B, Hq, D = q.shape
    _meta(block_tables, context_lens, B)
    if max_context_len is None:
        max_context_len = block_tables.shape[1] * pool.block_size
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    os_ = _rows3(out, "out")
    _rows_like(q, out, pool)
    _one_device(q, out, block_tables, context_lens, pool.k)
    _check(lib().pa_decode_noalloc(_ptr(out), os_[0], os_[1], _ptr(q), qs[0], qs[1],
                                   _DTYPE_CODE[q.dtype], B, Hq, pool.struct, _ptr(block_tables),
                                   block_tables.shape[1], _ptr(context_lens),
                                   int(max_context_len), float(scale), int(split_tokens),
                                   _stream()),
           "pa_decode_noalloc")
    return out


def decode_step(q, pool, k_new, v_new, slot_mapping, block_tables, context_lens, scale,
                max_context_len=None, split_tokens=0, out=None, workspace=None):
    """One decode step: store row s of k_new / v_new [B, kv_heads, head_dim] at
    slot_mapping[s] (int64; negative = no new token), then attend as decode(); the same
    result as store_kv() followed by decode(), in one launch for small batches."""
    qs = _rows3(q, "q")
    B, Hq, D = q.shape
    _meta(block_tables, context_lens, B)
    ks, vs = _rows3(k_new, "k_new"), _rows3(v_new, "v_new")
    _need(k_new.shape == v_new.shape and k_new.shape == (B, pool.kv_heads, pool.head_dim),
          "k_new/v_new shape [B, kv_heads, head_dim]")
    _need(k_new.dtype == v_new.dtype, "k_new/v_new dtype")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1
          and slot_mapping.shape[0] == B and slot_mapping.is_contiguous(),
          "slot_mapping must be contiguous int64 [B]")
    if max_context_len is None:
        max_context_len = block_tables.shape[1] * pool.block_size
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    os_ = _rows3(out, "out")
    _rows_like(q, out, pool)
    _one_device(q, out, k_new, v_new, slot_mapping, block_tables, context_lens, workspace, pool.k)
    need = decode_workspace_bytes(B, Hq, pool.kv_heads, D, max_context_len, split_tokens)
    if need and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_decode_step(_ptr(out), os_[0], os_[1], _ptr(q), qs[0], qs[1],
                                _DTYPE_CODE[q.dtype], B, Hq, pool.struct, _ptr(k_new),
                                _ptr(v_new), _DTYPE_CODE[k_new.dtype], ks[0], ks[1], vs[0],
                                vs[1], _ptr(slot_mapping), _ptr(block_tables),
                                block_tables.shape[1], _ptr(context_lens), int(max_context_len),
                                float(scale), int(split_tokens), _ptr(workspace), wbytes,
                                _stream()),
           "pa_decode_step")
    return out


def varlen_prefill_workspace_bytes(total_tokens, q_heads, head_dim, max_context_len,
                                   split_tokens=0):
    return int(lib().pa_varlen_prefill_workspace_bytes(total_tokens, q_heads, head_dim,
                                                       max_context_len, split_tokens))


def varlen_prefill_workspace(total_tokens, q_heads, head_dim, max_context_len, split_tokens=0,
                             device="cuda"):
    """A workspace for varlen_prefill() calls of these sizes (and split length)."""
    need = varlen_prefill_workspace_bytes(total_tokens, q_heads, head_dim, max_context_len,
                                          split_tokens)
    return torch.empty(max(need, 1), dtype=torch.uint8, device=device)


def varlen_prefill(q, cu_seqlens, pool, block_tables, context_lens, scale, max_q_len=None,
                   max_context_len=None, split_tokens=0, out=None, workspace=None):
    """Varlen causal prefill: q [T, Hq, D] with chunks cu_seqlens [B+1] -> out [T, Hq, D].
    split_tokens: keys per work item (0 = library default); workspace: optional
    preallocated uint8 tensor (varlen_prefill_workspace())."""
    _need(cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1
          and cu_seqlens.is_contiguous() and cu_seqlens.shape[0] >= 1,
          "cu_seqlens must be contiguous int32 [B+1]")
    qs = _rows3(q, "q")
    T, Hq, D = q.shape
    B = cu_seqlens.shape[0] - 1
    _meta(block_tables, context_lens, B)
    if max_context_len is None:
        max_context_len = block_tables.shape[1] * pool.block_size
    if max_q_len is None:
        max_q_len = min(T, max_context_len)
    if out is None:
        out = torch.empty((T, Hq, D), dtype=q.dtype, device=q.device)
    os_ = _rows3(out, "out")
    _rows_like(q, out, pool)
    _one_device(q, out, cu_seqlens, block_tables, context_lens, workspace, pool.k)
    need = varlen_prefill_workspace_bytes(T, Hq, D, max_context_len, split_tokens)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_varlen_prefill(_ptr(out), os_[0], os_[1], _ptr(q), qs[0], qs[1],
                                   _DTYPE_CODE[q.dtype], _ptr(cu_seqlens), B, T, int(max_q_len),
                                   Hq, pool.struct, _ptr(block_tables), block_tables.shape[1],
                                   _ptr(context_lens), int(max_context_len), float(scale),
                                   int(split_tokens), _ptr(workspace), wbytes, _stream()),
           "pa_varlen_prefill")
    return out
