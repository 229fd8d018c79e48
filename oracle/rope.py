"""Rotary position embedding and the fused RoPE + KV store (oracle; test infrastructure).

What is computed follows the fused RoPE + KV-cache store of the koas-w "errors and
solutions" post ("hand-written Triton kernels") with its table-driven real-valued RoPE,
aligned with the HuggingFace model (milestone log): dim i of a head is paired with dim
i + D/2 and the pair is rotated by the angle whose cosine and sine are table[p][i] for
the token's position p. Reading taken here (the pages give no precision): the rotation
runs in float32 from the exact float32 values of the inputs, each product and each sum
rounded on its own,
    r_i = x_i c_i - x_{i+D/2} s_i,    r_{i+D/2} = x_{i+D/2} c_i + x_i s_i,
and the rotated rows are then rounded (q, and k in a bf16 pool) or quantised (k in an
FP8 / INT8 pool) exactly as a stored source row would be.

Pinned by the -m "not gpu" tests: the identity at angle 0, a quarter turn giving
(-x_{i+D/2}, x_i) (this fixes the pairing and the sign), a half turn giving -x, the
relative-position property of rotated dot products, composition of angles, and the
float64 error bound of the float32 arithmetic.
"""
import numpy as np


def rotate(x, positions, cos_table, sin_table):
    """float32 [T, H, D] rotated rows of x (float32 [T, H, D]) for positions [T]."""
    x = np.asarray(x, dtype=np.float32)
    half = x.shape[-1] // 2
    c = np.asarray(cos_table, dtype=np.float32)[np.asarray(positions, dtype=np.int64)][:, None, :]
    s = np.asarray(sin_table, dtype=np.float32)[np.asarray(positions, dtype=np.int64)][:, None, :]
    a, b = x[..., :half], x[..., half:]
    lo = (a * c).astype(np.float32) - (b * s).astype(np.float32)
    hi = (b * c).astype(np.float32) + (a * s).astype(np.float32)
    return np.concatenate([lo, hi], axis=-1).astype(np.float32)


def bf16_round(x):
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(np.shape(x))


def rope_store_ref(kind, pool_k, pool_v, scales, q, k, v, positions, cos_table, sin_table,
                   slot_mapping):
    """The fused op on host arrays.

    kind: "f32" | "bf16" | "fp8" | "int8" (pool type); q, k, v: float32 source values
    (exact bf16 values when the source is bf16). pool_k / pool_v: value pools for
    f32 / bf16 ([nb, bs, Hkv, D] float32), code pools for fp8 / int8; scales: (k_scale,
    v_scale) float32 [nb, bs, Hkv] for fp8 / int8, else None.
    Returns (q_rot float32 [T, Hq, D] before rounding to the source dtype, pool_k, pool_v,
    scales) after the store."""
    from . import ref
    q_rot = rotate(q, positions, cos_table, sin_table)
    k_rot = rotate(k, positions, cos_table, sin_table)
    if kind in ("f32", "bf16"):
        rk = k_rot if kind == "f32" else bf16_round(k_rot)
        pk = ref.store_ref(pool_k, rk.astype(np.float64), slot_mapping)
        pv = ref.store_ref(pool_v, np.asarray(v, dtype=np.float64), slot_mapping)
        return q_rot, pk, pv, None
    store = ref.store_fp8_ref if kind == "fp8" else ref.store_int8_ref
    ck, sk = store(pool_k, scales[0], k_rot, slot_mapping)
    cv, sv = store(pool_v, scales[1], np.asarray(v, dtype=np.float32), slot_mapping)
    return q_rot, ck, cv, (sk, sv)
