"""Oracle-side test helpers: build the oracle's pool from a generated step and
compute reference outputs. Nothing here imports the library."""

from __future__ import annotations

import numpy as np

import oracle


def pool(step, with_new: bool = True) -> oracle.OraclePool:
    p = oracle.OraclePool(step.num_blocks, step.num_kv_heads, step.block_size, step.head_dim, step.kv_dtype)
    oracle.reshape_and_cache(p, step.prefix_k, step.prefix_v, step.src_dtype, step.prefix_slots)
    if with_new:
        oracle.reshape_and_cache(p, step.new_k, step.new_v, step.src_dtype, step.new_slots)
    return p


def pool_bytes(p: oracle.OraclePool) -> dict:
    out = {"k": p.k.tobytes(), "v": p.v.tobytes()}
    if p.k_scale is not None:
        out["k_scale"] = p.k_scale.tobytes()
        out["v_scale"] = p.v_scale.tobytes()
    return out


def decode(step, p, rows=None):
    q, tables, ctx, _ = step.decode_batch()
    return oracle.paged_decode(oracle.decode_rows(q, step.q_dtype), p, tables, ctx, step.scale, rows=rows)


def chunked(step, p):
    q, cu, tables, ctx = step.chunk_batch()
    return oracle.paged_chunked(oracle.decode_rows(q, step.q_dtype), cu, p, tables, ctx, step.scale)


ATOL, RTOL = 2e-3, 1e-2


def compare(got: np.ndarray, ref: np.ndarray, atol: float = ATOL, rtol: float = RTOL, mask=None) -> dict:
    """Element-wise |got - ref| <= atol + rtol |ref| (NaN only where ref is NaN
    is not allowed: ref must be finite where compared). Returns error stats."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    fin = np.isfinite(ref)
    inf_ok = np.array_equal(got[~fin], ref[~fin]) if (~fin).any() else True
    d = np.abs(got[fin] - ref[fin])
    ok = bool(inf_ok and np.isfinite(got[fin]).all() and (d <= atol + rtol * np.abs(ref[fin])).all())
    return {
        "ok": ok,
        "max_abs": float(d.max()) if d.size else 0.0,
        "max_rel": float((d / np.maximum(np.abs(ref[fin]), 1e-3)).max()) if d.size else 0.0,
        "n": int(d.size),
    }
