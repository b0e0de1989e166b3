"""GPU-side test helpers: move a generated step to the device and run it
through the library's C ABI (via the Python binding). Nothing here imports
the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_attention_19_amd as pkv

CODE = {"f32": pkv.F32, "bf16": pkv.BF16, "i8": pkv.I8, "fp8": pkv.FP8}


def announce(msg: str) -> None:
    """Name the case on stderr before a GPU step (visible with pytest -s)."""
    sys.stderr.write(f"[gpu] {msg}\n")
    sys.stderr.flush()


def tensor(a: np.ndarray, dtype: str, dev) -> torch.Tensor:
    """Storage array -> device tensor (bf16 arrives as uint16 bit patterns)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(dev)


def ints(a, dev, dtype=torch.int32) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(dev)


def build_cache(step, dev, with_new: bool = True) -> pkv.KVCache:
    """Allocate the pool (NaN-filled) and write the prefix rows, then the new rows,
    with the library's reshape_and_cache."""
    cache = pkv.KVCache.allocate(step.num_blocks, step.num_kv_heads, step.head_dim, CODE[step.kv_dtype], dev,
                                 block_size=step.block_size)
    if len(step.prefix_slots):
        pkv.reshape_and_cache(tensor(step.prefix_k, step.src_dtype, dev), tensor(step.prefix_v, step.src_dtype, dev),
                              ints(step.prefix_slots, dev, torch.int64), cache)
    if with_new and len(step.new_slots):
        pkv.reshape_and_cache(tensor(step.new_k, step.src_dtype, dev), tensor(step.new_v, step.src_dtype, dev),
                              ints(step.new_slots, dev, torch.int64), cache)
    return cache


def cache_bytes(cache: pkv.KVCache) -> dict:
    out = {"k": cache.k.cpu().view(torch.uint8).numpy().tobytes(), "v": cache.v.cpu().view(torch.uint8).numpy().tobytes()}
    if cache.k_scale is not None:
        out["k_scale"] = cache.k_scale.cpu().numpy().tobytes()
        out["v_scale"] = cache.v_scale.cpu().numpy().tobytes()
    return out


def run_decode(step, cache, dev, num_splits=None, max_num_splits=None):
    """Decode rows of ``step`` -> (out, lse) numpy float32."""
    q, tables, ctx, ns = step.decode_batch()
    if num_splits is not None:
        ns = np.broadcast_to(np.asarray(num_splits, np.int32), ns.shape).copy()
    mx = int(max_num_splits or max(1, int(ns.max())))
    announce(f"decode {step.name} B={len(ctx)} Hq={step.num_q_heads} Hkv={step.num_kv_heads} "
             f"D={step.head_dim} kv={step.kv_dtype} max_ns={mx}")
    out, lse = pkv.paged_attention_decode(tensor(q, step.q_dtype, dev), cache, ints(tables, dev), ints(ctx, dev),
                                          ints(ns, dev), mx, float(step.scale), return_lse=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def run_chunked(step, cache, dev):
    q, cu, tables, ctx = step.chunk_batch()
    announce(f"chunked {step.name} S={len(ctx)} rows={len(q)} kv={step.kv_dtype}")
    out, lse = pkv.paged_attention_chunked(tensor(q, step.q_dtype, dev), ints(cu, dev), int(np.diff(cu).max()), cache,
                                           ints(tables, dev), ints(ctx, dev), float(step.scale), return_lse=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()
