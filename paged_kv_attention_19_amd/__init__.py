"""Paged-KV attention for AMD MI355X (gfx950): Python binding of ``libpkv.so``.

Every step of the computation runs in the HIP kernels of ``libpkv.so``
(``include/pkv.h`` is the C ABI). This module only marshals arguments: it
checks tensors' dtype, shape, contiguity and device, allocates outputs with
torch when the caller gives none, and passes raw device pointers and the
current HIP stream to the C entry points. There is no CPU fallback: if the
library is missing, or the tensors are not on a GPU, the calls raise.

Names follow the C ABI: :func:`reshape_and_cache`,
:func:`paged_attention_decode`, :func:`paged_attention_decode_append`,
:func:`paged_attention_chunked`, :func:`lse_combine`,
:func:`decode_workspace_bytes`.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

__all__ = [
    "F32", "BF16", "I8", "FP8", "PkvError", "KVCache", "lib", "library_path", "exported_symbols",
    "reshape_and_cache", "decode_workspace_bytes", "decode_default_max_num_splits", "paged_attention_decode",
    "paged_attention_decode_append", "paged_attention_decode_noalloc", "paged_attention_chunked", "lse_combine",
    "version", "NOALLOC_SCRATCH_BYTES", "stream_read", "chunked_kernel_for", "CHUNKED_DECODE_ROWS",
    "CHUNKED_ROWS_MFMA", "CHUNKED_TILES",
]

F32, BF16, I8, FP8 = 0, 1, 2, 3
NOALLOC_SCRATCH_BYTES = 48 << 20   # PKV_NOALLOC_SCRATCH_BYTES of the C header
# kernels of the chunked entry point (PKV_CHUNKED_* of the C header)
CHUNKED_DECODE_ROWS, CHUNKED_ROWS_MFMA, CHUNKED_TILES = 1, 2, 3
_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16, I8: torch.int8, FP8: torch.float8_e4m3fn}
_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8, torch.float8_e4m3fn: FP8}
_SCALED = (I8, FP8)   # 8-bit codes with a float32 scale per (token, kv head)

_HERE = os.path.dirname(os.path.abspath(__file__))
_INCLUDE = os.path.join(os.path.dirname(_HERE), "include")


def library_path() -> str:
    return os.path.join(_HERE, "libpkv.so")


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pkv status {status}: {message}")
        self.status = status


class _Cache(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


_LIB = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "pkv_last_error": ([], ctypes.c_char_p),
    "pkv_version": ([], ctypes.c_char_p),
    "pkv_reshape_and_cache": ([_P, _P, _I32, _P, _I32, ctypes.POINTER(_Cache), _P], _I32),
    "pkv_decode_workspace_bytes": ([_I32, _I32, _I32, _I32], ctypes.c_size_t),
    "pkv_decode_default_max_num_splits": ([_I32], _I32),
    "pkv_chunked_kernel_for": ([_I32, _I32, _I32, _I32], _I32),
    "pkv_paged_attention_decode": ([_P, _I32, _I32, _I32, ctypes.POINTER(_Cache), _P, _I32, _P, _P, _I32,
                                    ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P], _I32),
    "pkv_paged_attention_decode_append": ([_P, _P, _I32, _P, _P, _I32, _I32, _I32, ctypes.POINTER(_Cache), _P, _I32,
                                           _P, _P, _I32, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P], _I32),
    "pkv_paged_attention_decode_noalloc": ([_P, _I32, _I32, _I32, ctypes.POINTER(_Cache), _P, _I32, _P, _P, _I32,
                                            ctypes.c_float, _P, _P, _P], _I32),
    "pkv_paged_attention_chunked": ([_P, _I32, _I32, _I32, _P, _I32, ctypes.POINTER(_Cache), _P, _I32, _P,
                                     ctypes.c_float, _P, _P, _P], _I32),
    "pkv_lse_combine": ([_P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P], _I32),
    "pkv_stream_read": ([_P, ctypes.c_size_t, _P, _P], _I32),
    "pkv_stream_read_workgroups": ([ctypes.c_size_t], _I32),
}


def lib():
    """Load ``libpkv.so`` (built in-tree by ``paged_kv_attention_19_amd.build``)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m paged_kv_attention_19_amd.build`")
        L = ctypes.CDLL(path)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = L
    return _LIB


def exported_symbols() -> list[str]:
    """Function names the public headers (``include/*.h``) declare."""
    names = set()
    for h in sorted(os.listdir(_INCLUDE)):
        if h.endswith(".h"):
            with open(os.path.join(_INCLUDE, h)) as f:
                names.update(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", f.read()))
    return sorted(names)


def version() -> str:
    return lib().pkv_version().decode()


def _check(status: int):
    if status != 0:
        raise PkvError(status, lib().pkv_last_error().decode())


def _stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtypes, ndim: int | None = None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (the library has no CPU path)")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: {t.dim()} dims, expected {ndim}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_out(out, out_lse, rows: int, Hq: int, D: int, dev, return_lse: bool):
    """Allocate or check ``out [rows][Hq][D]`` and ``out_lse [rows][Hq]`` (float32)."""
    if out is None:
        out = torch.empty((rows, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), 3)
    if tuple(out.shape) != (rows, Hq, D):
        raise ValueError(f"out shape {tuple(out.shape)}, expected {(rows, Hq, D)}")
    if out_lse is None and return_lse:
        out_lse = torch.empty((rows, Hq), dtype=torch.float32, device=dev)
    if out_lse is not None:
        _need(out_lse, "out_lse", (torch.float32,), 2)
        if tuple(out_lse.shape) != (rows, Hq):
            raise ValueError(f"out_lse shape {tuple(out_lse.shape)}, expected {(rows, Hq)}")
    return out, out_lse


def _check_decode_inputs(q, cache, block_tables, context_lens, num_splits):
    """Host-side checks shared by every decode mode; returns ``(B, Hq, D)``."""
    _need(q, "q", (torch.float32, torch.bfloat16), 3)
    B, Hq, D = q.shape
    _need(block_tables, "block_tables", (torch.int32,), 2)
    _need(context_lens, "context_lens", (torch.int32,), 1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens batch mismatch")
    if D != cache.head_dim:
        raise ValueError(f"q head_dim {D} != cache head_dim {cache.head_dim}")
    if num_splits is not None:
        _need(num_splits, "num_splits", (torch.int32,), 1)
        if num_splits.shape[0] != B:
            raise ValueError("num_splits batch mismatch")
    return B, Hq, D


def _check_workspace(workspace, need: int):
    if workspace is None:
        return 0
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    _need(workspace, "workspace", (workspace.dtype,))
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace of {nbytes} bytes, {need} needed")
    return nbytes


@dataclass
class KVCache:
    """The block pool: ``k, v [num_blocks][num_kv_heads][block_size][head_dim]``,
    plus ``k_scale, v_scale [num_blocks][num_kv_heads][block_size]`` float32 for
    int8 and fp8 (OCP E4M3, stored as ``torch.float8_e4m3fn``)."""

    k: torch.Tensor
    v: torch.Tensor
    k_scale: torch.Tensor | None = None
    v_scale: torch.Tensor | None = None

    @property
    def num_blocks(self) -> int:
        return self.k.shape[0]

    @property
    def num_kv_heads(self) -> int:
        return self.k.shape[1]

    @property
    def block_size(self) -> int:
        return self.k.shape[2]

    @property
    def head_dim(self) -> int:
        return self.k.shape[3]

    @property
    def kv_dtype(self) -> int:
        return _CODE[self.k.dtype]

    @classmethod
    def allocate(cls, num_blocks: int, num_kv_heads: int, head_dim: int, kv_dtype: int,
                 device="cuda", block_size: int = 16, fill_nan: bool = True) -> "KVCache":
        """Allocate a pool; float rows (int8 and fp8: the scales; fp8 codes too)
        start as NaN so that a read of an unwritten row shows up in the output."""
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        dt = _TORCH_DTYPE[kv_dtype]
        if kv_dtype in _SCALED:
            if kv_dtype == FP8:   # 0x7F is an E4M3 NaN
                k = torch.full(shape, 0x7F if fill_nan else 0, dtype=torch.uint8, device=device).view(dt)
                v = torch.full(shape, 0x7F if fill_nan else 0, dtype=torch.uint8, device=device).view(dt)
            else:
                k = torch.zeros(shape, dtype=dt, device=device)
                v = torch.zeros(shape, dtype=dt, device=device)
            fill = float("nan") if fill_nan else 1.0
            ks = torch.full(shape[:3], fill, dtype=torch.float32, device=device)
            vs = torch.full(shape[:3], fill, dtype=torch.float32, device=device)
            return cls(k, v, ks, vs)
        fill = float("nan") if fill_nan else 0.0
        return cls(torch.full(shape, fill, dtype=dt, device=device), torch.full(shape, fill, dtype=dt, device=device))

    def descriptor(self) -> _Cache:
        for name in ("k", "v"):
            _need(getattr(self, name), f"cache.{name}", tuple(_CODE), 4)
        if self.v.shape != self.k.shape or self.v.dtype != self.k.dtype:
            raise ValueError("cache.k and cache.v differ in shape or dtype")
        if self.kv_dtype in _SCALED:
            for name in ("k_scale", "v_scale"):
                t = getattr(self, name)
                if t is None:
                    raise ValueError(f"int8 / fp8 cache needs {name}")
                _need(t, f"cache.{name}", (torch.float32,), 3)
                if tuple(t.shape) != tuple(self.k.shape[:3]):
                    raise ValueError(f"cache.{name} shape {tuple(t.shape)} != {tuple(self.k.shape[:3])}")
        return _Cache(self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim, self.kv_dtype,
                      self.k.data_ptr(), self.v.data_ptr(),
                      _ptr(self.k_scale) if self.kv_dtype in _SCALED else None,
                      _ptr(self.v_scale) if self.kv_dtype in _SCALED else None)


def reshape_and_cache(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                      cache: KVCache) -> None:
    """Write rows ``[T][Hkv][D]`` into the pool at ``slot_mapping`` (int64; < 0 skips)."""
    _need(k_new, "k_new", (torch.float32, torch.bfloat16), 3)
    _need(v_new, "v_new", (k_new.dtype,), 3)
    _need(slot_mapping, "slot_mapping", (torch.int64,), 1)
    T = k_new.shape[0]
    if tuple(v_new.shape) != tuple(k_new.shape) or slot_mapping.shape[0] != T:
        raise ValueError("k_new, v_new, slot_mapping disagree on the token count")
    if tuple(k_new.shape[1:]) != (cache.num_kv_heads, cache.head_dim):
        raise ValueError(f"rows are {tuple(k_new.shape[1:])}, cache wants ({cache.num_kv_heads}, {cache.head_dim})")
    d = cache.descriptor()
    _check(lib().pkv_reshape_and_cache(k_new.data_ptr(), v_new.data_ptr(), _CODE[k_new.dtype],
                                       slot_mapping.data_ptr(), T, ctypes.byref(d), _stream_handle()))


def decode_workspace_bytes(batch: int, num_q_heads: int, head_dim: int, max_num_splits: int) -> int:
    return int(lib().pkv_decode_workspace_bytes(batch, num_q_heads, head_dim, max_num_splits))


def decode_default_max_num_splits(max_blocks_per_seq: int) -> int:
    """The library's choice of decode mode for a table width, for calls
    without a split plan: 1 (one split per sequence) or 0 (balanced)."""
    r = int(lib().pkv_decode_default_max_num_splits(max_blocks_per_seq))
    if r < 0:
        raise PkvError(-1, lib().pkv_last_error().decode())
    return r


def chunked_kernel_for(max_q_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int) -> int:
    """The kernel ``paged_attention_chunked`` runs for this call shape (host
    only): CHUNKED_DECODE_ROWS, CHUNKED_ROWS_MFMA or CHUNKED_TILES."""
    r = int(lib().pkv_chunked_kernel_for(max_q_len, num_q_heads, num_kv_heads, head_dim))
    if r < 0:
        raise PkvError(-1, lib().pkv_last_error().decode())
    return r


def paged_attention_decode(q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, num_splits: torch.Tensor | None,
                           max_num_splits: int | str, scale: float, out: torch.Tensor | None = None,
                           out_lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                           return_lse: bool = False, partials_only: bool = False):
    """Decode attention: ``q [B][Hq][D]`` -> ``out [B][Hq][D]`` float32 (and lse).

    ``max_num_splits=0`` with ``num_splits=None`` selects the balanced mode; a
    workspace passed for it must have been zero-filled once (every call
    leaves its counters at zero).

    ``max_num_splits="auto"`` (with ``num_splits=None``) takes
    :func:`decode_default_max_num_splits` of the table width.

    ``partials_only=True`` (needs ``max_num_splits > 1`` and a ``workspace``)
    runs only the split pass and returns ``(o_part [B][S][Hq][D],
    lse_part [B][S][Hq])`` views of the workspace, for :func:`lse_combine`."""
    if max_num_splits == "auto":
        if num_splits is not None or partials_only:
            raise ValueError('max_num_splits="auto" takes no num_splits and no partials_only')
        _need(block_tables, "block_tables", (torch.int32,), 2)
        max_num_splits = decode_default_max_num_splits(block_tables.shape[1])
    B, Hq, D = _check_decode_inputs(q, cache, block_tables, context_lens, num_splits)
    if partials_only:
        if not isinstance(max_num_splits, int) or max_num_splits < 2 or workspace is None:
            raise ValueError("partials_only needs max_num_splits > 1 and a workspace")
        if out is not None or out_lse is not None:
            raise ValueError("partials_only writes the workspace only: pass no out / out_lse")
        ws_bytes = _check_workspace(workspace, decode_workspace_bytes(B, Hq, D, max_num_splits))
        d = cache.descriptor()
        _check(lib().pkv_paged_attention_decode(
            q.data_ptr(), _CODE[q.dtype], B, Hq, ctypes.byref(d), block_tables.data_ptr(), block_tables.shape[1],
            context_lens.data_ptr(), _ptr(num_splits), max_num_splits, float(scale), None, None,
            workspace.data_ptr(), ws_bytes, _stream_handle()))
        f = workspace.view(torch.float32)
        n_o = B * max_num_splits * Hq * D
        return (f[:n_o].view(B, max_num_splits, Hq, D),
                f[n_o:n_o + B * max_num_splits * Hq].view(B, max_num_splits, Hq))
    out, out_lse = _check_out(out, out_lse, B, Hq, D, q.device, return_lse)
    need = decode_workspace_bytes(B, Hq, D, max_num_splits)
    if need and workspace is None:
        # zero-filled: the balanced mode's arrival counters must start at 0
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, need)
    d = cache.descriptor()
    _check(lib().pkv_paged_attention_decode(
        q.data_ptr(), _CODE[q.dtype], B, Hq, ctypes.byref(d), block_tables.data_ptr(), block_tables.shape[1],
        context_lens.data_ptr(), _ptr(num_splits), max_num_splits, float(scale), out.data_ptr(),
        _ptr(out_lse), _ptr(workspace), ws_bytes, _stream_handle()))
    return (out, out_lse) if (return_lse or out_lse is not None) else out


def paged_attention_decode_append(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                                  q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, num_splits: torch.Tensor | None,
                                  max_num_splits: int, scale: float, out: torch.Tensor | None = None,
                                  out_lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                  return_lse: bool = False, partials_only: bool = False):
    """:func:`reshape_and_cache` of the step's new rows ``[B][Hkv][D]`` (one per
    sequence, at ``slot_mapping``) followed by :func:`paged_attention_decode`,
    in one pass. Split mode only (``max_num_splits >= 1``); ``partials_only``
    as for :func:`paged_attention_decode`."""
    B, Hq, D = _check_decode_inputs(q, cache, block_tables, context_lens, num_splits)
    _need(k_new, "k_new", (torch.float32, torch.bfloat16), 3)
    _need(v_new, "v_new", (k_new.dtype,), 3)
    _need(slot_mapping, "slot_mapping", (torch.int64,), 1)
    if tuple(k_new.shape) != (B, cache.num_kv_heads, cache.head_dim) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError(f"new rows are {tuple(k_new.shape)}, want ({B}, {cache.num_kv_heads}, {cache.head_dim})")
    if slot_mapping.shape[0] != B:
        raise ValueError("slot_mapping batch mismatch")
    if partials_only:
        if max_num_splits < 2 or workspace is None:
            raise ValueError("partials_only needs max_num_splits > 1 and a workspace")
        if out is not None or out_lse is not None:
            raise ValueError("partials_only writes the workspace only: pass no out / out_lse")
    else:
        out, out_lse = _check_out(out, out_lse, B, Hq, D, q.device, return_lse)
    need = decode_workspace_bytes(B, Hq, D, max_num_splits) if max_num_splits > 0 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, need)
    d = cache.descriptor()
    _check(lib().pkv_paged_attention_decode_append(
        k_new.data_ptr(), v_new.data_ptr(), _CODE[k_new.dtype], slot_mapping.data_ptr(),
        q.data_ptr(), _CODE[q.dtype], B, Hq, ctypes.byref(d), block_tables.data_ptr(), block_tables.shape[1],
        context_lens.data_ptr(), _ptr(num_splits), max_num_splits, float(scale), _ptr(out),
        _ptr(out_lse), _ptr(workspace), ws_bytes, _stream_handle()))
    if partials_only:
        f = workspace.view(torch.float32)
        n_o = B * max_num_splits * Hq * D
        return (f[:n_o].view(B, max_num_splits, Hq, D),
                f[n_o:n_o + B * max_num_splits * Hq].view(B, max_num_splits, Hq))
    return (out, out_lse) if (return_lse or out_lse is not None) else out


def paged_attention_decode_noalloc(q: torch.Tensor, cache: KVCache, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, num_splits: torch.Tensor | None,
                                   max_num_splits: int, scale: float, out: torch.Tensor | None = None,
                                   out_lse: torch.Tensor | None = None, return_lse: bool = False):
    """:func:`paged_attention_decode` without a workspace: the library keeps
    the partials in its own fixed device array (``NOALLOC_SCRATCH_BYTES`` per
    GPU), for callers that cannot allocate. Pass ``out`` (and ``out_lse``) to
    allocate nothing here either. Calls that overlap on one GPU race."""
    B, Hq, D = _check_decode_inputs(q, cache, block_tables, context_lens, num_splits)
    out, out_lse = _check_out(out, out_lse, B, Hq, D, q.device, return_lse)
    d = cache.descriptor()
    _check(lib().pkv_paged_attention_decode_noalloc(
        q.data_ptr(), _CODE[q.dtype], B, Hq, ctypes.byref(d), block_tables.data_ptr(), block_tables.shape[1],
        context_lens.data_ptr(), _ptr(num_splits), int(max_num_splits), float(scale), out.data_ptr(),
        _ptr(out_lse), _stream_handle()))
    return (out, out_lse) if (return_lse or out_lse is not None) else out


def paged_attention_chunked(q: torch.Tensor, cu_q_lens: torch.Tensor, max_q_len: int, cache: KVCache,
                            block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                            out: torch.Tensor | None = None, out_lse: torch.Tensor | None = None,
                            return_lse: bool = False):
    """Chunked prefill: ``q [sum L][Hq][D]`` bf16 -> ``out [sum L][Hq][D]`` float32 (and lse)."""
    _need(q, "q", (torch.bfloat16,), 3)
    T, Hq, D = q.shape
    if D != cache.head_dim:
        raise ValueError(f"q head_dim {D} != cache head_dim {cache.head_dim}")
    _need(cu_q_lens, "cu_q_lens", (torch.int32,), 1)
    S = cu_q_lens.shape[0] - 1
    if S < 0:
        raise ValueError("cu_q_lens needs num_seqs + 1 entries")
    _need(block_tables, "block_tables", (torch.int32,), 2)
    _need(context_lens, "context_lens", (torch.int32,), 1)
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens / cu_q_lens disagree on the sequence count")
    out, out_lse = _check_out(out, out_lse, T, Hq, D, q.device, return_lse)
    d = cache.descriptor()
    _check(lib().pkv_paged_attention_chunked(
        q.data_ptr(), BF16, S, Hq, cu_q_lens.data_ptr(), int(max_q_len), ctypes.byref(d),
        block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(), float(scale),
        out.data_ptr(), _ptr(out_lse), _stream_handle()))
    return (out, out_lse) if (return_lse or out_lse is not None) else out


def lse_combine(o_part: torch.Tensor, lse_part: torch.Tensor, num_splits: torch.Tensor,
                out: torch.Tensor | None = None, out_lse: torch.Tensor | None = None):
    """Merge ``o_part [B][S][Hq][D]`` / ``lse_part [B][S][Hq]`` -> ``out [B][Hq][D]``, ``lse [B][Hq]``."""
    _need(o_part, "o_part", (torch.float32,), 4)
    _need(lse_part, "lse_part", (torch.float32,), 3)
    _need(num_splits, "num_splits", (torch.int32,), 1)
    B, S, Hq, D = o_part.shape
    if tuple(lse_part.shape) != (B, S, Hq) or num_splits.shape[0] != B:
        raise ValueError("o_part / lse_part / num_splits shapes disagree")
    out, out_lse = _check_out(out, out_lse, B, Hq, D, o_part.device, True)
    _check(lib().pkv_lse_combine(o_part.data_ptr(), lse_part.data_ptr(), B, Hq, D, S, num_splits.data_ptr(),
                                 out.data_ptr(), out_lse.data_ptr(), _stream_handle()))
    return out, out_lse


def stream_read(src: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Measurement aid (``include/pkv_measure.h``): one launch that reads every
    byte of ``src`` once and does nothing else. Returns the sink buffer (its
    contents carry no meaning); pass one to allocate nothing."""
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    groups = int(lib().pkv_stream_read_workgroups(nbytes))
    if sink is None:
        sink = torch.empty(max(1, groups), dtype=torch.int32, device=src.device)
    if sink.numel() * sink.element_size() < 4 * groups:
        raise ValueError("sink too small")
    st = int(lib().pkv_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), _stream_handle()))
    if st != 0:
        raise PkvError(st, "pkv_stream_read: bad arguments (16-byte aligned buffer of a multiple of 16 bytes) "
                           "or launch failure")
    return sink
