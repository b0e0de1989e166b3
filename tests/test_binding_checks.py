"""The Python binding's shape checks, on the CPU: a call whose tensors disagree
with each other or with the cache raises ValueError before the C library is
reached. The library is replaced by a stand-in that fails the test if any
entry point is called, and the binding's device check is relaxed so that CPU
tensors stand in for device ones (nothing is ever launched)."""

from __future__ import annotations

import pytest
import torch

import paged_kv_attention_19_amd as pkv


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"the binding reached the C library ({name}) before its shape checks failed")


@pytest.fixture
def host_only(monkeypatch):
    real_need = pkv._need

    def need(t, name, dtypes, ndim=None, device=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in dtypes:
            raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
        if ndim is not None and t.dim() != ndim:
            raise ValueError(f"{name}: {t.dim()} dims, expected {ndim}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    monkeypatch.setattr(pkv, "_need", need)
    monkeypatch.setattr(pkv, "lib", lambda: _NoCalls())
    # workspace sizes are host arithmetic; mirror the C formula for split mode
    monkeypatch.setattr(pkv, "decode_workspace_bytes",
                        lambda B, Hq, D, S: 0 if S <= 1 else (B * S * Hq * (D + 1) * 4 + 255) // 256 * 256)
    yield
    monkeypatch.setattr(pkv, "_need", real_need)


def _cache(D=128, Hkv=8, blocks=16):
    k = torch.zeros(blocks, Hkv, 16, D, dtype=torch.bfloat16)
    return pkv.KVCache(k, k.clone())


def _decode_args(B=4, Hq=16, D=128):
    return dict(q=torch.zeros(B, Hq, D, dtype=torch.bfloat16), block_tables=torch.zeros(B, 3, dtype=torch.int32),
                context_lens=torch.ones(B, dtype=torch.int32))


def test_decode_q_head_dim_must_match_cache(host_only):
    a = _decode_args(D=64)
    with pytest.raises(ValueError, match="head_dim"):
        pkv.paged_attention_decode(a["q"], _cache(D=128), a["block_tables"], a["context_lens"], None, 1, 0.1)


@pytest.mark.parametrize("field,shape", [("out", (4, 16, 64)), ("out", (3, 16, 128)), ("out_lse", (4, 8)),
                                         ("out_lse", (5, 16))])
def test_decode_output_shapes(host_only, field, shape):
    a = _decode_args()
    kw = {field: torch.zeros(shape, dtype=torch.float32)}
    with pytest.raises(ValueError, match=f"{field} shape"):
        pkv.paged_attention_decode(a["q"], _cache(), a["block_tables"], a["context_lens"], None, 1, 0.1, **kw)


def test_decode_partials_only_runs_the_same_checks(host_only):
    """partials_only used to skip the table, length and head_dim checks."""
    a = _decode_args()
    ns = torch.ones(4, dtype=torch.int32)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError, match="batch mismatch"):
        pkv.paged_attention_decode(a["q"], _cache(), torch.zeros(3, 3, dtype=torch.int32), a["context_lens"], ns, 2,
                                   0.1, workspace=ws, partials_only=True)
    with pytest.raises(TypeError, match="context_lens"):
        pkv.paged_attention_decode(a["q"], _cache(), a["block_tables"], a["context_lens"].long(), ns, 2, 0.1,
                                   workspace=ws, partials_only=True)
    with pytest.raises(ValueError, match="head_dim"):
        pkv.paged_attention_decode(a["q"], _cache(D=64), a["block_tables"], a["context_lens"], ns, 2, 0.1,
                                   workspace=ws, partials_only=True)
    with pytest.raises(ValueError, match="num_splits batch"):
        pkv.paged_attention_decode(a["q"], _cache(), a["block_tables"], a["context_lens"],
                                   torch.ones(5, dtype=torch.int32), 2, 0.1, workspace=ws, partials_only=True)
    with pytest.raises(ValueError, match="workspace of"):
        pkv.paged_attention_decode(a["q"], _cache(), a["block_tables"], a["context_lens"], ns, 2, 0.1,
                                   workspace=torch.zeros(64, dtype=torch.uint8), partials_only=True)


def test_decode_workspace_too_small(host_only):
    a = _decode_args()
    ns = torch.ones(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="workspace of"):
        pkv.paged_attention_decode(a["q"], _cache(), a["block_tables"], a["context_lens"], ns, 2, 0.1,
                                   workspace=torch.zeros(100, dtype=torch.uint8))


def test_append_output_shapes(host_only):
    a = _decode_args()
    rows = torch.zeros(4, 8, 128, dtype=torch.bfloat16)
    slots = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError, match="out_lse shape"):
        pkv.paged_attention_decode_append(rows, rows.clone(), slots, a["q"], _cache(), a["block_tables"],
                                          a["context_lens"], None, 1, 0.1, out_lse=torch.zeros(4, 15))
    with pytest.raises(ValueError, match="head_dim"):
        pkv.paged_attention_decode_append(rows, rows.clone(), slots, a["q"], _cache(D=64), a["block_tables"],
                                          a["context_lens"], None, 1, 0.1)


def test_chunked_q_head_dim_and_outputs(host_only):
    """A D=64 q against a D=128 cache, or a short out / out_lse, would let the
    kernel (which strides by the cache's head_dim) read past q or write past
    out: the binding refuses them."""
    q = torch.zeros(40, 16, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 40], dtype=torch.int32)
    tab = torch.zeros(1, 4, dtype=torch.int32)
    ctx = torch.tensor([60], dtype=torch.int32)
    with pytest.raises(ValueError, match="head_dim"):
        pkv.paged_attention_chunked(q, cu, 40, _cache(D=128), tab, ctx, 0.1)
    q = torch.zeros(40, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out shape"):
        pkv.paged_attention_chunked(q, cu, 40, _cache(), tab, ctx, 0.1, out=torch.zeros(39, 16, 128))
    with pytest.raises(ValueError, match="out_lse shape"):
        pkv.paged_attention_chunked(q, cu, 40, _cache(), tab, ctx, 0.1, out_lse=torch.zeros(40, 8))
    with pytest.raises(ValueError, match="sequence count"):
        pkv.paged_attention_chunked(q, cu, 40, _cache(), torch.zeros(2, 4, dtype=torch.int32), ctx, 0.1)


def test_combine_output_shapes(host_only):
    o = torch.zeros(3, 2, 16, 128)
    l = torch.zeros(3, 2, 16)
    ns = torch.ones(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="out shape"):
        pkv.lse_combine(o, l, ns, out=torch.zeros(3, 16, 64))
    with pytest.raises(ValueError, match="out_lse shape"):
        pkv.lse_combine(o, l, ns, out_lse=torch.zeros(3, 15))
