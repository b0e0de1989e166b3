"""The allocation-free decode entry point (pkv_paged_attention_decode_noalloc,
for callers that cannot allocate device memory) against the workspace decode
entry point it mirrors: the same kernels, so the outputs must agree bit for
bit. Two calls in a row on the library's one scratch array, the second with a
smaller input; split and balanced modes interleaved (a split call leaves its
partials where the balanced counters go, which the balanced call must clear);
and graph replays of a captured call."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_side as G

pytestmark = pytest.mark.gpu


def _inputs(step, gpu):
    q, tables, ctx, ns = step.decode_batch()
    return (G.tensor(q, step.q_dtype, gpu), G.ints(tables, gpu), G.ints(ctx, gpu), G.ints(ns, gpu), int(ns.max()))


def _pair(step, cache, gpu, mode):
    """(workspace decode, no-alloc decode) outputs of one step; mode "split"
    uses the step's split plan, "balanced" max_num_splits = 0."""
    import torch
    q, tables, ctx, ns, mx = _inputs(step, gpu)
    if mode == "balanced":
        ns, mx = None, 0
    G.announce(f"no-alloc decode {step.name} B={q.shape[0]} mode={mode} max_ns={mx}")
    ref, ref_lse = G.pkv.paged_attention_decode(q, cache, tables, ctx, ns, mx, float(step.scale), return_lse=True)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    G.pkv.paged_attention_decode_noalloc(q, cache, tables, ctx, ns, mx, float(step.scale), out=out, out_lse=lse)
    torch.cuda.synchronize()
    return ref, ref_lse, out, lse


def _same(a, b):
    import torch
    return torch.equal(a, b)


@pytest.mark.parametrize("mode", ["split", "balanced"])
def test_noalloc_matches_workspace_decode_two_calls(gpu, mode):
    big = W.ragged_decode(batch=96, seed=401, max_tokens_per_split=512)
    small = W.ragged_decode(batch=9, seed=402, max_tokens_per_split=256)
    for step in (big, small):
        cache = G.build_cache(step, gpu)
        ref, ref_lse, out, lse = _pair(step, cache, gpu, mode)
        assert _same(out, ref) and _same(lse, ref_lse), (mode, step.name, len(step.context_lens))
        assert bool(torch_isfinite(out))


def torch_isfinite(t):
    import torch
    return torch.isfinite(t).all()


def test_noalloc_split_then_balanced_then_split(gpu):
    """The split call's partials overwrite the start of the scratch array;
    the balanced call that follows clears its counters before it launches."""
    a = W.ragged_decode(batch=64, seed=403, max_tokens_per_split=512)
    b = W.mixed_int8(num_prefill=1, num_decode=30, seed=404, max_tokens_per_split=512)
    ca, cb = G.build_cache(a, gpu), G.build_cache(b, gpu)
    for step, cache, mode in ((a, ca, "split"), (b, cb, "balanced"), (b, cb, "split"), (a, ca, "balanced")):
        ref, ref_lse, out, lse = _pair(step, cache, gpu, mode)
        assert _same(out, ref) and _same(lse, ref_lse), (step.name, mode)


def test_noalloc_one_split_needs_no_scratch(gpu):
    step = W.qwen3_decode(batch=16, seed=405)
    cache = G.build_cache(step, gpu)
    ref, ref_lse, out, lse = _pair(step, cache, gpu, "split")
    assert _same(out, ref) and _same(lse, ref_lse)


@pytest.mark.parametrize("mode", ["split", "balanced"])
def test_noalloc_graph_replays(gpu, mode):
    """A captured no-alloc call replayed several times, with eager calls of the
    other mode on the same scratch array in between, reproduces the eager
    result every time."""
    import torch
    step = W.ragged_decode(batch=48, seed=406, max_tokens_per_split=512)
    other = W.ragged_decode(batch=20, seed=407, max_tokens_per_split=256)
    cache, cache_o = G.build_cache(step, gpu), G.build_cache(other, gpu)
    q, tables, ctx, ns, mx = _inputs(step, gpu)
    if mode == "balanced":
        ns, mx = None, 0
    qo, to, co, nso, mxo = _inputs(other, gpu)
    ref = G.pkv.paged_attention_decode(q, cache, tables, ctx, ns, mx, float(step.scale))
    out = torch.empty_like(ref)
    out_o = torch.empty((qo.shape[0], 16, 128), dtype=torch.float32, device=gpu)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        # warm the entry point (its first call on a device looks up the array) before capture
        G.pkv.paged_attention_decode_noalloc(q, cache, tables, ctx, ns, mx, float(step.scale), out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    G.announce(f"no-alloc graph capture mode={mode}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.pkv.paged_attention_decode_noalloc(q, cache, tables, ctx, ns, mx, float(step.scale), out=out)
    for i in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, ref), (mode, i)
        # the other mode on the same array between replays
        if mode == "balanced":
            G.pkv.paged_attention_decode_noalloc(qo, cache_o, to, co, nso, mxo, float(other.scale), out=out_o)
        else:
            G.pkv.paged_attention_decode_noalloc(qo, cache_o, to, co, None, 0, float(other.scale), out=out_o)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out_o).all())


def test_noalloc_refuses_calls_beyond_the_array(gpu):
    """A call whose partials would not fit the fixed array is refused on the
    host (PKV_ERR_WORKSPACE) and launches nothing."""
    step = W.qwen3_decode(batch=8, seed=408)
    cache = G.build_cache(step, gpu)
    q, tables, ctx, _, _ = _inputs(step, gpu)
    mx = 20000   # 8 x 20000 x 16 x 129 x 4 bytes = 1.3 GB of partials
    ns = G.ints(np.full(8, 2, np.int32), gpu)
    with pytest.raises(G.pkv.PkvError, match="scratch"):
        G.pkv.paged_attention_decode_noalloc(q, cache, tables, ctx, ns, mx, float(step.scale))
