"""PKV_DEBUG=1: before launching, the entry points validate the metadata that
lives in device memory (context lengths, block tables, split counts,
cu_q_lens, slots), wait for that pass, and refuse a call whose metadata is bad
with PKV_ERR_INVALID_ARG and the first offending entry named. Without the
variable the kernels' own bounds checks turn such sequences into NaN instead
(tests/test_gpu_decode.py, test_gpu_chunked.py). With good metadata the
result is bit for bit the one without the check."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_side as G

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_on(monkeypatch):
    monkeypatch.setenv("PKV_DEBUG", "1")


def _decode(step, cache, gpu, tables=None, ctx=None, ns=None, max_ns=None, noalloc=False):
    import torch
    q, t, c, n = step.decode_batch()
    t = t if tables is None else tables
    c = c if ctx is None else ctx
    n = n if ns is None else ns
    mx = int(max_ns if max_ns is not None else max(1, int(n.max())))
    args = (G.tensor(q, step.q_dtype, gpu), cache, G.ints(t, gpu), G.ints(c, gpu),
            None if mx == 0 else G.ints(n, gpu), mx, float(step.scale))
    G.announce(f"debug-mode decode {step.name} max_ns={mx} noalloc={noalloc}")
    if noalloc:
        out = G.pkv.paged_attention_decode_noalloc(*args)
    else:
        out = G.pkv.paged_attention_decode(*args)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _expect(status_msg, fn):
    with pytest.raises(G.pkv.PkvError) as ei:
        fn()
    assert ei.value.status == -1, ei.value
    assert "PKV_DEBUG" in str(ei.value) and status_msg in str(ei.value), str(ei.value)


@pytest.mark.parametrize("mode", [1, 4, 0])
def test_decode_debug_mode_names_the_bad_entry(gpu, debug_on, mode):
    step = W.make_step("dbg", [40, 40, 40, 40], [1] * 4, num_q_heads=4, num_kv_heads=2, head_dim=64, seed=500,
                       num_splits=2)
    cache = G.build_cache(step, gpu)
    _, tables, ctx, ns = step.decode_batch()
    bad_ctx = ctx.copy()
    bad_ctx[2] = tables.shape[1] * 16 + 1
    _expect("context_lens[2]", lambda: _decode(step, cache, gpu, ctx=bad_ctx, max_ns=mode))
    bad_t = tables.copy()
    bad_t[1, 2] = step.num_blocks + 9
    _expect(f"block_tables entry {1 * tables.shape[1] + 2}", lambda: _decode(step, cache, gpu, tables=bad_t, max_ns=mode))
    if mode > 1:
        bad_ns = ns.copy()
        bad_ns[3] = mode + 1
        _expect("num_splits[3]", lambda: _decode(step, cache, gpu, ns=bad_ns, max_ns=mode))


def test_decode_debug_mode_good_metadata_changes_nothing(gpu, monkeypatch):
    step = W.ragged_decode(batch=24, seed=501)
    cache = G.build_cache(step, gpu)
    for mode in (1, 16, 0):
        monkeypatch.delenv("PKV_DEBUG", raising=False)
        ref = _decode(step, cache, gpu, max_ns=mode)
        monkeypatch.setenv("PKV_DEBUG", "1")
        got = _decode(step, cache, gpu, max_ns=mode)
        assert got.tobytes() == ref.tobytes(), mode
        got = _decode(step, cache, gpu, max_ns=mode, noalloc=True)
        assert got.tobytes() == ref.tobytes(), mode


def test_noalloc_decode_debug_mode(gpu, debug_on):
    step = W.make_step("dbgna", [40, 33], [1, 1], num_q_heads=4, num_kv_heads=2, head_dim=64, seed=502)
    cache = G.build_cache(step, gpu)
    _, tables, ctx, _ = step.decode_batch()
    bad = ctx.copy()
    bad[1] = -5
    _expect("context_lens[1]", lambda: _decode(step, cache, gpu, ctx=bad, max_ns=0, noalloc=True))


def test_chunked_debug_mode(gpu, debug_on):
    step = W.make_step("dbgc", [100, 100], [40, 30], num_q_heads=16, num_kv_heads=8, head_dim=128, seed=503)
    cache = G.build_cache(step, gpu)
    q, cu, tables, ctx = step.chunk_batch()

    def run(cu_=cu, ctx_=ctx, tables_=tables, max_q=40):
        G.announce("debug-mode chunked")
        return G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu_, gpu), max_q, cache,
                                             G.ints(tables_, gpu), G.ints(ctx_, gpu), float(step.scale))

    c = ctx.copy()
    c[1] = 20
    _expect("chunk 1 is longer than its context", lambda: run(ctx_=c))
    _expect("chunk 0 is longer than max_q_len", lambda: run(max_q=35))
    u = cu.copy()
    u[0] = 3
    _expect("cu_q_lens[0]", lambda: run(cu_=u))
    t = tables.copy()
    t[0, 0] = -1
    _expect("block_tables entry 0", lambda: run(tables_=t))
    out = run().cpu().numpy()
    assert np.isfinite(out).all()


def test_reshape_and_append_debug_mode(gpu, debug_on):
    import torch
    step = W.qwen3_decode(batch=4, seed=504)
    cache = G.build_cache(step, gpu, with_new=False)
    bad = step.new_slots.copy()
    bad[2] = step.num_blocks * 16 + 7
    _expect("slot_mapping[2] is past the pool", lambda: G.pkv.reshape_and_cache(
        G.tensor(step.new_k, "bf16", gpu), G.tensor(step.new_v, "bf16", gpu), G.ints(bad, gpu, torch.int64), cache))
    q, tables, ctx, _ = step.decode_batch()
    wrong = step.new_slots.copy()
    wrong[1] += 1
    _expect("slot_mapping[1] is not the slot", lambda: G.pkv.paged_attention_decode_append(
        G.tensor(step.new_k, "bf16", gpu), G.tensor(step.new_v, "bf16", gpu), G.ints(wrong, gpu, torch.int64),
        G.tensor(q, "bf16", gpu), cache, G.ints(tables, gpu), G.ints(ctx, gpu), None, 1, float(step.scale)))


def test_combine_debug_mode(gpu, debug_on):
    import torch
    o = torch.zeros(3, 4, 16, 128, device=gpu)
    l = torch.zeros(3, 4, 16, device=gpu)
    ns = G.ints(np.array([1, 5, 2], np.int32), gpu)
    _expect("num_splits[1]", lambda: G.pkv.lse_combine(o, l, ns))
