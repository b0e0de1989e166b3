"""GPU parity: decode with append (the step's new rows written inside the
decode pass, pkv_paged_attention_decode_append) against reshape_and_cache
followed by paged_attention_decode: the pool bytes and the outputs must be
identical bit for bit (NaN included), and the outputs match the oracle to
the decode tolerance, |gpu - oracle| <= 2e-3 + 1e-2 |oracle|."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_side as G
from tests import oracle_side as O

pytestmark = pytest.mark.gpu


def decode_new_rows(step):
    """The new rows of the step's decode sequences, in decode-batch order."""
    rows = step.cu_q_lens[:-1][step.decode_idx]
    return step.new_k[rows], step.new_v[rows], step.new_slots[rows].astype(np.int64)


def run_append(step, cache, dev, slots=None, num_splits=None):
    q, tables, ctx, ns = step.decode_batch()
    if num_splits is not None:
        ns = np.broadcast_to(np.asarray(num_splits, np.int32), ns.shape).copy()
    mx = max(1, int(ns.max()))
    kn, vn, sl = decode_new_rows(step)
    if slots is not None:
        sl = np.asarray(slots, np.int64)
    G.announce(f"decode_append {step.name} B={len(ctx)} kv={step.kv_dtype} src={step.src_dtype} max_ns={mx}")
    out, lse = G.pkv.paged_attention_decode_append(
        G.tensor(kn, step.src_dtype, dev), G.tensor(vn, step.src_dtype, dev), G.ints(sl, dev, torch.int64),
        G.tensor(q, step.q_dtype, dev), cache, G.ints(tables, dev), G.ints(ctx, dev), G.ints(ns, dev), mx,
        float(step.scale), return_lse=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def two_calls(step, dev, slots=None, num_splits=None):
    """The same step as reshape_and_cache (prefix, then the new rows) + decode."""
    cache = G.build_cache(step, dev, with_new=False)
    kn, vn, sl = decode_new_rows(step)
    if slots is not None:
        sl = np.asarray(slots, np.int64)
    G.pkv.reshape_and_cache(G.tensor(kn, step.src_dtype, dev), G.tensor(vn, step.src_dtype, dev),
                            G.ints(sl, dev, torch.int64), cache)
    out, lse = G.run_decode(step, cache, dev, num_splits=num_splits)
    return cache, out, lse


def assert_same(step, dev, slots=None, num_splits=None):
    cache_a = G.build_cache(step, dev, with_new=False)
    out_a, lse_a = run_append(step, cache_a, dev, slots=slots, num_splits=num_splits)
    cache_b, out_b, lse_b = two_calls(step, dev, slots=slots, num_splits=num_splits)
    ba, bb = G.cache_bytes(cache_a), G.cache_bytes(cache_b)
    for name in bb:
        assert ba[name] == bb[name], name
    assert out_a.tobytes() == out_b.tobytes()
    assert lse_a.tobytes() == lse_b.tobytes()
    return out_a, lse_a


STEPS = {
    "tiny_f32": lambda: W.tiny_decode(),
    "qwen3_bf16_b8": lambda: W.qwen3_decode(batch=8),
    # context lengths on both sides of a block boundary, and a one-token sequence
    "bf16_edges_d64": lambda: W.make_step("edges", [1, 15, 16, 17, 32, 33, 200], [1] * 7, num_q_heads=8,
                                          num_kv_heads=2, head_dim=64, seed=51),
    "int8_from_bf16": lambda: W.make_step("a8", [300, 77, 1, 16, 17], [1] * 5, num_q_heads=16, num_kv_heads=8,
                                          head_dim=128, kv_dtype="i8", src_dtype="bf16", seed=52, num_blocks=60),
    "int8_from_f32_d64": lambda: W.make_step("a8f", [40, 33, 16], [1] * 3, num_q_heads=4, num_kv_heads=2,
                                             head_dim=64, q_dtype="f32", kv_dtype="i8", src_dtype="f32", seed=53),
    "fp8_from_bf16": lambda: W.make_step("af8", [300, 77, 1, 16, 17], [1] * 5, num_q_heads=16, num_kv_heads=8,
                                         head_dim=128, kv_dtype="fp8", src_dtype="bf16", seed=56, num_blocks=60),
    "fp8_from_f32_d64": lambda: W.make_step("af8f", [40, 33, 16], [1] * 3, num_q_heads=4, num_kv_heads=2,
                                            head_dim=64, q_dtype="f32", kv_dtype="fp8", src_dtype="f32", seed=57),
}


@pytest.mark.parametrize("name", list(STEPS))
@pytest.mark.parametrize("ns", [1, 3])
def test_append_equals_two_calls_and_oracle(gpu, name, ns):
    step = STEPS[name]()
    out, lse = assert_same(step, gpu, num_splits=ns)
    ro, rl = O.decode(step, O.pool(step))
    st = O.compare(out, ro)
    assert st["ok"], st
    st = O.compare(lse, rl)
    assert st["ok"], st


def test_append_qwen3_full_size(gpu):
    """The benchmarked shape: B=32, one split per sequence."""
    step = W.qwen3_decode()
    out, lse = assert_same(step, gpu)
    ro, rl = O.decode(step, O.pool(step))
    st = O.compare(out, ro)
    assert st["ok"], st


def test_append_skips_slots_outside_the_pool(gpu):
    """A slot of -1 or past the pool is skipped exactly as reshape_and_cache
    skips it: the row stays unwritten (NaN) and the decode reads it as such."""
    step = W.make_step("skipa", [20, 33, 7], [1, 1, 1], num_q_heads=4, num_kv_heads=2, head_dim=64, seed=54,
                       num_blocks=8)
    _, _, sl = decode_new_rows(step)
    sl = sl.copy()
    sl[0] = -1
    sl[2] = step.num_blocks * 16 + 3
    out, _ = assert_same(step, gpu, slots=sl)
    assert np.isnan(out[0]).all() and np.isnan(out[2]).all() and np.isfinite(out[1]).all()


def test_append_repeated_is_idempotent(gpu):
    """Two calls in a row (as a replayed graph would make) leave the same pool
    and give the same outputs."""
    step = W.qwen3_decode(batch=4)
    cache = G.build_cache(step, gpu, with_new=False)
    out1, lse1 = run_append(step, cache, gpu)
    b1 = G.cache_bytes(cache)
    out2, lse2 = run_append(step, cache, gpu)
    assert G.cache_bytes(cache) == b1
    assert out1.tobytes() == out2.tobytes() and lse1.tobytes() == lse2.tobytes()


def test_append_partials_only_then_combine(gpu):
    """Partials-only mode: the pass writes the new rows and the per-split
    partials; lse_combine over them gives the one-call result bit for bit."""
    step = W.make_step("pa", [300, 77, 1, 16, 129], [1] * 5, num_q_heads=16, num_kv_heads=4, head_dim=128,
                       kv_dtype="bf16", src_dtype="bf16", seed=55, num_blocks=80)
    ns = 3
    cache_a = G.build_cache(step, gpu, with_new=False)
    out_a, lse_a = run_append(step, cache_a, gpu, num_splits=ns)
    q, tables, ctx, nsv = step.decode_batch()
    nsv = np.full_like(nsv, ns)
    kn, vn, sl = decode_new_rows(step)
    cache_b = G.build_cache(step, gpu, with_new=False)
    ws = torch.empty(G.pkv.decode_workspace_bytes(len(ctx), step.num_q_heads, step.head_dim, ns),
                     dtype=torch.uint8, device=gpu)
    G.announce(f"decode_append partials_only B={len(ctx)} ns={ns}")
    o_part, l_part = G.pkv.paged_attention_decode_append(
        G.tensor(kn, step.src_dtype, gpu), G.tensor(vn, step.src_dtype, gpu), G.ints(sl, gpu, torch.int64),
        G.tensor(q, step.q_dtype, gpu), cache_b, G.ints(tables, gpu), G.ints(ctx, gpu), G.ints(nsv, gpu), ns,
        float(step.scale), workspace=ws, partials_only=True)
    out_b, lse_b = G.pkv.lse_combine(o_part, l_part, G.ints(nsv, gpu))
    torch.cuda.synchronize()
    ba, bb = G.cache_bytes(cache_a), G.cache_bytes(cache_b)
    for name in bb:
        assert ba[name] == bb[name], name
    assert out_b.cpu().numpy().tobytes() == out_a.tobytes()
    assert lse_b.cpu().numpy().tobytes() == lse_a.tobytes()
