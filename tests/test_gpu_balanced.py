"""GPU parity of the balanced decode mode (max_num_splits = 0): the batch's
tiles are dealt to the GPU's wavefronts in equal ranges and cut sequences are
merged in the same launch. Same tolerance as the split-K decode tests."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_side as G
from tests import oracle_side as O

pytestmark = pytest.mark.gpu


def run_balanced(step, cache, dev, workspace=None):
    import torch
    q, tables, ctx, _ = step.decode_batch()
    G.announce(f"balanced decode {step.name} B={len(ctx)} kv={step.kv_dtype}")
    out, lse = G.pkv.paged_attention_decode(G.tensor(q, step.q_dtype, dev), cache, G.ints(tables, dev), G.ints(ctx, dev),
                                            None, 0, float(step.scale), workspace=workspace, return_lse=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(step, gpu):
    cache = G.build_cache(step, gpu)
    out, lse = run_balanced(step, cache, gpu)
    ro, rl = O.decode(step, O.pool(step))
    st = O.compare(out, ro)
    assert st["ok"], st
    st = O.compare(lse, rl)
    assert st["ok"], st
    return cache


@pytest.mark.parametrize("make", [
    lambda: W.tiny_decode(),
    lambda: W.qwen3_decode(),
    lambda: W.qwen3_decode(batch=5, seed=7),
    lambda: W.ragged_decode(batch=24, seed=1913),
    lambda: W.mixed_int8(num_prefill=1, num_decode=24, seed=1915),
    lambda: W.make_step("b64", [1, 15, 16, 17, 100, 257], [1] * 6, num_q_heads=8, num_kv_heads=2, head_dim=64,
                        q_dtype="f32", kv_dtype="f32", seed=140),
    lambda: W.mixed_int8(num_prefill=1, num_decode=24, seed=1915, kv_dtype="fp8"),
    lambda: W.make_step("b64f8", [1, 15, 16, 17, 100, 257], [1] * 6, num_q_heads=8, num_kv_heads=2, head_dim=64,
                        q_dtype="f32", kv_dtype="fp8", src_dtype="f32", seed=141),
], ids=["tiny", "qwen3", "qwen3_b5", "ragged24", "int8_rows", "f32_d64", "fp8_rows", "fp8_d64_f32q"])
def test_balanced_matches_oracle(gpu, make):
    check(make(), gpu)


@pytest.mark.slow
def test_balanced_ragged_full_size_sampled(gpu):
    step = W.ragged_decode()
    cache = G.build_cache(step, gpu)
    out, lse = run_balanced(step, cache, gpu)
    rng = np.random.default_rng(1)
    rows = [(int(b), int(h)) for b, h in zip(rng.integers(0, 256, 40), rng.integers(0, 16, 40))]
    rows.append((int(np.argmax(step.context_lens)), 3))
    ro, rl = O.decode(step, O.pool(step), rows=rows)
    mask = np.zeros(out.shape[:2], bool)
    for b, h in rows:
        mask[b, h] = True
    assert O.compare(out[mask], ro[mask])["ok"]
    assert O.compare(lse[mask], rl[mask])["ok"]
    assert np.isfinite(out).all()


def test_balanced_empty_and_bad_sequences(gpu):
    """n = 0 gives (0, -inf); a context longer than its table or a block id
    outside the pool gives NaN for that sequence only."""
    step = W.make_step("bal_bad", [40, 33, 70, 18], [1] * 4, num_q_heads=4, num_kv_heads=2, head_dim=64, seed=141)
    cache = G.build_cache(step, gpu)
    ro, _ = O.decode(step, O.pool(step))
    step.context_lens = step.context_lens.copy()
    step.block_tables = step.block_tables.copy()
    step.context_lens[1] = 0
    step.context_lens[2] = step.block_tables.shape[1] * 16 + 1
    step.block_tables[3, 1] = step.num_blocks + 2
    out, lse = run_balanced(step, cache, gpu)
    assert (out[1] == 0).all() and (lse[1] == -np.inf).all()
    assert np.isnan(out[2]).all() and np.isnan(out[3]).all()
    assert O.compare(out[0], ro[0])["ok"]


def test_balanced_repeats_and_graph_replays_bit_identically(gpu):
    """The arrival counters are left at zero: calls on one workspace, eager
    and graph-replayed, give the same bits every time."""
    import torch
    step = W.qwen3_decode(batch=32, seed=3)
    cache = G.build_cache(step, gpu)
    q, tables, ctx, _ = step.decode_batch()
    qd, td, cd = G.tensor(q, "bf16", gpu), G.ints(tables, gpu), G.ints(ctx, gpu)
    ws = torch.zeros(G.pkv.decode_workspace_bytes(32, 16, 128, 0), dtype=torch.uint8, device=gpu)
    out = torch.empty((32, 16, 128), dtype=torch.float32, device=gpu)
    G.announce("balanced eager x3 + graph x4")
    ref = None
    for _ in range(3):
        G.pkv.paged_attention_decode(qd, cache, td, cd, None, 0, float(step.scale), out=out, workspace=ws)
        torch.cuda.synchronize()
        ref = out.clone() if ref is None else ref
        assert torch.equal(out, ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.pkv.paged_attention_decode(qd, cache, td, cd, None, 0, float(step.scale), out=out, workspace=ws)
    for _ in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    ctr = ws[: 32 * 16 * 4].view(torch.int32)
    assert int(ctr.abs().sum()) == 0


def test_balanced_first_calls_on_fresh_workspaces_many_cuts(gpu):
    """A batch wide enough for 512 workgroups cuts most sequences between
    wavefronts. Each call runs on a freshly zeroed workspace, so a merge that
    read a contributor's partial before its stores had landed would take
    zeros and miss the oracle. Five first calls, each checked."""
    import torch
    step = W.make_step("cuts", np.full(128, 1100), np.ones(128, np.int64), num_q_heads=16, num_kv_heads=8,
                       head_dim=128, kv_dtype="bf16", seed=150)
    cache = G.build_cache(step, gpu)
    ro, rl = O.decode(step, O.pool(step))
    for i in range(5):
        ws = torch.zeros(G.pkv.decode_workspace_bytes(128, 16, 128, 0), dtype=torch.uint8, device=gpu)
        out, lse = run_balanced(step, cache, gpu, workspace=ws)
        for got, ref in ((out, ro), (lse, rl)):
            st = O.compare(got, ref)
            assert st["ok"], (i, st)


@pytest.mark.parametrize("make,mode", [
    (lambda: W.qwen3_decode(), 1),                        # 24-block tables: one split per sequence
    (lambda: W.ragged_decode(batch=24, seed=1913), 0),    # 512-block tables: balanced
], ids=["qwen3_one_split", "ragged24_balanced"])
def test_auto_mode_matches_oracle(gpu, make, mode):
    """max_num_splits="auto" runs the mode the library picks for the table
    width, and that mode matches the oracle."""
    import torch
    step = make()
    cache = G.build_cache(step, gpu)
    q, tables, ctx, _ = step.decode_batch()
    assert G.pkv.decode_default_max_num_splits(tables.shape[1]) == mode
    G.announce(f"auto-mode decode {step.name} B={len(ctx)} width={tables.shape[1]}")
    out, lse = G.pkv.paged_attention_decode(G.tensor(q, step.q_dtype, gpu), cache, G.ints(tables, gpu),
                                            G.ints(ctx, gpu), None, "auto", float(step.scale), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.decode(step, O.pool(step))
    st = O.compare(out.cpu().numpy(), ro)
    assert st["ok"], st
    st = O.compare(lse.cpu().numpy(), rl)
    assert st["ok"], st
