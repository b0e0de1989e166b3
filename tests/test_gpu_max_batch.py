"""GPU parity at the largest sizes the decode entry points accept.

- Batch 65535, in split mode (one and two splits) and in the balanced mode.
  The sequences hold 1 to 32 tokens whose blocks are drawn from a small pool
  written by reshape_and_cache, so the pool stays small while the batch, the
  grid and the balanced mode's search over the batch are at full size.
  Sampled outputs (the first, the last and random ones) are checked against
  the oracle one by one.
- max_num_splits 65535, where nearly every split is empty."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from tests import gpu_side as G
from tests import oracle_side as O

pytestmark = pytest.mark.gpu

B_MAX = 65535


@pytest.mark.parametrize("mode", ["one_split", "two_splits", "balanced"])
def test_decode_at_max_batch(gpu, mode):
    import torch
    base = W.make_step("maxb_pool", [512] * 4, [1] * 4, num_q_heads=4, num_kv_heads=2, head_dim=64,
                       kv_dtype="bf16", seed=61)
    cache = G.build_cache(base, gpu)
    _, base_tables, _, _ = base.decode_batch()
    pool_ids = np.unique(base_tables[base_tables >= 0])        # every row of these blocks is written

    rng = np.random.default_rng(62)
    ctx = rng.integers(1, 33, size=B_MAX).astype(np.int32)
    tables = pool_ids[rng.integers(0, len(pool_ids), size=(B_MAX, 2))].astype(np.int32)
    q_bits = W.f32_to_bf16_bits(rng.standard_normal((B_MAX, 4, 64)).astype(np.float32))
    q = G.tensor(q_bits, "bf16", gpu)
    t_tables, t_ctx = G.ints(tables, gpu), G.ints(ctx, gpu)
    G.announce(f"decode at batch {B_MAX}, {mode}")
    if mode == "balanced":
        out, lse = G.pkv.paged_attention_decode(q, cache, t_tables, t_ctx, None, 0, float(base.scale),
                                                return_lse=True)
    else:
        ns = 1 if mode == "one_split" else 2
        out, lse = G.pkv.paged_attention_decode(q, cache, t_tables, t_ctx,
                                                G.ints(np.full(B_MAX, ns, np.int32), gpu), ns,
                                                float(base.scale), return_lse=True)
    torch.cuda.synchronize()
    seqs = np.unique(np.concatenate([[0, B_MAX - 1], rng.integers(0, B_MAX, size=30)]))
    out_s = out[torch.from_numpy(seqs).to(gpu)].cpu().numpy()
    lse_s = lse[torch.from_numpy(seqs).to(gpu)].cpu().numpy()
    ro, rl = oracle.paged_decode(oracle.decode_rows(q_bits[seqs], "bf16"), O.pool(base), tables[seqs], ctx[seqs],
                                 base.scale)
    st = O.compare(out_s, ro)
    assert st["ok"], st
    st = O.compare(lse_s, rl)
    assert st["ok"], st


def test_decode_at_max_split_count(gpu):
    """max_num_splits = 65535, the largest accepted: nearly every split of
    every sequence is empty and must carry no weight in the merge."""
    import torch
    base = W.make_step("maxs_pool", [512] * 4, [1] * 4, num_q_heads=4, num_kv_heads=2, head_dim=64,
                       kv_dtype="bf16", seed=63)
    cache = G.build_cache(base, gpu)
    _, base_tables, _, _ = base.decode_batch()
    pool_ids = np.unique(base_tables[base_tables >= 0])
    rng = np.random.default_rng(64)
    ctx = np.array([1, 700, 1000], np.int32)
    tables = pool_ids[rng.integers(0, len(pool_ids), size=(3, 63))].astype(np.int32)
    ns = np.array([65535, 65535, 777], np.int32)
    q_bits = W.f32_to_bf16_bits(rng.standard_normal((3, 4, 64)).astype(np.float32))
    G.announce("decode with max_num_splits = 65535")
    out, lse = G.pkv.paged_attention_decode(G.tensor(q_bits, "bf16", gpu), cache, G.ints(tables, gpu),
                                            G.ints(ctx, gpu), G.ints(ns, gpu), 65535, float(base.scale),
                                            return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_decode(oracle.decode_rows(q_bits, "bf16"), O.pool(base), tables, ctx, base.scale)
    st = O.compare(out.cpu().numpy(), ro)
    assert st["ok"], st
    st = O.compare(lse.cpu().numpy(), rl)
    assert st["ok"], st
