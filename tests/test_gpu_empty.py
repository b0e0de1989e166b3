"""GPU edge cases with nothing (or nothing for one sequence) to attend: a
zero-length context in split mode, a zero-row chunk beside others, and empty
batches through every entry point."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from tests import gpu_side as G
from tests import oracle_side as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["bf16", "i8"])
@pytest.mark.parametrize("ns", [1, 3])
def test_decode_zero_length_sequence_split_mode(gpu, kv, ns):
    """n = 0 gives out = 0 and lse = -inf (every split empty); its neighbours
    are unaffected."""
    import torch
    step = W.make_step(f"zero_{kv}", [40, 17, 33], [1, 1, 1], num_q_heads=16, num_kv_heads=8, head_dim=128,
                       kv_dtype=kv, src_dtype="bf16", seed=5)
    cache = G.build_cache(step, gpu)
    q, tables, ctx, _ = step.decode_batch()
    ctx = ctx.copy()
    ctx[1] = 0
    nsp = np.full(len(ctx), ns, np.int32)
    G.announce(f"decode with n = 0, kv={kv}, ns={ns}")
    out, lse = G.pkv.paged_attention_decode(G.tensor(q, step.q_dtype, gpu), cache, G.ints(tables, gpu),
                                            G.ints(ctx, gpu), G.ints(nsp, gpu), ns, float(step.scale),
                                            return_lse=True)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    ro, rl = oracle.paged_decode(oracle.decode_rows(q, step.q_dtype), O.pool(step), tables, ctx, step.scale)
    assert (out[1] == 0).all() and np.isneginf(lse[1]).all()
    assert O.compare(out, ro)["ok"] and O.compare(lse, rl)["ok"]


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_chunked_zero_row_chunk(gpu, kv):
    """A sequence with an empty chunk (equal consecutive cu_q_lens) writes no
    rows; the chunks around it are exact."""
    import torch
    step = W.make_step(f"zc_{kv}", [100, 80], [30, 20], num_q_heads=16, num_kv_heads=8, head_dim=128,
                       kv_dtype=kv, src_dtype="bf16", seed=6)
    cache = G.build_cache(step, gpu)
    q, cu, tables, ctx = step.chunk_batch()
    cu3 = np.array([cu[0], cu[1], cu[1], cu[2]], np.int32)
    tables3 = np.stack([tables[0], tables[0], tables[1]])
    ctx3 = np.array([ctx[0], 50, ctx[1]], np.int32)
    G.announce(f"chunked with an empty chunk, kv={kv}")
    out, lse = G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu3, gpu), int(np.diff(cu3).max()),
                                             cache, G.ints(tables3, gpu), G.ints(ctx3, gpu), float(step.scale),
                                             return_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.chunked(step, O.pool(step))
    assert O.compare(out.cpu().numpy(), ro)["ok"] and O.compare(lse.cpu().numpy(), rl)["ok"]


def test_empty_batches_launch_nothing(gpu):
    """Zero tokens, sequences or batch rows: every entry point succeeds and
    the pool is left as it was."""
    import torch
    step = W.make_step("empty", [20], [1], num_q_heads=16, num_kv_heads=8, head_dim=128, kv_dtype="bf16", seed=7)
    cache = G.build_cache(step, gpu)
    torch.cuda.synchronize()
    before = G.cache_bytes(cache)
    kv0 = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=gpu)
    G.announce("empty calls")
    G.pkv.reshape_and_cache(kv0, kv0, torch.empty(0, dtype=torch.int64, device=gpu), cache)
    q0 = torch.empty((0, 16, 128), dtype=torch.bfloat16, device=gpu)
    t0 = torch.empty((0, 2), dtype=torch.int32, device=gpu)
    i0 = torch.empty(0, dtype=torch.int32, device=gpu)
    out = G.pkv.paged_attention_decode(q0, cache, t0, i0, i0, 1, float(step.scale))
    assert tuple(out.shape) == (0, 16, 128)
    out = G.pkv.paged_attention_decode(q0, cache, t0, i0, None, 0, float(step.scale))
    assert tuple(out.shape) == (0, 16, 128)
    out = G.pkv.paged_attention_chunked(q0, torch.zeros(1, dtype=torch.int32, device=gpu), 1, cache, t0, i0,
                                        float(step.scale))
    assert tuple(out.shape) == (0, 16, 128)
    torch.cuda.synchronize()
    assert G.cache_bytes(cache) == before
