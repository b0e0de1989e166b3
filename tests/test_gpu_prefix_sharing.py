"""GPU parity with prefix-shared blocks: sequences whose block tables name the
same physical blocks for a common prefix, so the pool holds one copy of that
prefix's K/V, as a prefix cache hands blocks out (shared prefixes and cached
chunks are the engine-level reuse the course README describes). Only whole
blocks of already-cached tokens are shared; each sequence's new rows stay in
blocks of its own.

The kernels read K/V only through the tables, so aliasing needs no kernel
change. These tests check that:
* decode (split and balanced modes) and chunked outputs over aliased tables
  match the oracle over the same pool and tables;
* a sequence that reads another's blocks gives, bit for bit, the output it gets
  from a private copy of those blocks.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_side as G
from tests import oracle_side as O

pytestmark = pytest.mark.gpu


def share_prefix(step, pairs):
    """Point the first ``nblk`` table entries of sequence ``dst`` at those of
    ``src`` for each ``(src, dst, nblk)``; the shared blocks must hold cached
    prefix tokens of both sequences."""
    t = step.block_tables.copy()
    bs = step.block_size
    for src, dst, nblk in pairs:
        for i in (src, dst):
            assert nblk * bs <= step.context_lens[i] - step.q_lens[i], "shared blocks must be cached prefix"
        t[dst, :nblk] = t[src, :nblk]
    return dataclasses.replace(step, block_tables=t)


def decode_step(kv):
    step = W.make_step(f"share_{kv}", [300, 260, 170, 96, 513, 1], [1] * 6, num_q_heads=16, num_kv_heads=8,
                       head_dim=128, kv_dtype=kv, src_dtype="bf16", seed=61, num_blocks=120)
    return share_prefix(step, [(0, 1, 12), (0, 2, 8), (4, 3, 5)])


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("ns", [1, 3])
def test_decode_over_shared_prefix_blocks(gpu, kv, ns):
    step = decode_step(kv)
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu, num_splits=ns)
    ro, rl = O.decode(step, O.pool(step))
    st = O.compare(out, ro)
    assert st["ok"], st
    st = O.compare(lse, rl)
    assert st["ok"], st


def test_balanced_decode_over_shared_prefix_blocks(gpu):
    step = decode_step("bf16")
    cache = G.build_cache(step, gpu)
    q, tables, ctx, _ = step.decode_batch()
    G.announce(f"balanced decode {step.name} B={len(ctx)}")
    out, lse = G.pkv.paged_attention_decode(G.tensor(q, step.q_dtype, gpu), cache, G.ints(tables, gpu),
                                            G.ints(ctx, gpu), None, 0, float(step.scale), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.decode(step, O.pool(step))
    st = O.compare(out.cpu().numpy(), ro)
    assert st["ok"], st
    st = O.compare(lse.cpu().numpy(), rl)
    assert st["ok"], st


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
def test_chunked_over_shared_prefix_blocks(gpu, kv):
    """Two chunks continue one cached prefix (the second request's prefix
    blocks are the first's), next to a decode row that shares them too."""
    step = W.make_step(f"sharec_{kv}", [700, 690, 300, 650], [100, 64, 1, 130], num_q_heads=16, num_kv_heads=8,
                       head_dim=128, kv_dtype=kv, src_dtype="bf16", seed=62, num_blocks=200)
    step = share_prefix(step, [(0, 1, 20), (0, 2, 10), (0, 3, 32)])
    cache = G.build_cache(step, gpu)
    out, lse = G.run_chunked(step, cache, gpu)
    ro, rl = O.chunked(step, O.pool(step))
    st = O.compare(out, ro)
    assert st["ok"], st
    st = O.compare(lse, rl)
    assert st["ok"], st
    dout, _ = G.run_decode(step, cache, gpu)
    st = O.compare(dout, O.decode(step, O.pool(step))[0])
    assert st["ok"], st


def test_shared_blocks_equal_private_copies_bit_for_bit(gpu):
    """Sequence 1 reads 12 blocks of sequence 0. Copy those blocks' bytes into
    unused pool blocks and point sequence 1 there instead: its output and lse
    must not change by a single bit (the arithmetic cannot depend on where a
    block lives)."""
    step = decode_step("bf16")
    cache = G.build_cache(step, gpu)
    out_a, lse_a = G.run_decode(step, cache, gpu, num_splits=2)
    used = set(int(x) for x in step.block_tables[step.block_tables >= 0].ravel())
    used |= set(int(s) // step.block_size for s in np.concatenate([step.prefix_slots, step.new_slots]))
    free = [b for b in range(step.num_blocks) if b not in used][:12]
    assert len(free) == 12
    src = step.block_tables[0, :12].astype(np.int64)
    dst = np.asarray(free, np.int64)
    si, di = torch.from_numpy(src).to(gpu), torch.from_numpy(dst).to(gpu)
    cache.k[di] = cache.k[si]
    cache.v[di] = cache.v[si]
    t = step.block_tables.copy()
    t[1, :12] = dst
    private = dataclasses.replace(step, block_tables=t)
    out_b, lse_b = G.run_decode(private, cache, gpu, num_splits=2)
    assert out_b.tobytes() == out_a.tobytes()
    assert lse_b.tobytes() == lse_a.tobytes()
