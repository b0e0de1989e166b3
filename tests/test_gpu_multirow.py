"""GPU parity of the chunked entry point's paths for chunks of a few rows
(speculative verification: k draft rows per sequence). When max_q_len times
the GQA group is at most 2 (4 with head_dim 64), the rows are computed by the
decode kernels (up to 16, with head_dim 128: by a decode-shaped kernel on
16x16 MFMAs), every chunk row of a kv head's query heads on each K/V tile, with row r of an
L-row chunk seeing tokens t <= n - L + r. Same tolerance as the other decode
tests; indexing checked bit for bit with a one-hot probe."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_side as G
from tests import oracle_side as O

pytestmark = pytest.mark.gpu


def check(got, ref, what):
    st = O.compare(got, ref)
    print(f"{what}: max_abs {st['max_abs']:.3g} max_rel {st['max_rel']:.3g} over {st['n']}")
    assert st["ok"], f"{what}: {st}"


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("Hq,Hkv,ql", [
    (8, 8, [2, 1, 2, 2, 1, 2]),        # group 1: up to 2 rows
    (8, 4, [1, 1, 1, 1, 1, 1]),        # group 2: one row per sequence through the chunked call
    (16, 16, [1, 1, 1, 1, 1, 1]),      # group 1: one row
])
def test_few_row_chunks_match_oracle(gpu, kv, Hq, Hkv, ql):
    """head_dim 128, up to 2 rows per kv head: the decode kernels."""
    ctx = [300, 77, 1025, 8, 129, 2000]
    step = W.make_step(f"rows_{kv}_{Hq}_{Hkv}", ctx, ql, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128,
                       kv_dtype=kv, src_dtype="bf16", seed=600 + Hkv + max(ql))
    assert G.pkv.chunked_kernel_for(max(ql), Hq, Hkv, 128) == G.pkv.CHUNKED_DECODE_ROWS
    cache = G.build_cache(step, gpu)
    # every sequence's rows as one chunk each (one-row chunks included)
    q, cu, tables, ctx = step.q, step.cu_q_lens, step.block_tables, step.context_lens
    G.announce(f"few-row chunks {step.name} max_q_len={max(ql)}")
    out, lse = G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu, gpu), max(ql), cache,
                                             G.ints(tables, gpu), G.ints(ctx, gpu), float(step.scale),
                                             return_lse=True)
    import torch
    torch.cuda.synchronize()
    ro, rl = O.oracle.paged_chunked(O.oracle.decode_rows(q, "bf16"), cu, O.pool(step), tables, ctx, step.scale)
    check(out.cpu().numpy(), ro, "out")
    check(lse.cpu().numpy(), rl, "lse")


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("Hq,Hkv,ql", [
    (8, 4, [2, 1, 2, 2, 1, 2]),        # group 2: up to 4 rows per kv head, the decode kernels
    (4, 4, [4, 3, 1, 4, 4, 2]),        # group 1: up to 4 rows
    (8, 2, [3, 1, 4, 2, 4, 1]),        # group 4 x up to 4 rows: 16 rows per kv head, the chunk kernel
])
def test_few_row_chunks_head_dim_64(gpu, kv, Hq, Hkv, ql):
    """head_dim 64: chunks of up to 4 rows per kv head run on the decode
    kernels, longer ones (the MFMA few-row kernel is built for 128) on the
    chunk kernel; both against the oracle."""
    import torch
    ctx = [300, 77, 1025, 8, 129, 2000]
    step = W.make_step(f"rows64_{kv}_{Hq}_{Hkv}", ctx, ql, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=64,
                       kv_dtype=kv, src_dtype="bf16", seed=640 + Hkv + max(ql))
    rows = max(ql) * (Hq // Hkv)
    assert G.pkv.chunked_kernel_for(max(ql), Hq, Hkv, 64) == (
        G.pkv.CHUNKED_DECODE_ROWS if rows <= 4 else G.pkv.CHUNKED_TILES)
    cache = G.build_cache(step, gpu)
    q, cu, tables, cc = step.q, step.cu_q_lens, step.block_tables, step.context_lens
    G.announce(f"few-row chunks head_dim 64 {step.name}")
    out, lse = G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu, gpu), max(ql), cache,
                                             G.ints(tables, gpu), G.ints(cc, gpu), float(step.scale),
                                             return_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.oracle.paged_chunked(O.oracle.decode_rows(q, "bf16"), cu, O.pool(step), tables, cc, step.scale)
    check(out.cpu().numpy(), ro, "out")
    check(lse.cpu().numpy(), rl, "lse")


def test_spec_verify_shape_matches_oracle(gpu):
    """The benchmark's verification shape: 32 sequences of 128..384 tokens,
    4 new rows each, Qwen3 heads, bf16 (8 rows per kv head: the MFMA kernel)."""
    rng = np.random.default_rng(np.random.SeedSequence([1906, 7]))
    ctx = rng.integers(128, 384, size=32, endpoint=True)
    step = W.make_step("spec_verify", ctx, np.full(32, 4), num_q_heads=16, num_kv_heads=8, head_dim=128,
                       num_blocks=4096, seed=1906)
    assert G.pkv.chunked_kernel_for(4, 16, 8, 128) == G.pkv.CHUNKED_ROWS_MFMA
    cache = G.build_cache(step, gpu)
    out, lse = G.run_chunked(step, cache, gpu)
    ro, rl = O.chunked(step, O.pool(step))
    check(out, ro, "out")
    check(lse, rl, "lse")


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_few_row_one_hot_rows_before_and_after_the_hot_key(gpu, kv):
    """2 rows per sequence at positions n-2, n-1 (one query head per kv head,
    2 rows per kv head: the decode kernels); key 0 is warm, key n-1 is hot,
    every other key zero: row n-2 returns V_0 and row n-1 returns V_{n-1}, bit
    for bit."""
    import torch
    Hq, Hkv, D = 8, 8, 128
    ctx = [300, 45, 17]
    ql = [2, 2, 2]
    assert G.pkv.chunked_kernel_for(2, Hq, Hkv, D) == G.pkv.CHUNKED_DECODE_ROWS
    step = W.make_step(f"rows1hot_{kv}", ctx, ql, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, kv_dtype=kv,
                       src_dtype="bf16", seed=610)
    rng = np.random.default_rng(611)
    slots, Ks, Vs = [], [], []
    for i, n in enumerate(ctx):
        k = np.zeros((n, Hkv, D), np.float32)
        k[0, :, :8] = 32.0
        k[n - 1, :, :8] = 128.0
        Ks.append(k)
        Vs.append(rng.standard_normal((n, Hkv, D)).astype(np.float32))
        t = np.arange(n)
        slots.append(step.block_tables[i, t // 16].astype(np.int64) * 16 + t % 16)
    Kb, Vb = W.f32_to_bf16_bits(np.concatenate(Ks)), W.f32_to_bf16_bits(np.concatenate(Vs))
    sl = np.concatenate(slots)
    cache = G.pkv.KVCache.allocate(step.num_blocks, Hkv, D, G.CODE[kv], gpu)
    G.pkv.reshape_and_cache(G.tensor(Kb, "bf16", gpu), G.tensor(Vb, "bf16", gpu), G.ints(sl, gpu, torch.int64), cache)
    pool = O.oracle.OraclePool(step.num_blocks, Hkv, 16, D, kv)
    O.oracle.reshape_and_cache(pool, Kb, Vb, "bf16", sl)
    qv = np.zeros((sum(ql), Hq, D), np.float32)
    qv[:, :, :8] = 1.0
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    G.announce(f"few-row one-hot kv={kv}")
    out = G.pkv.paged_attention_chunked(G.tensor(W.f32_to_bf16_bits(qv), "bf16", gpu), G.ints(cu, gpu), 2, cache,
                                        G.ints(step.block_tables, gpu), G.ints(np.array(ctx), gpu), 1.0)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for i, n in enumerate(ctx):
        _, V = O.oracle.gather_kv(pool, step.block_tables[i], n)
        for r in range(2):
            src = n - 1 if n - 2 + r >= n - 1 else 0
            for h in range(Hq):
                assert np.array_equal(out[cu[i] + r, h], V[src, h].astype(np.float32)), (kv, i, r, h)


def test_few_row_path_agrees_with_the_mfma_path(gpu):
    """The same 2-row chunks through the decode kernels (8 q / 8 kv heads,
    2 rows per kv head) and, with a larger max_q_len, through the 128-row MFMA
    kernel: both within tolerance of the oracle and of each other."""
    import torch
    step = W.make_step("rows_vs_mfma", [300, 77, 1025], [2, 2, 2], num_q_heads=8, num_kv_heads=8, head_dim=128,
                       seed=612)
    cache = G.build_cache(step, gpu)
    q, cu, tables, ctx = step.chunk_batch()
    args = (G.tensor(q, "bf16", gpu), G.ints(cu, gpu))
    G.announce("few-row vs MFMA path")
    a = G.pkv.paged_attention_chunked(*args, 2, cache, G.ints(tables, gpu), G.ints(ctx, gpu), float(step.scale))
    b = G.pkv.paged_attention_chunked(*args, 64, cache, G.ints(tables, gpu), G.ints(ctx, gpu), float(step.scale))
    torch.cuda.synchronize()
    a, b = a.cpu().numpy(), b.cpu().numpy()
    ro, _ = O.chunked(step, O.pool(step))
    check(a, ro, "few-row")
    check(b, ro, "mfma")
    check(a, b.astype(np.float64), "few-row vs mfma")


def test_few_row_bad_metadata_and_empty_chunks(gpu):
    """A chunk longer than its context or than max_q_len comes out NaN, an
    out-of-pool block id poisons its sequence, a zero-row chunk writes
    nothing, and the other sequences are unaffected (2-row chunks, 2 rows per
    kv head: the decode kernels)."""
    import torch
    step = W.make_step("rows_bad", [100, 100, 100, 100], [2, 2, 2, 2], num_q_heads=8, num_kv_heads=8,
                       head_dim=128, seed=613)
    cache = G.build_cache(step, gpu)
    ro, _ = O.chunked(step, O.pool(step))
    q, cu, tables, ctx = step.chunk_batch()
    ctx = ctx.copy()
    tables = tables.copy()
    ctx[0] = 1                         # shorter than its 2-row chunk
    tables[1, 3] = step.num_blocks + 4
    cu2 = cu.copy()
    cu2[3] = cu2[2]                    # sequence 2 has an empty chunk; sequence 3 takes 4 rows
    G.announce("few-row bad metadata")
    out = torch.full((len(q), 8, 128), 7.0, dtype=torch.float32, device=gpu)
    G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu2, gpu), 2, cache, G.ints(tables, gpu),
                                  G.ints(ctx, gpu), float(step.scale), out=out)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.isnan(out[0:2]).all()          # sequence 0: chunk longer than its context
    assert np.isnan(out[2:4]).all()          # sequence 1: block id outside the pool
    assert np.isnan(out[4:8]).all()          # sequence 3: 4 rows > max_q_len = 2
    G.announce("few-row clean rerun")
    out2 = G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu, gpu), 2, cache,
                                         G.ints(step.chunk_batch()[2], gpu), G.ints(step.chunk_batch()[3], gpu),
                                         float(step.scale))
    torch.cuda.synchronize()
    check(out2.cpu().numpy(), ro, "clean rerun")


# ---------------------------------------------------------------------------
# 3 .. 16 rows per kv head: the decode-shaped MFMA kernel
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("Hq,Hkv,ql", [
    (16, 8, [4, 3, 1, 4, 2, 4]),       # group 2: up to 4 rows (8 rows per kv head), the verify shape
    (16, 8, [8, 5, 1, 8, 8, 2]),       # group 2: up to 8 rows (16 rows per kv head)
    (8, 8, [16, 9, 1, 16, 7, 12]),     # group 1: up to 16 rows
    (16, 4, [4, 1, 3, 4, 2, 4]),       # group 4: up to 4 rows
    (16, 2, [2, 1, 2, 2, 1, 2]),       # group 8: up to 2 rows
    (16, 8, [2, 1, 2, 2, 1, 2]),       # group 2: up to 2 rows (4 rows per kv head)
    (8, 8, [4, 3, 1, 4, 4, 2]),        # group 1: up to 4 rows
    (8, 8, [3, 1, 3, 2, 3, 3]),        # group 1: up to 3 rows
    (16, 4, [1, 1, 1, 1, 1, 1]),       # group 4: one row per sequence
])
def test_mfma_few_row_chunks_match_oracle(gpu, kv, Hq, Hkv, ql):
    """Contexts from 16 tokens to 5,000 (more than 64 blocks per wavefront,
    so the block ids are read in several rounds)."""
    import torch
    ctx = [300, 77, 5000, 16, 129, 2000]
    step = W.make_step(f"mrows_{kv}_{Hq}_{Hkv}", ctx, ql, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128,
                       kv_dtype=kv, src_dtype="bf16", seed=700 + Hkv + max(ql))
    assert G.pkv.chunked_kernel_for(max(ql), Hq, Hkv, 128) == G.pkv.CHUNKED_ROWS_MFMA
    cache = G.build_cache(step, gpu)
    q, cu, tables, ctx_ = step.q, step.cu_q_lens, step.block_tables, step.context_lens
    G.announce(f"MFMA few-row chunks {step.name} max_q_len={max(ql)}")
    out, lse = G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu, gpu), max(ql), cache,
                                             G.ints(tables, gpu), G.ints(ctx_, gpu), float(step.scale),
                                             return_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.oracle.paged_chunked(O.oracle.decode_rows(q, "bf16"), cu, O.pool(step), tables, ctx_, step.scale)
    check(out.cpu().numpy(), ro, "out")
    check(lse.cpu().numpy(), rl, "lse")


def _pow2_v(rng, n, Hkv, D):
    """int8-quantizable value rows with power-of-two scales (exact weights)."""
    e = rng.integers(-3, 4, size=(n, Hkv, 1)).astype(np.float64)
    vals = rng.integers(-127, 128, size=(n, Hkv, D)).astype(np.float64)
    vals[:, :, 0] = 127.0 * np.where(rng.random((n, Hkv)) < 0.5, -1.0, 1.0)
    return (vals * 2.0 ** e).astype(np.float32)


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_mfma_few_row_one_hot(gpu, kv):
    """8 rows per kv head (4 rows x 2 heads) at positions n-4 .. n-1; key 0 is
    warm, key n-2 hot, the rest zero: rows n-4, n-3 return V_0 and rows n-2,
    n-1 return V_{n-2}, bit for bit (int8 with power-of-two V scales, so the
    weight's bf16 high part carries it whole)."""
    import torch
    Hq, Hkv, D = 16, 8, 128
    ctx = [300, 45, 17, 1100]
    ql = [4, 4, 4, 4]
    assert G.pkv.chunked_kernel_for(4, Hq, Hkv, D) == G.pkv.CHUNKED_ROWS_MFMA
    step = W.make_step(f"mrows1hot_{kv}", ctx, ql, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, kv_dtype=kv,
                       src_dtype="bf16", seed=710)
    rng = np.random.default_rng(711)
    slots, Ks, Vs = [], [], []
    for i, n in enumerate(ctx):
        k = np.zeros((n, Hkv, D), np.float32)
        k[0, :, :8] = 32.0
        k[n - 2, :, :8] = 128.0
        Ks.append(k)
        Vs.append(rng.standard_normal((n, Hkv, D)).astype(np.float32) if kv == "bf16" else _pow2_v(rng, n, Hkv, D))
        t = np.arange(n)
        slots.append(step.block_tables[i, t // 16].astype(np.int64) * 16 + t % 16)
    Kb, Vb = W.f32_to_bf16_bits(np.concatenate(Ks)), W.f32_to_bf16_bits(np.concatenate(Vs))
    sl = np.concatenate(slots)
    cache = G.pkv.KVCache.allocate(step.num_blocks, Hkv, D, G.CODE[kv], gpu)
    G.pkv.reshape_and_cache(G.tensor(Kb, "bf16", gpu), G.tensor(Vb, "bf16", gpu), G.ints(sl, gpu, torch.int64), cache)
    pool = O.oracle.OraclePool(step.num_blocks, Hkv, 16, D, kv)
    O.oracle.reshape_and_cache(pool, Kb, Vb, "bf16", sl)
    qv = np.zeros((sum(ql), Hq, D), np.float32)
    qv[:, :, :8] = 1.0
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    G.announce(f"MFMA few-row one-hot kv={kv}")
    out = G.pkv.paged_attention_chunked(G.tensor(W.f32_to_bf16_bits(qv), "bf16", gpu), G.ints(cu, gpu), 4, cache,
                                        G.ints(step.block_tables, gpu), G.ints(np.array(ctx), gpu), 1.0)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for i, n in enumerate(ctx):
        _, V = O.oracle.gather_kv(pool, step.block_tables[i], n)
        for r in range(4):
            src = n - 2 if n - 4 + r >= n - 2 else 0
            for h in range(Hq):
                assert np.array_equal(out[cu[i] + r, h], V[src, h // 2].astype(np.float32)), (kv, i, r, h)


def test_mfma_few_row_path_agrees_with_the_chunked_kernel(gpu):
    """The same 8-row chunks through the few-row MFMA kernel (max_q_len 8,
    16 rows per kv head) and the 128-row chunked kernel (max_q_len 64)."""
    import torch
    step = W.make_step("mrows_vs_chunked", [300, 77, 1025, 4000], [8, 8, 8, 8], num_q_heads=16, num_kv_heads=8,
                       head_dim=128, kv_dtype="i8", seed=712)
    cache = G.build_cache(step, gpu)
    q, cu, tables, ctx = step.chunk_batch()
    args = (G.tensor(q, "bf16", gpu), G.ints(cu, gpu))
    G.announce("MFMA few-row vs chunked kernel")
    a = G.pkv.paged_attention_chunked(*args, 8, cache, G.ints(tables, gpu), G.ints(ctx, gpu), float(step.scale))
    b = G.pkv.paged_attention_chunked(*args, 64, cache, G.ints(tables, gpu), G.ints(ctx, gpu), float(step.scale))
    torch.cuda.synchronize()
    a, b = a.cpu().numpy(), b.cpu().numpy()
    ro, _ = O.chunked(step, O.pool(step))
    check(a, ro, "few-row MFMA")
    check(b, ro, "chunked")


def test_mfma_few_row_bad_metadata(gpu):
    """The MFMA few-row path turns a chunk longer than its context or than
    max_q_len, and an out-of-pool block id, into NaN rows of that sequence
    only."""
    import torch
    step = W.make_step("mrows_bad", [100, 100, 100, 100], [4, 4, 4, 4], num_q_heads=16, num_kv_heads=8,
                       head_dim=128, seed=713)
    cache = G.build_cache(step, gpu)
    ro, _ = O.chunked(step, O.pool(step))
    q, cu, tables, ctx = step.chunk_batch()
    ctx = ctx.copy()
    tables = tables.copy()
    ctx[0] = 3                         # shorter than its 4-row chunk
    tables[1, 5] = step.num_blocks + 4
    cu2 = cu.copy()
    cu2[3] = cu2[2]                    # sequence 2 has an empty chunk; sequence 3 takes 8 rows
    G.announce("MFMA few-row bad metadata")
    out = torch.full((len(q), 16, 128), 7.0, dtype=torch.float32, device=gpu)
    G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu2, gpu), 4, cache, G.ints(tables, gpu),
                                  G.ints(ctx, gpu), float(step.scale), out=out)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.isnan(out[0:4]).all()
    assert np.isnan(out[4:8]).all()
    assert np.isnan(out[8:16]).all()   # 8 rows > max_q_len = 4
