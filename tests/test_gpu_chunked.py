"""GPU parity: chunked prefill (causal query chunks over a paged prefix, MFMA
kernel) against the oracle, at the tolerance of the decode tests."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_side as G
from tests import oracle_side as O

pytestmark = pytest.mark.gpu


def check(got, ref, what, atol=O.ATOL):
    st = O.compare(got, ref, atol=atol)
    print(f"{what}: max_abs {st['max_abs']:.3g} max_rel {st['max_rel']:.3g} over {st['n']}")
    assert st["ok"], f"{what}: {st}"
    return st


def run_and_check(step, gpu, out_atol=O.ATOL):
    cache = G.build_cache(step, gpu)
    out, lse = G.run_chunked(step, cache, gpu)
    ro, rl = O.chunked(step, O.pool(step))
    check(out, ro, "out", out_atol)
    check(lse, rl, "lse")
    return cache


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_mixed_quantized_prefill_full_size(gpu, kv):
    """4 chunks of 512 rows over a 1536-token prefix, int8 or fp8 KV: every output."""
    step = W.mixed_int8(num_decode=4, kv_dtype=kv)
    run_and_check(step, gpu)


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("lens", [
    ([64], [64]),                  # no prefix, one full tile
    ([200, 77, 1, 130], [70, 77, 1, 65]),  # ragged chunks and prefixes
    ([1000, 33], [300, 17]),
])
def test_chunked_shapes(gpu, kv, lens):
    ctx, ql = lens
    step = W.make_step(f"ch_{kv}", ctx, ql, num_q_heads=16, num_kv_heads=8, head_dim=128, kv_dtype=kv,
                       src_dtype="bf16", seed=80 + len(ctx))
    run_and_check(step, gpu)


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (16, 4), (16, 2)])
def test_chunked_group_sizes(gpu, kv, Hq, Hkv):
    step = W.make_step(f"grp{Hq}_{Hkv}_{kv}", [150, 96], [100, 40], num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128,
                       kv_dtype=kv, seed=90 + Hq)
    run_and_check(step, gpu)


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 1), (4, 4), (16, 2)])
def test_chunked_head_dim_64(gpu, kv, Hq, Hkv):
    """head_dim 64 (the 128-row kernel over 64-dim rows): ragged chunks and
    prefixes, a chunk of exactly one tile, and chunks of a few rows (one-row
    chunks among them), which a head_dim 64 cache also sends to this kernel."""
    import torch
    ctx = [200, 77, 1, 130, 64, 300, 9, 1000]
    ql = [70, 77, 1, 65, 64, 3, 2, 129]
    step = W.make_step(f"d64_{kv}_{Hq}_{Hkv}", ctx, ql, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=64, kv_dtype=kv,
                       src_dtype="bf16", seed=700 + Hq + Hkv)
    cache = G.build_cache(step, gpu)
    q, cu, tables, cc = step.q, step.cu_q_lens, step.block_tables, step.context_lens
    G.announce(f"chunked head_dim 64 {step.name}")
    out, lse = G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu, gpu), max(ql), cache,
                                             G.ints(tables, gpu), G.ints(cc, gpu), float(step.scale), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.oracle.paged_chunked(O.oracle.decode_rows(q, "bf16"), cu, O.pool(step), tables, cc, step.scale)
    check(out.cpu().numpy(), ro, "out")
    check(lse.cpu().numpy(), rl, "lse")


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("n", [65536, 70000])
def test_chunked_context_past_the_lds_block_ids(gpu, kv, n):
    """A 65,536-token context fills the 4,096 block ids the kernel keeps in
    LDS exactly (the variant that reads ids from LDS only); a 70,000-token one
    (4,375 blocks) takes the variant that reads the ids past the first 4,096
    from the table, in the tile loads and (8-bit caches) the V-scale scan."""
    step = W.make_step(f"longctx_{kv}_{n}", [n, 300], [40, 20], num_q_heads=2, num_kv_heads=1, head_dim=128,
                       kv_dtype=kv, src_dtype="bf16", seed=98)
    run_and_check(step, gpu)


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (16, 2)])
def test_chunked_full_prefill_one_long_chunk(gpu, kv, Hq, Hkv):
    """A whole 4,096-token prompt as one chunk with no prefix: every query
    tile's keys end on its own diagonal tile, and the causal mask covers the
    whole range."""
    L = 4096 if Hq == 2 else 1024
    step = W.make_step(f"fullprefill_{kv}_{Hq}", [L], [L], num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128,
                       kv_dtype=kv, src_dtype="bf16", seed=77)
    run_and_check(step, gpu)


def _scale_bf16(bits: np.ndarray, log2: int) -> np.ndarray:
    """bf16 values times 2^log2 (exact for these magnitudes)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** log2)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("log2", [-12, 12])
def test_chunked_quantized_value_magnitudes(gpu, kv, log2):
    """8-bit caches weight V in fp16 with the V scale folded into the weight:
    V values 2^12 times larger (V scales ~130 for int8) stay finite, and 2^12
    times smaller ones put the weights in fp16's subnormal range. The
    absolute bound scales with |V| (any weighting's rounding error does); the
    lse, which does not depend on V, keeps the plain bound. Chunks with no
    prefix give rows that see 1, 2, 3 ... keys."""
    import dataclasses
    step = W.make_step(f"mag_{kv}_{log2}", [64, 300, 90], [64, 120, 90], num_q_heads=16, num_kv_heads=8,
                       head_dim=128, kv_dtype=kv, src_dtype="bf16", seed=97)
    step = dataclasses.replace(step, prefix_v=_scale_bf16(step.prefix_v, log2), new_v=_scale_bf16(step.new_v, log2))
    run_and_check(step, gpu, out_atol=O.ATOL * 2.0 ** max(log2, 0))


def test_chunk_rows_match_decode_at_their_positions(gpu):
    """Cross-path: row r of a chunk equals a decode of the same cache with
    context n - L + r + 1 (both GPU paths, against each other and the oracle)."""
    import torch
    step = W.make_step("xpath", [300], [90], num_q_heads=16, num_kv_heads=8, head_dim=128, kv_dtype="bf16", seed=95)
    cache = G.build_cache(step, gpu)
    out, _ = G.run_chunked(step, cache, gpu)
    q, cu, tables, ctx = step.chunk_batch()
    rows = [0, 1, 45, 89]
    qd = q[rows]
    ctx_d = np.array([300 - 90 + r + 1 for r in rows], np.int32)
    tab = np.repeat(tables, len(rows), axis=0)
    G.announce("decode for cross-path rows")
    od = G.pkv.paged_attention_decode(G.tensor(qd, "bf16", gpu), cache, G.ints(tab, gpu), G.ints(ctx_d, gpu),
                                      None, 1, float(step.scale))
    torch.cuda.synchronize()
    od = od.cpu().numpy()
    for i, r in enumerate(rows):
        assert O.compare(out[r], od[i])["ok"], r


def test_chunked_bad_metadata_gives_nan(gpu):
    """A chunk longer than its context, or than max_q_len, comes out NaN; a
    block id outside the pool poisons its sequence; the others are exact."""
    step = W.make_step("badc", [100, 100, 100], [40, 40, 40], num_q_heads=16, num_kv_heads=8, head_dim=128,
                       kv_dtype="bf16", seed=96)
    cache = G.build_cache(step, gpu)
    ro, _ = O.chunked(step, O.pool(step))
    q, cu, tables, ctx = step.chunk_batch()
    ctx = ctx.copy()
    tables = tables.copy()
    ctx[0] = 30                       # shorter than its 40-row chunk
    tables[1, 2] = step.num_blocks + 3
    G.announce("chunked bad metadata")
    out = G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu, gpu), 40, cache, G.ints(tables, gpu),
                                        G.ints(ctx, gpu), float(step.scale)).cpu().numpy()
    assert np.isnan(out[:80]).all()
    assert O.compare(out[80:], ro[80:])["ok"]


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("Hq,Hkv", [(16, 8), (16, 4), (16, 2)])
def test_multi_token_decode_rows(gpu, kv, Hq, Hkv):
    """The speculative-verification shape: 2..8 new rows per sequence over
    paged histories of very different lengths (one sequence of exactly q_len
    tokens), GQA-packed, through the chunked entry point: row r of a q_len-row
    step sits at position n - q_len + r."""
    ctx = [300, 77, 1025, 8, 129, 2000]
    ql = [2, 4, 8, 8, 5, 7]
    step = W.make_step(f"mtd_{kv}_{Hq}_{Hkv}", ctx, ql, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128,
                       kv_dtype=kv, src_dtype="bf16", seed=95 + Hkv)
    run_and_check(step, gpu)
