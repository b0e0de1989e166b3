"""Bit-exact indexing probes for the chunked prefill kernel and the balanced
decode, and the full mixed-step decode rows at the split size the benchmark
uses.

Course README "Build an LLM Inference Engine From Scratch", section "The code
asserts its own claims", claim s06: paged attention equals contiguous
attention. On the GPU that is checked two ways that leave no room for
tolerance:

* one-hot probes: every key is zero except a few "hot" keys whose scores
  exceed all others by hundreds (in log2 units), so every other weight
  underflows to exactly 0 and the hot key's weight is exactly 1. The output
  must then be the hot key's stored value row, bit for bit, which is only
  true if the block table sent every row to the right physical slot;
* block placement: moving every block elsewhere in the pool (same logical
  contents, tables remapped) must leave the output bits unchanged.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_side as G
from tests import oracle_side as O

pytestmark = pytest.mark.gpu

HOT_DIMS = 8          # q is 1.0 on dims 0..7 of every head, 0 elsewhere
WARM = 32.0           # key 0 of every sequence: score 8 * 32 = 256
HOT = 128.0           # the hot key: score 8 * 128 = 1024 (powers of two: score * scale is exact)


def _q_rows(T, Hq, D):
    q = np.zeros((T, Hq, D), np.float32)
    q[:, :, :HOT_DIMS] = 1.0
    return W.f32_to_bf16_bits(q)


def _pow2_value_rows(rng, n, Hkv, D, kv):
    """Value rows whose quantization is exact with a power-of-two scale 2^e
    per (token, head): element 0 is +-top * 2^e (top = 127 for int8, 448 for
    fp8), the rest are codes' values times 2^e. float32, exact in bf16."""
    e = rng.integers(-3, 4, size=(n, Hkv, 1)).astype(np.float64)
    if kv == "i8":
        vals = rng.integers(-127, 128, size=(n, Hkv, D)).astype(np.float64)
        top = 127.0
    else:
        codes = rng.integers(0, 0x7F, size=(n, Hkv, D))
        vals = O.oracle.fp8_e4m3_value(codes) * np.where(rng.random((n, Hkv, D)) < 0.5, -1.0, 1.0)
        top = 448.0
    vals[:, :, 0] = top * np.where(rng.random((n, Hkv)) < 0.5, -1.0, 1.0)
    return (vals * 2.0 ** e).astype(np.float32)


def _write(step, K, V, cache, gpu):
    """Write full sequences' K/V rows (float32 [n][Hkv][D] each) to the GPU
    cache and to an oracle pool; returns the oracle pool."""
    import torch
    Ks = np.concatenate(K)
    Vs = np.concatenate(V)
    slots = np.concatenate([step.block_tables[i, np.arange(len(K[i])) // 16].astype(np.int64) * 16
                            + np.arange(len(K[i])) % 16 for i in range(len(K))])
    Kb, Vb = W.f32_to_bf16_bits(Ks), W.f32_to_bf16_bits(Vs)
    G.pkv.reshape_and_cache(G.tensor(Kb, "bf16", gpu), G.tensor(Vb, "bf16", gpu), G.ints(slots, gpu, torch.int64),
                            cache)
    pool = O.oracle.OraclePool(step.num_blocks, step.num_kv_heads, 16, step.head_dim, step.kv_dtype)
    O.oracle.reshape_and_cache(pool, Kb, Vb, "bf16", slots)
    return pool


def _stored_rows(pool, table_row, n):
    """The value rows as stored, decoded exactly, in float32 [n][Hkv][D]."""
    _, Vs = O.oracle.gather_kv(pool, table_row, n)
    return Vs.astype(np.float32)


# ---------------------------------------------------------------------------
# chunked prefill
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("Hq,Hkv,D", [(16, 8, 128), (16, 4, 128), (16, 8, 64)])
def test_chunked_one_hot_rows_before_on_and_after_the_hot_key(gpu, kv, Hq, Hkv, D):
    """Every sequence holds a warm key at token 0 and one hot key at token j;
    all other keys are zero. Chunk rows at positions before j see only the
    warm key (out == V_0); the row on j and the rows after it see the hot
    key (out == V_j), bit for bit. j sits on a tile boundary, inside a tile
    and on the chunk's last row. bf16 caches run the PV product on a bf16
    high part (1.0) and residual (0); 8-bit caches on fp16 weights with the
    V scale folded in, exact here because the V scales are powers of two."""
    import torch
    ctx, ql, hot = [300, 200, 130], [200, 64, 130], [128, 170, 129]
    step = W.make_step(f"ch1hot_{kv}", ctx, ql, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, kv_dtype=kv,
                       src_dtype="bf16", seed=300)
    rng = np.random.default_rng(301)
    K, V = [], []
    for n, j in zip(ctx, hot):
        k = np.zeros((n, Hkv, D), np.float32)
        k[0, :, :HOT_DIMS] = WARM
        k[j, :, :HOT_DIMS] = HOT
        K.append(k)
        V.append(rng.standard_normal((n, Hkv, D)).astype(np.float32) if kv == "bf16"
                 else _pow2_value_rows(rng, n, Hkv, D, kv))
    cache = G.pkv.KVCache.allocate(step.num_blocks, Hkv, D, G.CODE[kv], gpu)
    pool = _write(step, K, V, cache, gpu)
    T = int(sum(ql))
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    G.announce(f"chunked one-hot kv={kv} Hq={Hq} Hkv={Hkv}")
    out = G.pkv.paged_attention_chunked(G.tensor(_q_rows(T, Hq, D), "bf16", gpu), G.ints(cu, gpu), max(ql), cache,
                                        G.ints(step.block_tables, gpu), G.ints(np.array(ctx), gpu), 1.0)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    grp = Hq // Hkv
    for i, (n, L, j) in enumerate(zip(ctx, ql, hot)):
        Vs = _stored_rows(pool, step.block_tables[i], n)
        for r in range(L):
            pos = n - L + r
            src = j if pos >= j else 0
            for h in range(Hq):
                got = out[cu[i] + r, h]
                assert np.array_equal(got, Vs[src, h // grp]), (kv, i, r, pos, h, src)


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_chunked_output_is_bit_identical_under_block_placement(gpu, kv):
    """Claim s06 for the chunked kernel: the same logical cache with every
    block moved elsewhere in the pool gives the same output bits."""
    import torch
    step = W.make_step(f"chplace_{kv}", [700, 300, 129], [300, 64, 100], num_q_heads=16, num_kv_heads=8,
                       head_dim=128, kv_dtype=kv, src_dtype="bf16", seed=302)
    cache = G.build_cache(step, gpu)
    out1, lse1 = G.run_chunked(step, cache, gpu)
    perm = np.random.default_rng(6).permutation(step.num_blocks)
    cache2 = G.pkv.KVCache.allocate(step.num_blocks, 8, 128, G.CODE[kv], gpu)
    pt = torch.from_numpy(perm).to(gpu)
    cache2.k[pt] = cache.k
    cache2.v[pt] = cache.v
    if cache.k_scale is not None:
        cache2.k_scale[pt] = cache.k_scale
        cache2.v_scale[pt] = cache.v_scale
    step.block_tables = np.where(step.block_tables >= 0, perm[np.maximum(step.block_tables, 0)], -1).astype(np.int32)
    out2, lse2 = G.run_chunked(step, cache2, gpu)
    assert out1.tobytes() == out2.tobytes() and lse1.tobytes() == lse2.tobytes()
    assert np.isfinite(out1).all()


# ---------------------------------------------------------------------------
# balanced decode (segments cut between wavefronts)
# ---------------------------------------------------------------------------

def _balanced(step_q, cache, tables, ctx, gpu, scale):
    import torch
    G.announce(f"balanced decode B={len(ctx)}")
    out, lse = G.pkv.paged_attention_decode(G.tensor(step_q, "bf16", gpu), cache, G.ints(tables, gpu),
                                            G.ints(ctx, gpu), None, 0, scale, return_lse=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_balanced_one_hot_with_cut_segments(gpu, kv):
    """16 sequences of 1000-1200 tokens x 8 kv heads: about 8,800 tiles over
    the balanced mode's 1,024 wavefronts, so every (sequence, kv head) is cut
    between about eight wavefronts and merged by the last to finish. One hot
    key per sequence, at a seeded position; every other key is zero. The
    output must be the hot value row, bit for bit (int8: value(code) * scale
    rounded once to float32), whichever wavefront held it."""
    B, Hq, Hkv, D = 16, 16, 8, 128
    rng = np.random.default_rng(303)
    ctx = rng.integers(1000, 1201, size=B)
    step = W.make_step(f"bal1hot_{kv}", ctx, np.ones(B, np.int64), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                       kv_dtype=kv, src_dtype="bf16", seed=304)
    hot = [int(rng.integers(0, n)) for n in ctx]
    K, V = [], []
    for n, j in zip(ctx, hot):
        k = np.zeros((n, Hkv, D), np.float32)
        k[j, :, :HOT_DIMS] = HOT
        K.append(k)
        V.append(rng.standard_normal((n, Hkv, D)).astype(np.float32))
    cache = G.pkv.KVCache.allocate(step.num_blocks, Hkv, D, G.CODE[kv], gpu)
    pool = _write(step, K, V, cache, gpu)
    assert len(ctx) * Hkv * step.block_tables.shape[1] <= 65536    # 256 workgroups x 4 wavefronts
    out, _ = _balanced(_q_rows(B, Hq, D), cache, step.block_tables, ctx.astype(np.int32), gpu, 1.0)
    for b in range(B):
        Vs = _stored_rows(pool, step.block_tables[b], int(ctx[b]))
        for h in range(Hq):
            assert np.array_equal(out[b, h], Vs[hot[b], h // 2]), (kv, b, h, hot[b])


def test_balanced_output_is_bit_identical_under_block_placement(gpu):
    """The balanced deal depends on the context lengths only, so moving the
    blocks in the pool leaves every partial, and the merged output, bit for
    bit the same."""
    import torch
    step = W.ragged_decode(batch=40, seed=305)
    cache = G.build_cache(step, gpu)
    q, tables, ctx, _ = step.decode_batch()
    out1, lse1 = _balanced(q, cache, tables, ctx, gpu, float(step.scale))
    perm = np.random.default_rng(7).permutation(step.num_blocks)
    cache2 = G.pkv.KVCache.allocate(step.num_blocks, 8, 128, G.pkv.BF16, gpu)
    pt = torch.from_numpy(perm).to(gpu)
    cache2.k[pt] = cache.k
    cache2.v[pt] = cache.v
    tables2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    out2, lse2 = _balanced(q, cache2, tables2, ctx, gpu, float(step.scale))
    assert out1.tobytes() == out2.tobytes() and lse1.tobytes() == lse2.tobytes()
    assert np.isfinite(out1).all()


# ---------------------------------------------------------------------------
# the mixed step's decode rows, as the benchmark runs them
# ---------------------------------------------------------------------------

@pytest.mark.slow
@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_mixed_step_all_decode_rows_at_1024_token_splits(gpu, kv):
    """All 124 decode rows of the mixed step (n uniform in [256, 4096]) at
    ceil(n / 1024) splits each, the split plan the benchmark times, against the
    oracle: every output element and lse."""
    step = W.mixed_int8(kv_dtype=kv, max_tokens_per_split=1024)
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu)
    ro, rl = O.decode(step, O.pool(step))
    assert out.shape == (124, 16, 128)
    for got, ref, what in ((out, ro, "out"), (lse, rl, "lse")):
        st = O.compare(got, ref)
        print(f"{what}: {st}")
        assert st["ok"], (what, st)
