"""GPU parity: reshape_and_cache and split-K paged decode against the oracle.

Tolerance (float): |gpu - oracle| <= 2e-3 + 1e-2 |oracle| per element, the
(max-abs 2e-3, max-rel 1e-2) pair for bf16 inputs, float32 accumulation and a
float64 oracle. Indexing work (the cache bytes, the one-hot probe, the
placement-permutation check) is compared bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_side as G
from tests import oracle_side as O

pytestmark = pytest.mark.gpu


def check(got, ref, what):
    st = O.compare(got, ref)
    assert st["ok"], f"{what}: {st}"
    return st


# ---------------------------------------------------------------------------
# reshape_and_cache: bit-exact pool bytes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("make", [
    lambda: W.tiny_decode(),
    lambda: W.qwen3_decode(batch=8),
    lambda: W.make_step("q8", [300, 77, 1, 16, 17], [300, 1, 1, 1, 5], num_q_heads=16, num_kv_heads=8,
                        head_dim=128, kv_dtype="i8", src_dtype="bf16", seed=41, num_blocks=40),
    lambda: W.make_step("q8f", [40, 33], [3, 1], num_q_heads=4, num_kv_heads=2, head_dim=64, q_dtype="f32",
                        kv_dtype="i8", src_dtype="f32", seed=42),
    lambda: W.make_step("bf64", [40, 33], [1, 1], num_q_heads=8, num_kv_heads=2, head_dim=64, seed=43),
    lambda: W.make_step("f8", [300, 77, 1, 16, 17], [300, 1, 1, 1, 5], num_q_heads=16, num_kv_heads=8,
                        head_dim=128, kv_dtype="fp8", src_dtype="bf16", seed=44, num_blocks=40),
    lambda: W.make_step("f8f", [40, 33], [3, 1], num_q_heads=4, num_kv_heads=2, head_dim=64, q_dtype="f32",
                        kv_dtype="fp8", src_dtype="f32", seed=45),
], ids=["tiny_f32", "qwen3_bf16", "int8_from_bf16", "int8_from_f32_d64", "bf16_d64", "fp8_from_bf16",
        "fp8_from_f32_d64"])
def test_reshape_and_cache_bytes_match_oracle(gpu, make):
    step = make()
    G.announce(f"reshape {step.name}")
    got = G.cache_bytes(G.build_cache(step, gpu))
    ref = O.pool_bytes(O.pool(step))
    for name in ref:
        assert got[name] == ref[name], name


def _quantizer_edge_rows(kv: str, T: int, H: int, D: int, seed: int) -> np.ndarray:
    """float32 rows [T][H][D] whose first element sets amax so that the scale is
    a power of two s exactly (amax = 127 s or 448 s), the rest placed at the
    quantizer's hard cases times s: for int8 the quotients k + 1/2 and a few
    ulps either side; for fp8 the midpoints between neighbouring E4M3 values,
    their float32 neighbours, and the subnormal range below 2^-6."""
    rng = np.random.default_rng(seed)
    top = 127.0 if kv == "i8" else 448.0
    if kv == "i8":
        k = np.arange(-127, 127, dtype=np.float64)
        hard = np.float32(k + 0.5)
    else:
        pos = O.oracle.fp8_e4m3_value(np.arange(0x7F))
        hard = np.float32((pos[:-1] + pos[1:]) / 2)
        hard = np.concatenate([hard, np.float32(rng.uniform(0, 2.0 ** -6, 200))])
    hard = np.concatenate([hard, np.nextafter(hard, np.float32(0)), np.nextafter(hard, np.float32(1e9))])
    hard = np.concatenate([hard, -hard]).astype(np.float32)
    rows = np.empty((T, H, D), np.float32)
    for t in range(T):
        for h in range(H):
            e = int(rng.integers(-6, 7))
            sc = np.float32(2.0 ** e)
            rows[t, h, 0] = np.float32(top) * sc * (1 if rng.random() < 0.5 else -1)
            rows[t, h, 1:] = rng.choice(hard, D - 1) * sc
    return rows


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_quantizer_hard_cases_bit_exact(gpu, kv):
    """Quotients on and next to the rounding boundaries (and, for fp8, in the
    subnormal range): the cache bytes must equal the oracle's."""
    import torch
    T, H, D = 64, 2, 64
    K = _quantizer_edge_rows(kv, T, H, D, 7)
    V = _quantizer_edge_rows(kv, T, H, D, 8)
    slots = np.random.default_rng(9).permutation(4 * 16)[:T].astype(np.int64)
    cache = G.pkv.KVCache.allocate(4, H, D, G.CODE[kv], gpu)
    G.announce(f"reshape hard cases {kv}")
    G.pkv.reshape_and_cache(G.tensor(K, "f32", gpu), G.tensor(V, "f32", gpu), G.ints(slots, gpu, torch.int64), cache)
    torch.cuda.synchronize()
    p = O.oracle.OraclePool(4, H, 16, D, kv)
    O.oracle.reshape_and_cache(p, K, V, "f32", slots)
    got, ref = G.cache_bytes(cache), O.pool_bytes(p)
    for name in ref:
        assert got[name] == ref[name], name


def test_reshape_skips_negative_and_out_of_range_slots(gpu):
    import torch
    step = W.make_step("skip", [20], [20], num_q_heads=4, num_kv_heads=2, head_dim=64, seed=44, num_blocks=4)
    slots = step.new_slots.copy()
    slots[3] = -1
    slots[5] = step.num_blocks * 16 + 7     # past the pool: skipped like a negative slot
    cache = G.pkv.KVCache.allocate(step.num_blocks, 2, 64, G.pkv.BF16, gpu)
    G.announce("reshape skip")
    G.pkv.reshape_and_cache(G.tensor(step.new_k, "bf16", gpu), G.tensor(step.new_v, "bf16", gpu),
                            G.ints(slots, gpu, torch.int64), cache)
    keep = np.ones(len(slots), bool)
    keep[[3, 5]] = False
    p = O.oracle.OraclePool(step.num_blocks, 2, 16, 64, "bf16")
    O.oracle.reshape_and_cache(p, step.new_k[keep], step.new_v[keep], "bf16", slots[keep])
    assert G.cache_bytes(cache)["k"] == O.pool_bytes(p)["k"]


# ---------------------------------------------------------------------------
# decode parity
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ns", [1, 2, 3])
def test_tiny_decode(gpu, ns):
    step = W.tiny_decode(num_splits=ns)
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu)
    ro, rl = O.decode(step, O.pool(step))
    check(out, ro, "out")
    check(lse, rl, "lse")


@pytest.mark.parametrize("max_tok", [None, 64, 128, 256])
def test_qwen3_decode_full_size(gpu, max_tok):
    step = W.qwen3_decode(max_tokens_per_split=max_tok)
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu)
    ro, rl = O.decode(step, O.pool(step))
    check(out, ro, "out")
    check(lse, rl, "lse")


def test_ragged_decode_small(gpu):
    """The ragged shape at 24 sequences: every output against the oracle."""
    step = W.ragged_decode(batch=24, seed=1913)
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu)
    ro, rl = O.decode(step, O.pool(step))
    check(out, ro, "out")
    check(lse, rl, "lse")


@pytest.mark.slow
def test_ragged_decode_full_size_sampled(gpu):
    """B=256, n log-uniform in [64, 8192], ceil(n/512) splits: 48 sampled
    (sequence, head) outputs against the oracle, one by one."""
    step = W.ragged_decode()
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu)
    rng = np.random.default_rng(0)
    longest = int(np.argmax(step.context_lens))
    rows = [(int(b), int(h)) for b, h in zip(rng.integers(0, 256, 46), rng.integers(0, 16, 46))]
    rows += [(longest, 0), (int(np.argmin(step.context_lens)), 15)]
    ro, rl = O.decode(step, O.pool(step), rows=rows)
    mask = np.zeros(out.shape[:2], bool)
    for b, h in rows:
        mask[b, h] = True
    st = O.compare(out[mask], ro[mask])
    assert st["ok"], st
    st = O.compare(lse[mask], rl[mask])
    assert st["ok"], st
    assert np.isfinite(out).all()


@pytest.mark.slow
def test_long_decode_full_size_sampled(gpu):
    """B=8 x 32768 tokens with 1% x8 key outliers, 64 splits: 24 sampled
    outputs against the oracle."""
    step = W.long_decode()
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu)
    rows = [(b, h) for b in range(8) for h in (0, 7, 15)]
    ro, rl = O.decode(step, O.pool(step), rows=rows)
    mask = np.zeros(out.shape[:2], bool)
    for b, h in rows:
        mask[b, h] = True
    st = O.compare(out[mask], ro[mask])
    assert st["ok"], st
    st = O.compare(lse[mask], rl[mask])
    assert st["ok"], st
    assert np.isfinite(out).all()


@pytest.mark.parametrize("D,G_,kv,qd", [(64, 1, "bf16", "bf16"), (64, 4, "bf16", "f32"), (128, 8, "f32", "f32"),
                                        (128, 4, "i8", "bf16"), (64, 2, "i8", "f32"), (128, 1, "bf16", "bf16"),
                                        (128, 2, "fp8", "bf16"), (64, 4, "fp8", "f32"), (128, 8, "fp8", "bf16")])
def test_decode_shapes_and_dtypes(gpu, D, G_, kv, qd):
    Hkv = 2
    scaled = kv in ("i8", "fp8")
    step = W.make_step(f"shape{D}_{G_}_{kv}", [1, 15, 16, 17, 100, 257], [1] * 6, num_q_heads=Hkv * G_,
                       num_kv_heads=Hkv, head_dim=D, q_dtype=qd, kv_dtype=kv,
                       src_dtype=(qd if scaled else kv),
                       num_splits=[1, 1, 2, 2, 3, 5], seed=50 + D + G_)
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu)
    ro, rl = O.decode(step, O.pool(step))
    check(out, ro, "out")
    check(lse, rl, "lse")


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_quantized_decode_rows_of_mixed_step(gpu, kv):
    step = W.mixed_int8(num_prefill=1, num_decode=24, seed=1915, kv_dtype=kv)
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu)
    ro, rl = O.decode(step, O.pool(step))
    check(out, ro, "out")
    check(lse, rl, "lse")


def test_every_split_count_agrees(gpu):
    """Any ns in [1, ceil(n/16)] (and beyond: empty splits) gives the same result."""
    step = W.make_step("sweep", [70, 33, 16, 1], [1, 1, 1, 1], num_q_heads=16, num_kv_heads=8, head_dim=128,
                       seed=60)
    cache = G.build_cache(step, gpu)
    ro, rl = O.decode(step, O.pool(step))
    for ns in range(1, 8):
        out, lse = G.run_decode(step, cache, gpu, num_splits=ns, max_num_splits=8)
        check(out, ro, f"ns={ns}")
        check(lse, rl, f"lse ns={ns}")


@pytest.mark.parametrize("D,G_,qd", [(128, 2, "bf16"), (64, 4, "f32"), (128, 8, "bf16"), (64, 1, "bf16")])
def test_deep_ring_many_splits(gpu, D, G_, qd):
    """bf16 caches cut into 8 or more splits per sequence stream with two
    blocks in flight per wavefront (one otherwise). Against the oracle, with
    splits from whole blocks down to empty ones; and the split partials bit
    for bit against the same splits launched with a split bound of 7 (one
    block in flight): the ring depth changes when loads are issued, not the
    arithmetic. (The combined outputs may differ in rounding: from 8 splits
    on, the combine sums them over four wavefronts.)"""
    Hkv = 2
    ctx = [1, 16, 17, 129, 700, 2049, 3000]
    ns = [8, 8, 9, 12, 16, 20, 11]
    step = W.make_step(f"deep{D}_{G_}", ctx, [1] * len(ctx), num_q_heads=Hkv * G_, num_kv_heads=Hkv, head_dim=D,
                       q_dtype=qd, kv_dtype="bf16", src_dtype="bf16", num_splits=ns, seed=70 + D + G_)
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu, max_num_splits=20)
    ro, rl = O.decode(step, O.pool(step))
    check(out, ro, "out")
    check(lse, rl, "lse")
    few = [min(7, n) for n in ns]
    o8, _ = G.run_decode(step, cache, gpu, num_splits=few, max_num_splits=8)
    check(o8, ro, "out, 8-split bound")
    q, tables, ctxs, _ = step.decode_batch()
    parts = {}
    for bound in (7, 8):
        ws = G.torch.zeros(G.pkv.decode_workspace_bytes(len(ctx), step.num_q_heads, D, bound), dtype=G.torch.uint8,
                           device=gpu)
        op, lp = G.pkv.paged_attention_decode(G.tensor(q, step.q_dtype, gpu), cache, G.ints(tables, gpu),
                                              G.ints(ctxs, gpu), G.ints(np.asarray(few, np.int32), gpu), bound,
                                              float(step.scale), workspace=ws, partials_only=True)
        G.torch.cuda.synchronize()
        parts[bound] = (op.cpu().numpy(), lp.cpu().numpy())
    for b, k in enumerate(few):
        assert np.array_equal(parts[8][0][b, :k].view(np.uint32), parts[7][0][b, :k].view(np.uint32)), b
        assert np.array_equal(parts[8][1][b, :k].view(np.uint32), parts[7][1][b, :k].view(np.uint32)), b


# ---------------------------------------------------------------------------
# indexing: bit-exact probes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv", ["bf16", "f32", "i8", "fp8"])
def test_one_hot_probe_returns_the_value_row_exactly(gpu, kv):
    """All keys zero except key j = alpha q, with the q heads of a group equal:
    every other weight underflows to exactly 0, so out == V_j bit for bit
    (int8 and fp8: value(code) * scale rounded once to float32)."""
    import torch
    n, Hq, Hkv, D = 45, 4, 2, 64
    qd = "f32" if kv == "f32" else "bf16"
    base = W.make_step("onehot", [n], [1], num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, q_dtype=qd,
                       kv_dtype=kv, src_dtype=("bf16" if kv in ("i8", "fp8") else kv), seed=70, num_blocks=6)
    qv = np.zeros((1, Hq, D), np.float32)
    qv[0, :, :8] = 1.0                       # all heads equal; |q|^2 = 8
    q = qv if qd == "f32" else W.f32_to_bf16_bits(qv)
    for j in (0, 16, 44):
        kf = np.zeros((n, Hkv, D), np.float32)
        kf[j, :, :8] = 64.0                  # s_j = 64 * 8 * scale = 64 > others (0) by 64 -> exp(-64 * ...)=0
        vf = np.random.default_rng(j).standard_normal((n, Hkv, D)).astype(np.float32)
        K = kf if base.src_dtype == "f32" else W.f32_to_bf16_bits(kf)
        V = vf if base.src_dtype == "f32" else W.f32_to_bf16_bits(vf)
        slots = np.concatenate([base.prefix_slots, base.new_slots])
        cache = G.pkv.KVCache.allocate(base.num_blocks, Hkv, D, G.CODE[kv], gpu)
        G.announce(f"one-hot kv={kv} j={j}")
        G.pkv.reshape_and_cache(G.tensor(K, base.src_dtype, gpu), G.tensor(V, base.src_dtype, gpu),
                                G.ints(slots, gpu, torch.int64), cache)
        _, tables, ctx, _ = base.decode_batch()
        out = G.pkv.paged_attention_decode(G.tensor(q, qd, gpu), cache, G.ints(tables, gpu), G.ints(ctx, gpu),
                                           None, 1, 4.0)
        out = out.cpu().numpy()
        # expected: the stored value row j, decoded exactly, in float32
        p = O.oracle.OraclePool(base.num_blocks, Hkv, 16, D, kv)
        O.oracle.reshape_and_cache(p, K, V, base.src_dtype, slots)
        _, Vj = O.oracle.gather_kv(p, tables[0], n)
        for h in range(Hq):
            want = Vj[j, h // 2].astype(np.float32)
            assert np.array_equal(out[0, h], want), (kv, j, h)


def test_output_is_bit_identical_under_block_placement(gpu):
    """Claim s06 on the GPU: moving the blocks elsewhere in the pool (same
    logical contents) leaves the output bits unchanged."""
    import torch
    step = W.qwen3_decode(batch=8, max_tokens_per_split=128, seed=71)
    cache = G.build_cache(step, gpu)
    out1, lse1 = G.run_decode(step, cache, gpu)
    perm = np.random.default_rng(5).permutation(step.num_blocks)
    cache2 = G.pkv.KVCache.allocate(step.num_blocks, 8, 128, G.pkv.BF16, gpu)
    pt = torch.from_numpy(perm).to(gpu)
    cache2.k[pt] = cache.k
    cache2.v[pt] = cache.v
    step.block_tables = np.where(step.block_tables >= 0, perm[np.maximum(step.block_tables, 0)], -1).astype(np.int32)
    out2, lse2 = G.run_decode(step, cache2, gpu)
    assert out1.tobytes() == out2.tobytes() and lse1.tobytes() == lse2.tobytes()


@pytest.mark.parametrize("S,ns,D", [
    (6, [1, 6, 3, 2, 6], 128),             # one wavefront per (sequence, head)
    (40, [1, 40, 3, 9, 33], 128),          # four wavefronts per pair (some with one split or none)
    (150, [1, 150, 70, 65, 129], 128),     # four wavefronts, several chunks of 16 splits each
    (150, [2, 149, 70, 66, 150], 64),
])
def test_lse_combine_alone(gpu, S, ns, D):
    import torch
    rng = np.random.default_rng(3 + S + D)
    B, Hq = 5, 4
    o = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    l = rng.standard_normal((B, S, Hq)).astype(np.float32) * 3
    ns = np.array(ns, np.int32)
    l[1, 2] = -np.inf
    l[3, :ns[3], 0] = -np.inf      # all live splits empty for (3, head 0)
    l[4, ns[4] - 1, 1] = 40.0      # one split far above the others of (4, head 1)
    l[2, :64, 0] = -np.inf         # with several chunks: the first chunk of every wavefront empty
    G.announce(f"lse_combine S={S} D={D}")
    out, lse = G.pkv.lse_combine(torch.from_numpy(o).to(gpu), torch.from_numpy(l).to(gpu), G.ints(ns, gpu))
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            ro, rl = O.oracle.lse_combine(o[b, :ns[b], h].astype(np.float64), l[b, :ns[b], h].astype(np.float64))
            assert O.compare(out[b, h], ro, atol=1e-5, rtol=1e-5)["ok"], (b, h)
            assert (rl == -np.inf and lse[b, h] == -np.inf) or abs(lse[b, h] - rl) < 1e-5


@pytest.mark.parametrize("S", [6, 40, 100])
def test_lse_combine_nan_and_bad_split_counts(gpu, S):
    """A NaN lse among a pair's live splits makes that pair NaN; a split count
    outside [1, S] makes the whole sequence NaN; the rest are untouched."""
    import torch
    rng = np.random.default_rng(11 + S)
    B, Hq, D = 4, 4, 128
    o = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    l = rng.standard_normal((B, S, Hq)).astype(np.float32)
    ns = np.array([S, 0, S + 1, 2], np.int32)
    l[0, S - 1, 2] = np.nan
    G.announce(f"lse_combine NaN S={S}")
    out, lse = G.pkv.lse_combine(torch.from_numpy(o).to(gpu), torch.from_numpy(l).to(gpu), G.ints(ns, gpu))
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isnan(out[0, 2]).all() and np.isnan(lse[0, 2])
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all() and np.isnan(lse[1]).all() and np.isnan(lse[2]).all()
    for b, h in [(0, 0), (0, 1), (0, 3), (3, 0), (3, 3)]:
        ro, rl = O.oracle.lse_combine(o[b, :ns[b], h].astype(np.float64), l[b, :ns[b], h].astype(np.float64))
        assert O.compare(out[b, h], ro, atol=1e-5, rtol=1e-5)["ok"], (b, h)
        assert abs(lse[b, h] - rl) < 1e-5


def test_bad_device_metadata_gives_nan_not_a_fault(gpu):
    """Block ids outside the pool, a context longer than the table, and a split
    count outside [1, max] are caught by the kernels' own bounds checks:
    those sequences come out NaN, the others are untouched."""
    step = W.make_step("bad", [40, 40, 40, 40], [1] * 4, num_q_heads=4, num_kv_heads=2, head_dim=64,
                       seed=72, num_splits=2)
    cache = G.build_cache(step, gpu)
    ro, _ = O.decode(step, O.pool(step))
    step.block_tables[0, 1] = step.num_blocks + 5     # id past the pool
    step.block_tables[1, 0] = -3                      # negative id
    step.context_lens[2] = step.block_tables.shape[1] * 16 + 1   # longer than its table
    ns = np.array([2, 2, 2, 9], np.int32)             # 9 > max_num_splits = 4
    out, _ = G.run_decode(step, cache, gpu, num_splits=ns, max_num_splits=4)
    assert np.isnan(out[:4]).all()
    step2 = W.make_step("bad", [40, 40, 40, 40], [1] * 4, num_q_heads=4, num_kv_heads=2, head_dim=64,
                        seed=72, num_splits=2)
    out2, _ = G.run_decode(step2, cache, gpu, num_splits=2, max_num_splits=4)
    check(out2, ro, "clean rerun")
