"""Seeded generators for the five workload shapes and for ad-hoc test steps.

Recipe (the same for every shape):

* One parent stream ``numpy.random.default_rng(SeedSequence(seed))`` draws the
  per-sequence context lengths (where random) and the block permutation.
* Sequence ``i`` draws from its own child stream
  ``SeedSequence(seed).spawn(S)[i]``, in this order: K ``[n_i][Hkv][D]``,
  V ``[n_i][Hkv][D]`` and q ``[q_len_i][Hq][D]``, all float32 N(0, 1); then, if
  key outliers are asked for, a Bernoulli mask ``[n_i][Hkv]`` whose key vectors
  are multiplied by the outlier factor (a power of two, so exact). Child
  streams make every sequence reproducible on its own and let the draws run on
  several threads.
* bfloat16 values are the float32 draws rounded to nearest-even.
* The pool is a seeded permutation of ``num_blocks`` physical blocks; sequence
  ``i`` takes the next ``ceil(n_i / bs)`` entries as its block table (``-1``
  past them). Tokens ``[0, n_i - q_len_i)`` form the cached prefix; the last
  ``q_len_i`` tokens are the step's new rows. Slot of token ``t`` of sequence
  ``i``: ``table[i][t // bs] * bs + t % bs``, as an allocator hands it out.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

F32, BF16, I8, FP8 = "f32", "bf16", "i8", "fp8"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the
    16-bit patterns. Inputs here are finite draws, so no NaN handling."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(x32, np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(f"inputs are generated as f32 or bf16, not {dtype}")


@dataclass
class Step:
    """One step's inputs: a pool geometry, the sequences, and their rows.

    ``q_lens[i] == 1`` marks a decode row; ``q_lens[i] > 1`` a prefill chunk.
    Arrays are in storage form (float32, or uint16 bfloat16 bit patterns).
    """

    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    q_dtype: str
    kv_dtype: str            # cache storage dtype: f32, bf16, i8 or fp8
    src_dtype: str           # dtype of the K/V rows handed to reshape_and_cache
    scale: np.float32
    context_lens: np.ndarray  # int32 [S]
    q_lens: np.ndarray        # int32 [S]
    block_tables: np.ndarray  # int32 [S][max_blocks], -1 padded
    q: np.ndarray             # [sum q_lens][Hq][D]
    prefix_k: np.ndarray      # [P][Hkv][D]
    prefix_v: np.ndarray
    prefix_slots: np.ndarray  # int64 [P]
    new_k: np.ndarray         # [N][Hkv][D]
    new_v: np.ndarray
    new_slots: np.ndarray     # int64 [N]
    num_splits: np.ndarray    # int32 [S] (1 for chunk rows)
    meta: dict = field(default_factory=dict)

    # ---- convenience views -------------------------------------------------
    @property
    def cu_q_lens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def decode_idx(self) -> np.ndarray:
        return np.nonzero(self.q_lens == 1)[0]

    @property
    def chunk_idx(self) -> np.ndarray:
        return np.nonzero(self.q_lens > 1)[0]

    def decode_batch(self):
        """``(q [B][Hq][D], block_tables, context_lens, num_splits)`` of the decode rows."""
        idx = self.decode_idx
        cu = self.cu_q_lens
        q = self.q[cu[idx]]
        return (np.ascontiguousarray(q), np.ascontiguousarray(self.block_tables[idx]),
                np.ascontiguousarray(self.context_lens[idx]),
                np.ascontiguousarray(self.num_splits[idx]))

    def chunk_batch(self):
        """``(q [sum L][Hq][D], cu_q_lens, block_tables, context_lens)`` of the chunk rows."""
        idx = self.chunk_idx
        cu = self.cu_q_lens
        q = np.concatenate([self.q[cu[i]:cu[i + 1]] for i in idx]) if len(idx) else self.q[:0]
        lens = self.q_lens[idx]
        cuc = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        return (np.ascontiguousarray(q), cuc, np.ascontiguousarray(self.block_tables[idx]),
                np.ascontiguousarray(self.context_lens[idx]))

    def kv_contiguous(self, i: int):
        """Storage rows of sequence ``i`` in token order: ``(K, V)`` ``[n_i][Hkv][D]``."""
        return self.meta["seq_k"][i], self.meta["seq_v"][i]


def _draw_seq(child, n, q_len, Hq, Hkv, D, outlier_frac, outlier_mult):
    rng = np.random.default_rng(child)
    k = rng.standard_normal((n, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((n, Hkv, D), dtype=np.float32)
    q = rng.standard_normal((q_len, Hq, D), dtype=np.float32)
    if outlier_frac > 0.0:
        mask = rng.random((n, Hkv)) < outlier_frac
        k[mask] *= np.float32(outlier_mult)
    return k, v, q


def make_step(name: str, context_lens, q_lens, *, num_q_heads: int, num_kv_heads: int,
              head_dim: int, block_size: int = 16, num_blocks: int | None = None,
              q_dtype: str = BF16, kv_dtype: str = BF16, src_dtype: str | None = None,
              num_splits=None, seed: int = 0, outlier_frac: float = 0.0,
              outlier_mult: float = 8.0, scale: float | None = None,
              max_blocks_per_seq: int | None = None, threads: int | None = None,
              values_seed: int | None = None) -> Step:
    """Build a step for arbitrary sequences (see the module docstring).

    ``values_seed`` (default ``seed``) seeds the per-sequence value streams
    alone: steps that share ``seed`` and differ in ``values_seed`` have the same
    context lengths, block tables and slots but their own q/K/V -- the layers
    of one model step, which share the batch's block tables and each own a
    KV pool."""
    ctx = np.asarray(context_lens, np.int64)
    ql = np.asarray(q_lens, np.int64)
    S = len(ctx)
    assert ql.shape == (S,) and (ql >= 1).all() and (ql <= ctx).all()
    Hq, Hkv, D, bs = num_q_heads, num_kv_heads, head_dim, block_size
    src_dtype = src_dtype or (kv_dtype if kv_dtype not in (I8, FP8) else BF16)
    nblk = -(-ctx // bs)
    need = int(nblk.sum())
    num_blocks = need if num_blocks is None else int(num_blocks)
    assert num_blocks >= need, "pool too small for the sequences"
    ss = np.random.SeedSequence(seed)
    parent = np.random.default_rng(ss)
    perm = parent.permutation(num_blocks).astype(np.int32)
    maxb = int(max_blocks_per_seq or max(1, int(nblk.max()) if S else 1))
    tables = np.full((S, maxb), -1, np.int32)
    pos = 0
    for i in range(S):
        tables[i, :nblk[i]] = perm[pos:pos + nblk[i]]
        pos += nblk[i]

    kids = (ss if values_seed is None else np.random.SeedSequence(values_seed)).spawn(S)
    nthreads = threads or min(16, os.cpu_count() or 1)
    args = [(kids[i], int(ctx[i]), int(ql[i]), Hq, Hkv, D, outlier_frac, outlier_mult) for i in range(S)]
    if S > 4 and nthreads > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            draws = list(ex.map(lambda a: _draw_seq(*a), args))
    else:
        draws = [_draw_seq(*a) for a in args]

    seq_k = [_store(d[0], src_dtype) for d in draws]
    seq_v = [_store(d[1], src_dtype) for d in draws]
    q = np.concatenate([_store(d[2], q_dtype) for d in draws]) if S else np.zeros((0, Hq, D))

    def slots_of(i, t0, t1):
        t = np.arange(t0, t1, dtype=np.int64)
        return tables[i, t // bs].astype(np.int64) * bs + t % bs

    pre_k, pre_v, pre_s, new_k, new_v, new_s = [], [], [], [], [], []
    for i in range(S):
        n, L = int(ctx[i]), int(ql[i])
        pre_k.append(seq_k[i][:n - L]); pre_v.append(seq_v[i][:n - L]); pre_s.append(slots_of(i, 0, n - L))
        new_k.append(seq_k[i][n - L:]); new_v.append(seq_v[i][n - L:]); new_s.append(slots_of(i, n - L, n))

    def cat(xs, shape_tail, dt):
        return np.concatenate(xs) if xs else np.zeros((0,) + shape_tail, dt)

    sd = np.float32 if src_dtype == F32 else np.uint16
    if num_splits is None:
        ns = np.ones(S, np.int32)
    elif np.isscalar(num_splits):
        ns = np.full(S, int(num_splits), np.int32)
    else:
        ns = np.asarray(num_splits, np.int32)
    ns = np.where(ql == 1, ns, 1).astype(np.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Step(
        name=name, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
        num_blocks=num_blocks, q_dtype=q_dtype, kv_dtype=kv_dtype, src_dtype=src_dtype,
        scale=np.float32(scale), context_lens=ctx.astype(np.int32), q_lens=ql.astype(np.int32),
        block_tables=tables, q=q,
        prefix_k=cat(pre_k, (Hkv, D), sd), prefix_v=cat(pre_v, (Hkv, D), sd),
        prefix_slots=cat(pre_s, (), np.int64),
        new_k=cat(new_k, (Hkv, D), sd), new_v=cat(new_v, (Hkv, D), sd),
        new_slots=cat(new_s, (), np.int64),
        num_splits=ns, meta={"seq_k": seq_k, "seq_v": seq_v},
    )


# --------------------------------------------------------------------------
# the five workload shapes
# --------------------------------------------------------------------------

def splits_for(context_lens, max_tokens_per_split: int) -> np.ndarray:
    """``ceil(n / max_tokens)`` splits per sequence (a scheduling choice)."""
    c = np.asarray(context_lens, np.int64)
    return np.maximum(1, -(-c // max_tokens_per_split)).astype(np.int32)


def tiny_decode(num_splits: int = 1, seed: int = 1901) -> Step:
    """Tiny decode: B=3, n=[5,17,40], 4 q / 2 kv heads, D=64, bs=16, an 8-block
    pool (tables a seeded permutation of it), fp32 q/K/V from N(0,1),
    scale 1/sqrt(64)."""
    return make_step("tiny_decode", [5, 17, 40], [1, 1, 1], num_q_heads=4, num_kv_heads=2,
                     head_dim=64, block_size=16, num_blocks=8, q_dtype=F32, kv_dtype=F32,
                     num_splits=num_splits, seed=seed)


def qwen3_decode(batch: int = 32, num_splits=None, max_tokens_per_split: int | None = None,
                 seed: int = 1902, num_blocks: int = 4096, values_seed: int | None = None) -> Step:
    """Qwen3-0.6B-shaped single-layer decode step: 16 q / 8 kv heads, D=128,
    bf16 N(0,1), n uniform in [128, 384] (128-token prompt + up to 256 new),
    bs=16, tables from a permutation of a 4096-block pool; the step writes one
    new token per sequence."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    ctx = rng.integers(128, 384, size=batch, endpoint=True)
    if num_splits is None and max_tokens_per_split is not None:
        num_splits = splits_for(ctx, max_tokens_per_split)
    return make_step("qwen3_decode", ctx, np.ones(batch, np.int64), num_q_heads=16, num_kv_heads=8,
                     head_dim=128, num_blocks=num_blocks, num_splits=num_splits, seed=seed,
                     values_seed=values_seed)


def ragged_decode(batch: int = 256, max_tokens_per_split: int = 512, seed: int = 1903,
                  lo: int = 64, hi: int = 8192) -> Step:
    """Saturated ragged decode: n log-uniform in [64, 8192] (``round(exp(U))``
    clamped), 16q/8kv/128, bf16, a pool of exactly the blocks needed, shuffled;
    ``ceil(n / 512)`` splits per sequence."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    ctx = np.clip(np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch))), lo, hi).astype(np.int64)
    return make_step("ragged_decode", ctx, np.ones(batch, np.int64), num_q_heads=16, num_kv_heads=8,
                     head_dim=128, num_splits=splits_for(ctx, max_tokens_per_split), seed=seed)


def long_decode(batch: int = 8, context_len: int = 32768, num_splits: int = 64,
                seed: int = 1904) -> Step:
    """Long-context decode: every sequence 32768 tokens, 16q/8kv/128, bf16
    N(0,1) with 1% of key vectors (per token and kv head) scaled x8, bs=16,
    64 splits per sequence."""
    ctx = np.full(batch, context_len, np.int64)
    return make_step("long_decode", ctx, np.ones(batch, np.int64), num_q_heads=16, num_kv_heads=8,
                     head_dim=128, num_splits=num_splits, seed=seed, outlier_frac=0.01, outlier_mult=8.0)


def mixed_int8(num_prefill: int = 4, chunk: int = 512, prefix: int = 1536, num_decode: int = 124,
               lo: int = 256, hi: int = 4096, max_tokens_per_split: int = 512,
               seed: int = 1905, kv_dtype: str = I8, values_seed: int | None = None) -> Step:
    """Mixed chunked-prefill + decode step over an int8 (or, with ``kv_dtype=
    "fp8"``, an fp8; with ``"bf16"``, a bf16 one of the same shape) KV cache: ``num_prefill``
    sequences with a ``chunk``-row causal chunk after a ``prefix``-token cached
    prefix, plus ``num_decode`` decode rows with n uniform in [256, 4096].
    16q/8kv/128, q and the new K/V rows bf16 (quantized by the cache write),
    bs=16, pool = blocks needed, shuffled; decode splits ``ceil(n / 512)``.
    ``values_seed`` draws other values over the same shapes and tables."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    dec = rng.integers(lo, hi, size=num_decode, endpoint=True)
    ctx = np.concatenate([np.full(num_prefill, prefix + chunk), dec]).astype(np.int64)
    ql = np.concatenate([np.full(num_prefill, chunk), np.ones(num_decode)]).astype(np.int64)
    assert kv_dtype in (I8, FP8, BF16)
    name = {I8: "mixed_int8", FP8: "mixed_fp8", BF16: "mixed_bf16"}[kv_dtype]
    return make_step(name, ctx, ql, num_q_heads=16, num_kv_heads=8,
                     head_dim=128, q_dtype=BF16, kv_dtype=kv_dtype, src_dtype=BF16,
                     num_splits=splits_for(ctx, max_tokens_per_split), seed=seed, values_seed=values_seed)
