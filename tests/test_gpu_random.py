"""GPU parity over seeded random configurations: every head_dim, GQA group
size, cache and q dtype the library builds, random context lengths (block
multiples and ragged tails), random split counts (past the block count too:
empty splits), split and balanced decode modes, and random chunk / prefix
lengths for chunked prefill, chunks of a few rows per sequence (the
decode-shaped paths of the chunked call), and longer contexts cut into many
splits. The cases are drawn once, from a
fixed seed, so every run tests the same ones."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_side as G
from tests import oracle_side as O

pytestmark = pytest.mark.gpu


def _decode_cases(n_cases: int = 24, seed: int = 20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        D = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 4]))
        kv = str(rng.choice(["f32", "bf16", "i8", "fp8"]))
        qd = str(rng.choice(["f32", "bf16"]))
        B = int(rng.integers(1, 13))
        ctx = rng.integers(1, 701, size=B)
        mult = rng.random(B) < 0.25                      # some contexts end on a block boundary
        ctx[mult] = 16 * rng.integers(1, 44, size=int(mult.sum()))
        blocks = -(-ctx // 16)
        ns = np.minimum(rng.integers(1, 9, size=B), blocks + 1).astype(np.int32)
        mode = str(rng.choice(["splits", "balanced"]))
        cases.append(dict(id=f"d{i}_{mode}_D{D}_g{g}_h{hkv}_{kv}_q{qd}_B{B}", D=D, g=g, hkv=hkv, kv=kv, qd=qd,
                          ctx=[int(c) for c in ctx], ns=[int(x) for x in ns], mode=mode, seed=3000 + i))
    return cases


def _chunked_cases(n_cases: int = 16, seed: int = 20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        g = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2]))
        kv = str(rng.choice(["bf16", "i8", "fp8"]))
        S = int(rng.integers(1, 5))
        L = rng.integers(2, 201, size=S)                 # (one-row sequences are decode rows)
        prefix = rng.integers(0, 601, size=S)
        D = 64 if i % 4 == 3 else 128                    # every fourth case over a head_dim 64 cache
        cases.append(dict(id=f"c{i}_D{D}_g{g}_h{hkv}_{kv}_S{S}", D=D, g=g, hkv=hkv, kv=kv,
                          ctx=[int(a + b) for a, b in zip(prefix, L)], ql=[int(x) for x in L], seed=4000 + i))
    return cases


def _few_row_cases(n_cases: int = 12, n_short: int = 4, seed: int = 20261204):
    """Chunks of 1 to 16 / G rows per sequence, one-row chunks among them, over
    random prefixes: up to 2 rows per kv head (4 with head_dim 64) take the
    decode kernels, more up to 16 the 16x16 MFMA kernel (the chunk kernel with
    head_dim 64). The last ``n_short`` cases keep head_dim 128 chunks to at
    most 2 rows per kv head, so that the decode kernels' share of the random
    cases does not hang on the draws."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases + n_short):
        short = i >= n_cases
        g = int(rng.choice([1, 2] if short else [1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 4]))
        kv = str(rng.choice(["bf16", "i8", "fp8"]))
        S = int(rng.integers(1, 25))
        lmax = 2 // g if short else int(rng.integers(1, 16 // g + 1))
        L = rng.integers(1, lmax + 1, size=S)
        prefix = rng.integers(0, 900, size=S)
        D = 64 if i % 3 == 2 and not short else 128     # every third case over a head_dim 64 cache
        cases.append(dict(id=f"r{i}_D{D}_g{g}_h{hkv}_{kv}_S{S}_L{int(L.max())}", D=D, g=g, hkv=hkv, kv=kv,
                          ctx=[int(a + b) for a, b in zip(prefix, L)], ql=[int(x) for x in L], seed=5000 + i))
    return cases


def _long_split_cases(n_cases: int = 8, seed: int = 20261205):
    """Longer contexts cut into many splits: past 8 splits per sequence the
    bf16 decode keeps two blocks in flight per wavefront and the combine runs
    four wavefronts per pair, past 64 it takes a wavefront's splits in several
    chunks."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        D = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2]))
        kv = "bf16" if i % 2 == 0 else str(rng.choice(["f32", "i8", "fp8"]))
        qd = str(rng.choice(["f32", "bf16"]))
        B = int(rng.integers(1, 5))
        ctx = rng.integers(700, 6001, size=B)
        blocks = -(-ctx // 16)
        ns = np.minimum(rng.integers(8, 161, size=B), blocks + 1).astype(np.int32)
        cases.append(dict(id=f"l{i}_D{D}_g{g}_h{hkv}_{kv}_q{qd}_B{B}_ns{int(ns.max())}", D=D, g=g, hkv=hkv, kv=kv,
                          qd=qd, ctx=[int(c) for c in ctx], ns=[int(x) for x in ns], mode="splits",
                          seed=6000 + i))
    return cases


DECODE = _decode_cases()
CHUNKED = _chunked_cases()
FEW_ROWS = _few_row_cases()
LONG_SPLITS = _long_split_cases()


def _check(out, ref, what, case):
    st = O.compare(out, ref)
    assert st["ok"], f"{case['id']} {what}: {st}"


@pytest.mark.parametrize("case", DECODE, ids=[c["id"] for c in DECODE])
def test_random_decode(gpu, case):
    import torch
    scaled = case["kv"] in ("i8", "fp8")
    step = W.make_step(case["id"], case["ctx"], [1] * len(case["ctx"]), num_q_heads=case["g"] * case["hkv"],
                       num_kv_heads=case["hkv"], head_dim=case["D"], q_dtype=case["qd"], kv_dtype=case["kv"],
                       src_dtype=(case["qd"] if scaled else case["kv"]), num_splits=case["ns"], seed=case["seed"])
    cache = G.build_cache(step, gpu)
    if case["mode"] == "splits":
        out, lse = G.run_decode(step, cache, gpu)
    else:
        q, tables, ctx, _ = step.decode_batch()
        G.announce(f"balanced decode {case['id']}")
        out, lse = G.pkv.paged_attention_decode(G.tensor(q, step.q_dtype, gpu), cache, G.ints(tables, gpu),
                                                G.ints(ctx, gpu), None, 0, float(step.scale), return_lse=True)
        torch.cuda.synchronize()
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
    ro, rl = O.decode(step, O.pool(step))
    _check(out, ro, "out", case)
    _check(lse, rl, "lse", case)


@pytest.mark.parametrize("case", LONG_SPLITS, ids=[c["id"] for c in LONG_SPLITS])
def test_random_long_split_decode(gpu, case):
    scaled = case["kv"] in ("i8", "fp8")
    step = W.make_step(case["id"], case["ctx"], [1] * len(case["ctx"]), num_q_heads=case["g"] * case["hkv"],
                       num_kv_heads=case["hkv"], head_dim=case["D"], q_dtype=case["qd"], kv_dtype=case["kv"],
                       src_dtype=(case["qd"] if scaled else case["kv"]), num_splits=case["ns"], seed=case["seed"])
    cache = G.build_cache(step, gpu)
    out, lse = G.run_decode(step, cache, gpu)
    ro, rl = O.decode(step, O.pool(step))
    _check(out, ro, "out", case)
    _check(lse, rl, "lse", case)


@pytest.mark.parametrize("case", CHUNKED, ids=[c["id"] for c in CHUNKED])
def test_random_chunked(gpu, case):
    step = W.make_step(case["id"], case["ctx"], case["ql"], num_q_heads=case["g"] * case["hkv"],
                       num_kv_heads=case["hkv"], head_dim=case["D"], kv_dtype=case["kv"], src_dtype="bf16",
                       seed=case["seed"])
    cache = G.build_cache(step, gpu)
    out, lse = G.run_chunked(step, cache, gpu)
    ro, rl = O.chunked(step, O.pool(step))
    _check(out, ro, "out", case)
    _check(lse, rl, "lse", case)


@pytest.mark.parametrize("case", FEW_ROWS, ids=[c["id"] for c in FEW_ROWS])
def test_random_few_row_chunks(gpu, case):
    import torch
    step = W.make_step(case["id"], case["ctx"], case["ql"], num_q_heads=case["g"] * case["hkv"],
                       num_kv_heads=case["hkv"], head_dim=case["D"], kv_dtype=case["kv"], src_dtype="bf16",
                       seed=case["seed"])
    cache = G.build_cache(step, gpu)
    # every sequence's rows as one chunk (one-row chunks included)
    q, cu, tables, ctx = step.q, step.cu_q_lens, step.block_tables, step.context_lens
    G.announce(f"few-row chunks {case['id']}")
    out, lse = G.pkv.paged_attention_chunked(G.tensor(q, "bf16", gpu), G.ints(cu, gpu), int(max(case["ql"])), cache,
                                             G.ints(tables, gpu), G.ints(ctx, gpu), float(step.scale),
                                             return_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.oracle.paged_chunked(O.oracle.decode_rows(q, "bf16"), cu, O.pool(step), tables, ctx, step.scale)
    _check(out.cpu().numpy(), ro, "out", case)
    _check(lse.cpu().numpy(), rl, "lse", case)
