#!/usr/bin/env python3
"""Decode-step benchmark of the paged-KV attention library on one MI355X.

A step is one pass of the decode hot path over one batch: reshape_and_cache of
the batch's new token (one row per sequence), the split-K partial pass, and the
log-sum-exp merge. The workload is a Qwen3-0.6B-shaped single layer: 32
sequences, 16 query / 8 KV heads, head_dim 128, bf16 q/K/V from N(0, 1),
context lengths uniform in [128, 384], 16-token blocks drawn from a 4096-block
pool. Inputs are resident in HBM before timing starts.

One step's KV (33.6 MB) would sit in MI355X's 256 MB Infinity Cache if the
same step were repeated, so the timed loop rotates through R replicas that
stand for R layers of one model step: they share the batch's block tables,
context lengths and slots (as an engine's layers do) and each owns its KV pool
and its q/K/V values. Between two uses of one replica the other R - 1 replicas
stream well over 256 MB of KV, so every step reads its KV from HBM.
Steps are launched from HIP graphs (each graph holds many steps) so that host
launch cost does not pace the GPU.

Output: one JSON line on stdout (everything else goes to stderr).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn decode KV GB/s (% HBM peak) + seq-steps/s; chunked-prefill MFMA util"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
KERNEL_FILES = ("paged_kv_attention_19_amd/csrc/decode_kernel.h", "paged_kv_attention_19_amd/csrc/decode_core.h",
                "paged_kv_attention_19_amd/csrc/decode_bf16.hip", "paged_kv_attention_19_amd/csrc/pkv_device.h",
                "paged_kv_attention_19_amd/csrc/quant_row.h", "paged_kv_attention_19_amd/csrc/api.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partial_qwen3_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int, scale_bytes: int = 0,
                       layers: int = 1) -> int:
    """Algorithmic KV bytes one token of one layer holds: K and V rows of every
    KV head, plus their scales for int8."""
    return layers * 2 * num_kv_heads * (head_dim * elem_bytes + scale_bytes)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_FILES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# The mixed step leaves the decode rows' split to the caller. Measured on
# MI355X (int8, decode launch alone): 110.5 us with 512-token splits, 104.1 with
# 1024, 103.9 with 1536, 108.1 with 2048 and 123.5 with one split per sequence:
# longer splits spread each workgroup's start-up over more blocks until too few
# workgroups are left to fill the GPU.
MIXED_SPLIT = 1024

# name -> (builder(seed, max_tokens_per_split), default replicas, default split size, config text)
WORKLOADS = {
    "qwen3_decode": (lambda W, seed, mts, batch, r: W.qwen3_decode(batch=batch, seed=seed, values_seed=seed + 1000 * r,
                                                                    max_tokens_per_split=mts or None),
                     16, 0, {"workload": "qwen3_0.6b_layer_decode_step", "context_lens": "uniform[128,384]",
                             "pool_blocks": 4096}),
    "ragged_decode": (lambda W, seed, mts, batch, r: W.ragged_decode(seed=seed + 1000 * r,
                                                                      max_tokens_per_split=mts or 512),
                      1, 512, {"workload": "ragged_decode_b256", "context_lens": "log-uniform[64,8192]"}),
    "long_decode": (lambda W, seed, mts, batch, r: W.long_decode(seed=seed + 1000 * r,
                                                                  num_splits=(32768 // mts) if mts else 64),
                    1, 512, {"workload": "long_decode_b8_32k", "context_lens": "32768"}),
    "mixed_int8_decode": (lambda W, seed, mts, batch, r: W.mixed_int8(seed=seed + 1000 * r,
                                                                       max_tokens_per_split=mts or MIXED_SPLIT),
                          1, MIXED_SPLIT, {"workload": "mixed_int8_step_decode_rows", "context_lens": "uniform[256,4096]"}),
    "mixed_fp8_decode": (lambda W, seed, mts, batch, r: W.mixed_int8(seed=seed + 1000 * r, kv_dtype="fp8",
                                                                      max_tokens_per_split=mts or MIXED_SPLIT),
                         1, MIXED_SPLIT, {"workload": "mixed_fp8_step_decode_rows", "context_lens": "uniform[256,4096]"}),
}
DEFAULT_SEEDS = {"qwen3_decode": 1902, "ragged_decode": 1903, "long_decode": 1904, "mixed_int8_decode": 1905,
                 "mixed_fp8_decode": 1905}
# Decode mode measured fastest on MI355X per shape: one workgroup per
# (split, kv head) for the Qwen3 step (one split per sequence), the uniform
# long contexts (64 splits of 512 tokens, as the workload states) and the
# mixed step's decode rows (1024-token splits); the log-uniform ragged batch
# gains from the balanced deal of tiles.
DEFAULT_MODES = {"qwen3_decode": "splits", "ragged_decode": "balanced", "long_decode": "splits",
                 "mixed_int8_decode": "splits", "mixed_fp8_decode": "splits"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8192)
    ap.add_argument("--warmup", type=int, default=512)
    ap.add_argument("--replicas", type=int, default=None,
                    help="independent copies rotated through (default: 16 for the Qwen3 step, else 1)")
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--max-tokens-per-split", type=int, default=None,
                    help="num_splits[b] = ceil(n_b / this); 0 = one split per sequence "
                         "(default: 0 for the Qwen3 step, 1024 for the mixed step's decode rows, 512 for the others)")
    ap.add_argument("--steps-per-graph", type=int, default=256)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunked", action="store_true", help="skip the chunked-prefill MFMA measurement")
    ap.add_argument("--chunked-kv", choices=("i8", "fp8"), default="i8",
                    help="KV cache dtype of the mixed step in the chunked-prefill measurement")
    ap.add_argument("--no-fuse", action="store_true",
                    help="write the new rows with a separate reshape_and_cache launch instead of inside the decode")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--workload", default="qwen3_decode", choices=sorted(WORKLOADS),
                    help="the step's shape (default: the Qwen3-0.6B decode step)")
    ap.add_argument("--decode-mode", choices=("balanced", "splits"), default=None,
                    help="balanced: the library deals the batch's tiles evenly over the GPU and merges cut "
                         "sequences in the same launch (max_num_splits = 0); splits: caller-chosen "
                         "num_splits (from --max-tokens-per-split) with a separate merge pass")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 8 times (to scale HBM counters)")
    return ap.parse_args()


def copy_calibration(nbytes: int) -> None:
    """A plain copy kernel of known size: FETCH_SIZE / WRITE_SIZE of its dispatches
    give the factor between the counters and bytes actually moved."""
    import torch
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "copies": 8}), flush=True)


def copy_reference(nbytes: int):
    """A plain device-to-device copy that moves the same number of HBM bytes as
    one decode launch (nbytes / 2 read, nbytes / 2 written), rotated over
    enough buffers that every copy comes from HBM: the rate a memory-bound
    kernel of this size can reach on this machine with no attention work."""
    import torch
    copies, steps = (16, 2048) if nbytes < (64 << 20) else (2, 64)
    half = max(16, (nbytes // 2) // 16 * 16)
    pairs = [(torch.randint(0, 255, (half,), dtype=torch.uint8, device="cuda:0"),
              torch.empty(half, dtype=torch.uint8, device="cuda:0")) for _ in range(copies)]
    sec = time_graphs(lambda pr: pr[1].copy_(pr[0]), pairs, steps, 256, 64)
    us = sec / steps * 1e6
    return {"bytes_moved": 2 * half, "us": round(us, 3), "GB/s": round(2 * half / (sec / steps) / 1e9, 1)}


class Replica:
    """One independent copy of the workload, resident on the GPU."""

    def __init__(self, step, dev, max_tokens_per_split, balanced=False, fuse=True):
        import numpy as np
        import torch

        import paged_kv_attention_19_amd as pkv
        self.step = step

        def dt(a, kind):
            if kind == "bf16":
                return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        code = {"f32": pkv.F32, "bf16": pkv.BF16, "i8": pkv.I8, "fp8": pkv.FP8}
        self.cache = pkv.KVCache.allocate(step.num_blocks, step.num_kv_heads, step.head_dim, code[step.kv_dtype], dev)
        pkv.reshape_and_cache(dt(step.prefix_k, step.src_dtype), dt(step.prefix_v, step.src_dtype),
                              dt(step.prefix_slots.astype(np.int64), "i64"), self.cache)
        q, tables, ctx, ns = step.decode_batch()
        self.q = dt(q, step.q_dtype)
        self.tables = dt(tables.astype(np.int32), "i32")
        self.ctx = dt(ctx.astype(np.int32), "i32")
        self.balanced = balanced
        self.max_ns = 0 if balanced else int(ns.max())
        self.ns = None if balanced else dt(ns.astype(np.int32), "i32")
        # the step's new rows: one per decode sequence (chunk rows belong to the chunked pass)
        dec_rows = np.concatenate([np.arange(step.cu_q_lens[i], step.cu_q_lens[i + 1]) for i in step.decode_idx])
        self.new_k = dt(step.new_k[dec_rows], step.src_dtype)
        self.new_v = dt(step.new_v[dec_rows], step.src_dtype)
        self.new_slots = dt(step.new_slots[dec_rows].astype(np.int64), "i64")
        B, Hq, D = q.shape
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        wsb = pkv.decode_workspace_bytes(B, Hq, D, self.max_ns)
        self.ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device=dev)   # balanced counters start at 0
        S = self.max_ns
        if S > 1:
            flat = self.ws.view(torch.float32)
            self.o_part = flat[: B * S * Hq * D].view(B, S, Hq, D)
            self.lse_part = flat[B * S * Hq * D: B * S * Hq * (D + 1)].view(B, S, Hq)
        self.tokens = int(ctx.sum())
        eb, sb = {"f32": (4, 0), "bf16": (2, 0), "i8": (1, 4), "fp8": (1, 4)}[step.kv_dtype]
        self.kv_bytes = self.tokens * kv_bytes_per_token(step.num_kv_heads, step.head_dim, eb, sb)
        self.batch = B
        # the decode launch writes the new rows too (split mode)
        self.fused = fuse and not balanced
        src_eb = {"f32": 4, "bf16": 2}[step.src_dtype]
        self.append_bytes = B * (kv_bytes_per_token(step.num_kv_heads, step.head_dim, src_eb)
                                 + kv_bytes_per_token(step.num_kv_heads, step.head_dim, eb, sb))

    def reshape(self):
        import paged_kv_attention_19_amd as pkv
        pkv.reshape_and_cache(self.new_k, self.new_v, self.new_slots, self.cache)

    def decode(self):
        import paged_kv_attention_19_amd as pkv
        pkv.paged_attention_decode(self.q, self.cache, self.tables, self.ctx, self.ns, self.max_ns,
                                   float(self.step.scale), out=self.out, out_lse=self.lse, workspace=self.ws)

    def decode_append(self):
        import paged_kv_attention_19_amd as pkv
        pkv.paged_attention_decode_append(self.new_k, self.new_v, self.new_slots, self.q, self.cache, self.tables,
                                          self.ctx, self.ns, self.max_ns, float(self.step.scale), out=self.out,
                                          out_lse=self.lse, workspace=self.ws)

    def partials(self):
        import paged_kv_attention_19_amd as pkv
        if self.fused and self.max_ns <= 1:
            self.decode_append()
        elif self.fused:
            pkv.paged_attention_decode_append(self.new_k, self.new_v, self.new_slots, self.q, self.cache,
                                              self.tables, self.ctx, self.ns, self.max_ns, float(self.step.scale),
                                              workspace=self.ws, partials_only=True)
        elif self.max_ns <= 1:
            self.decode()
        else:
            pkv.paged_attention_decode(self.q, self.cache, self.tables, self.ctx, self.ns, self.max_ns,
                                       float(self.step.scale), workspace=self.ws, partials_only=True)

    def combine(self):
        import paged_kv_attention_19_amd as pkv
        if self.max_ns <= 1:
            return
        pkv.lse_combine(self.o_part, self.lse_part, self.ns, out=self.out, out_lse=self.lse)

    def step_once(self):
        if self.fused:
            self.decode_append()
        else:
            self.reshape()
            self.decode()


def time_graphs(fn_per_step, reps, steps, steps_per_graph, warmup):
    """Capture graphs of ``steps_per_graph`` consecutive steps (rotating over the
    replicas) and replay them until exactly ``steps`` steps ran; returns seconds."""
    import torch
    R = len(reps)

    def capture(n, start):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn_per_step(reps[(start + i) % R])
        return g

    per = max(1, min(steps_per_graph, steps))
    per = max(R, (per // R) * R)          # whole rotations inside a graph
    g_full = capture(per, 0)
    rem = steps % per
    g_rem = capture(rem, 0) if rem else None
    torch.cuda.synchronize()
    for _ in range(max(1, warmup // per)):
        g_full.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps // per):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3


def chunked_flops(step) -> int:
    """Algorithmic FLOPs of the chunked pass: every unmasked (row, key) pair of
    every query head costs 2 D for q.k and 2 D for p v."""
    _, cu, _, ctx = step.chunk_batch()
    total = 0
    for i in range(len(ctx)):
        L, n = int(cu[i + 1] - cu[i]), int(ctx[i])
        total += L * (n - L) + L * (L + 1) // 2
    return total * step.num_q_heads * 4 * step.head_dim


def measure_chunked(dev, iters: int = 200, kv_dtype: str = "i8"):
    """The mixed int8 (or fp8) step: 4 x 512-row causal chunks over a
    1536-token cached prefix plus 124 decode rows. Times the chunked (MFMA)
    pass alone, and the whole step (cache write of 2172 rows, chunked pass,
    decode pass)."""
    import numpy as np
    import torch

    import paged_kv_attention_19_amd as pkv
    import workloads as W
    step = W.mixed_int8(kv_dtype=kv_dtype, max_tokens_per_split=MIXED_SPLIT)

    def dt(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    cache = pkv.KVCache.allocate(step.num_blocks, 8, 128, {"i8": pkv.I8, "fp8": pkv.FP8}[kv_dtype], dev)
    pkv.reshape_and_cache(dt(step.prefix_k, "bf16"), dt(step.prefix_v, "bf16"),
                          dt(step.prefix_slots.astype(np.int64), "i64"), cache)
    new_k, new_v = dt(step.new_k, "bf16"), dt(step.new_v, "bf16")
    new_s = dt(step.new_slots.astype(np.int64), "i64")
    # the step's new rows (the chunks' own K/V and the decode tokens) are in the
    # cache before any pass reads it; the whole-step timing writes them again
    # (the same bytes)
    pkv.reshape_and_cache(new_k, new_v, new_s, cache)
    qc, cu, tc, cc = step.chunk_batch()
    qc, cu, tc, cc = dt(qc, "bf16"), dt(cu, "i32"), dt(tc, "i32"), dt(cc, "i32")
    max_q = int(np.diff(step.chunk_batch()[1]).max())
    qd, td, ctxd, nsd = step.decode_batch()
    max_ns = int(nsd.max())   # the decode rows: ceil(n / MIXED_SPLIT) splits each
    qd, td, ctxd, nsd = dt(qd, "bf16"), dt(td, "i32"), dt(ctxd, "i32"), dt(nsd, "i32")
    out_c = torch.empty((qc.shape[0], 16, 128), dtype=torch.float32, device=dev)
    out_d = torch.empty((qd.shape[0], 16, 128), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(256, pkv.decode_workspace_bytes(qd.shape[0], 16, 128, max_ns)), dtype=torch.uint8, device=dev)
    scale = float(step.scale)

    def chunked():
        pkv.paged_attention_chunked(qc, cu, max_q, cache, tc, cc, scale, out=out_c)

    def whole():
        pkv.reshape_and_cache(new_k, new_v, new_s, cache)
        chunked()
        pkv.paged_attention_decode(qd, cache, td, ctxd, nsd, max_ns, scale, out=out_d, workspace=ws)

    res = {}
    for name, fn in (("chunked", chunked), ("step", whole)):
        fn()
        torch.cuda.synchronize()
        eager = (out_c.clone(), out_d.clone())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(20):
                fn()
        g.replay()
        torch.cuda.synchronize()
        # the replayed graph must reproduce the eager call bit for bit (and a
        # NaN, from a pool row never written, fails the comparison)
        if not torch.equal(out_c, eager[0]) or (name == "step" and not torch.equal(out_d, eager[1])):
            raise RuntimeError(f"the {name} graph replay differs from the eager call")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(max(1, iters // 20)):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) / 1e3 / (max(1, iters // 20) * 20)
    flops = chunked_flops(step)
    tflops = flops / res["chunked"] / 1e12
    kv_name = {"i8": "int8", "fp8": "fp8"}[kv_dtype]
    return {
        "workload": f"4 x 512-row causal chunks over 1536-token {kv_name} prefixes (16q/8kv/128), "
                    f"plus 124 {kv_name} decode rows in the whole step",
        "kernel": "chunked_kernel",
        "chunked_us": round(res["chunked"] * 1e6, 3),
        "algorithmic_gflop": round(flops / 1e9, 3),
        "tflops": round(tflops, 2),
        "mfma_util": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "whole_step_us": round(res["step"] * 1e6, 3),
    }


def cpu_baseline(step, seconds):
    """The oracle as it stands, on the host: decode sequences of the step one at
    a time (gather through the block table + float64 attention for every query
    head), cycling through the batch for about ``seconds``."""
    from threadpoolctl import threadpool_limits

    import oracle
    pool = oracle.OraclePool(step.num_blocks, step.num_kv_heads, step.block_size, step.head_dim, step.kv_dtype)
    oracle.reshape_and_cache(pool, step.prefix_k, step.prefix_v, step.src_dtype, step.prefix_slots)
    oracle.reshape_and_cache(pool, step.new_k, step.new_v, step.src_dtype, step.new_slots)
    q, tables, ctx, _ = step.decode_batch()
    q64 = oracle.decode_rows(q, step.q_dtype)
    eb, sb = {"f32": (4, 0), "bf16": (2, 0), "i8": (1, 4), "fp8": (1, 4)}[step.kv_dtype]
    per_tok = kv_bytes_per_token(step.num_kv_heads, step.head_dim, eb, sb)
    done_bytes = 0
    seqs = 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while True:
            b = seqs % len(ctx)
            oracle.paged_decode(q64[b:b + 1], pool, tables[b:b + 1], ctx[b:b + 1], step.scale)
            done_bytes += int(ctx[b]) * per_tok
            seqs += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{seqs} sequence decodes ({min(seqs, len(ctx))} distinct of the step's {len(ctx)}; "
                      f"{done_bytes / 1e6:.1f} MB of KV) in {el:.1f} s, float64 NumPy, BLAS limited to 1 thread"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures one GPU: the library has no multi-GPU path. Decode would shard by sequence or "
            "by KV head with no exchange, and a long context by splits merged with pkv_lse_combine. "
            "Run with --gpus 1.")
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    import paged_kv_attention_19_amd as pkv
    import workloads as W

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    pkv.lib()
    build, default_reps, default_mts, cfg_text = WORKLOADS[args.workload]
    if args.decode_mode is None:
        args.decode_mode = DEFAULT_MODES[args.workload]
    if args.max_tokens_per_split is None:
        args.max_tokens_per_split = default_mts
    if args.replicas is None:
        args.replicas = default_reps
    seed0 = DEFAULT_SEEDS[args.workload] if args.seed is None else args.seed
    t0 = time.time()
    reps = []
    for r in range(args.replicas):
        step = build(W, seed0, args.max_tokens_per_split, args.batch, r)
        reps.append(Replica(step, dev, args.max_tokens_per_split, balanced=args.decode_mode == "balanced",
                            fuse=not args.no_fuse))
    torch.cuda.synchronize()
    log(f"built {len(reps)} replicas in {time.time() - t0:.1f}s; max_ns={[r.max_ns for r in reps][:4]}...")

    # eager reference of one step per replica, then check graph replays against it
    eager = []
    for r in reps:
        r.step_once()
    torch.cuda.synchronize()
    for r in reps:
        eager.append((r.out.clone(), r.lse.clone()))
        r.out.fill_(float("nan"))
        r.lse.fill_(float("nan"))

    steps = args.steps
    sec = time_graphs(lambda r: r.step_once(), reps, steps, args.steps_per_graph, args.warmup)
    for r, (eo, el) in zip(reps, eager):
        if not (torch.equal(r.out, eo) and torch.equal(r.lse, el)):
            log("graph replay output differs from the eager step")
            sys.exit(1)
    R = len(reps)
    kv_total = sum(reps[i % R].kv_bytes for i in range(steps))
    seqs_total = sum(reps[i % R].batch for i in range(steps))
    value = kv_total / sec / 1e9

    # per-kernel launch durations: graphs holding one kind of launch
    per_kernel = {}
    n_k = min(steps, 4096)
    sec_p = time_graphs(lambda r: r.partials(), reps, n_k, args.steps_per_graph, 64)
    fused = reps[0].fused
    dom = "decode_balanced" if reps[0].balanced else ("decode_append" if fused else "decode_partial")
    per_kernel[dom] = sec_p / n_k
    if reps[0].max_ns > 1:
        sec_c = time_graphs(lambda r: r.combine(), reps, n_k, args.steps_per_graph, 64)
        per_kernel["lse_combine"] = sec_c / n_k
    sec_r = time_graphs(lambda r: r.reshape(), reps, n_k, args.steps_per_graph, 64)
    per_kernel["reshape_and_cache"] = sec_r / n_k
    partial_bytes = sum(reps[i % R].kv_bytes for i in range(n_k)) / n_k
    # algorithmic bytes of the dominant launch: the KV it reads, plus, when it
    # appends, the new rows it reads and writes
    launch_bytes = partial_bytes + (sum(reps[i % R].append_bytes for i in range(n_k)) / n_k if fused else 0)
    achieved = launch_bytes / per_kernel[dom] / 1e9

    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("workload") == args.workload
                and tr.get("decode_mode") == args.decode_mode and tr.get("append") == fused
                and tr.get("max_tokens_per_split") == args.max_tokens_per_split):
            traffic = tr.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        pass

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec / steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "i8": "i8 kv / bf16 q",
                  "fp8": "fp8 e4m3 kv / bf16 q"}[reps[0].step.kv_dtype],
        "data": "synthetic",
        "config": dict(cfg_text, **{
            "batch": reps[0].batch,
            "num_q_heads": 16, "num_kv_heads": 8, "head_dim": 128, "block_size": 16,
            "decode_mode": args.decode_mode,
            "append": "in the decode pass" if fused else "separate reshape_and_cache launch",
            "max_tokens_per_split": None if reps[0].balanced else args.max_tokens_per_split,
            "replicas": R, "kv_bytes_per_step": int(kv_total / steps),
            "parallelism": "none",
        }),
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "seq_steps_per_s": round(seqs_total / sec, 1),
        "kernel_us": {k: round(v * 1e6, 3) for k, v in per_kernel.items()},
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_balanced_kernel" if reps[0].balanced else "decode_partial_kernel",
            "algorithmic_bytes": int(launch_bytes),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
    }
    line["copy_reference"] = copy_reference(int(partial_bytes))
    if not args.no_chunked:
        log("timing the chunked prefill ...")
        line["chunked_prefill"] = measure_chunked(dev, kv_dtype=args.chunked_kv)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        line["cpu_baseline"] = cpu_baseline(reps[0].step, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
