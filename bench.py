#!/usr/bin/env python3
"""Decode-step benchmark of the paged-KV attention library on one MI355X.

A step is one pass of the decode hot path over one batch: reshape_and_cache of
the batch's new token (one row per sequence), the split-K partial pass, and the
log-sum-exp merge. The workload is a Qwen3-0.6B-shaped single layer: 32
sequences, 16 query / 8 KV heads, head_dim 128, bf16 q/K/V from N(0, 1),
context lengths uniform in [128, 384], 16-token blocks drawn from a 4096-block
pool. Inputs are resident in HBM before timing starts.

One step's KV (34.4 MB) would sit in MI355X's 256 MB Infinity Cache if the
same step were repeated, so the timed loop rotates through R replicas that
stand for R layers of one model step: they share the batch's block tables,
context lengths and slots (as an engine's layers do) and each owns its KV pool
and its q/K/V values. Between two uses of one replica the other R - 1 replicas
stream well over 256 MB of KV, so every step reads its KV from HBM.
Steps are launched from HIP graphs (each graph holds many steps) so that host
launch cost does not pace the GPU.

Timing: a window is exactly --steps steps, bracketed by HIP events on the
stream the work runs on. Windows are replayed back to back until at least
--min-seconds of GPU time and 5 windows have run (so a small --steps still
gives a stable figure), and the median window gives the per-step time.

Output: one JSON line on stdout (everything else goes to stderr).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn decode KV GB/s (% HBM peak) + seq-steps/s; chunked-prefill MFMA util"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16, published
# the files a kernel's code is built from (its per-source compiler flags
# included): profile figures recorded for other contents are not used
DECODE_FILES = ("paged_kv_attention_19_amd/csrc/decode_kernel.h", "paged_kv_attention_19_amd/csrc/decode_core.h",
                "paged_kv_attention_19_amd/csrc/decode_bf16.hip", "paged_kv_attention_19_amd/csrc/pkv_device.h",
                "paged_kv_attention_19_amd/csrc/quant_row.h", "paged_kv_attention_19_amd/csrc/api.hip",
                "paged_kv_attention_19_amd/build.py")
CHUNKED_FILES = ("paged_kv_attention_19_amd/csrc/chunked.hip", "paged_kv_attention_19_amd/csrc/pkv_device.h",
                 "paged_kv_attention_19_amd/csrc/api.hip", "paged_kv_attention_19_amd/build.py")
DECODE_PROFILE = os.path.join(ROOT, "profiles", "decode_partial_qwen3_traffic.json")
CHUNKED_PROFILE = os.path.join(ROOT, "profiles", "chunked_kernel_mixed_int8_traffic.json")
WINDOWS_MIN = 5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int, scale_bytes: int = 0,
                       layers: int = 1) -> int:
    """Algorithmic KV bytes one token of one layer holds: K and V rows of every
    KV head, plus their scales for int8."""
    return layers * 2 * num_kv_heads * (head_dim * elem_bytes + scale_bytes)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    return source_hash(DECODE_FILES)


def profile_figures(path: str, files, **match):
    """Counter / trace figures recorded in profiles/ for the current sources
    of a kernel (None if the kernel changed since they were taken, or if the
    profile was taken on another configuration)."""
    try:
        with open(path) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None
    if tr.get("kernel_source_hash") != source_hash(files):
        return None
    for k, v in match.items():
        if tr.get(k) != v:
            return None
    return tr


# The mixed step leaves the decode rows' split to the caller. Measured on
# MI355X (int8, decode launch alone): 110.5 us with 512-token splits, 104.1 with
# 1024, 103.9 with 1536, 108.1 with 2048 and 123.5 with one split per sequence:
# longer splits spread each workgroup's start-up over more blocks until too few
# workgroups are left to fill the GPU.
MIXED_SPLIT = 1024

# name -> (builder(W, seed, max_tokens_per_split, batch, replica), default replicas, default split size, config)
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
    # the same decode rows over a bf16 cache: the int8 rows' traffic compared at the same tokens
    "mixed_bf16_decode": (lambda W, seed, mts, batch, r: W.mixed_int8(seed=seed + 1000 * r, kv_dtype="bf16",
                                                                       max_tokens_per_split=mts or MIXED_SPLIT),
                          1, MIXED_SPLIT, {"workload": "mixed_bf16_step_decode_rows", "context_lens": "uniform[256,4096]"}),
}
DEFAULT_SEEDS = {"qwen3_decode": 1902, "ragged_decode": 1903, "long_decode": 1904, "mixed_int8_decode": 1905,
                 "mixed_fp8_decode": 1905, "mixed_bf16_decode": 1905}
# Decode mode measured fastest on MI355X per shape: one workgroup per
# (split, kv head) for the Qwen3 step (one split per sequence), the uniform
# long contexts (64 splits of 512 tokens, as the workload states) and the
# mixed step's decode rows (1024-token splits); the log-uniform ragged batch
# gains from the balanced deal of tiles.
DEFAULT_MODES = {"qwen3_decode": "splits", "ragged_decode": "balanced", "long_decode": "splits",
                 "mixed_int8_decode": "splits", "mixed_fp8_decode": "splits", "mixed_bf16_decode": "splits"}
# the other decode configurations reported beside the headline one (each in
# its default mode and split plan)
OTHER_CONFIGS = ("ragged_decode", "long_decode", "mixed_int8_decode")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8192, help="steps per timed window")
    ap.add_argument("--warmup", type=int, default=512)
    ap.add_argument("--min-seconds", type=float, default=0.25,
                    help="windows of --steps steps are timed until at least this much GPU time (and 5 windows)")
    ap.add_argument("--replicas", type=int, default=None,
                    help="independent copies rotated through (default: 16 for the Qwen3 step, else 1)")
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--max-tokens-per-split", type=int, default=None,
                    help="num_splits[b] = ceil(n_b / this); 0 = one split per sequence "
                         "(default: 0 for the Qwen3 step, 1024 for the mixed step's decode rows, 512 for the others)")
    ap.add_argument("--steps-per-graph", type=int, default=256)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunked", action="store_true", help="skip the chunked-prefill MFMA measurement")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other decode configurations and the speculative-verify shape")
    ap.add_argument("--chunked-kv", choices=("i8", "fp8", "bf16"), default="i8",
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


def window_plan(steps: int, steps_per_graph: int, replicas: int):
    """How a window of exactly ``steps`` steps is captured: ``(per, n_full,
    rem)`` = ``n_full`` replays of a graph of ``per`` steps, then one graph of
    ``rem`` steps (none if 0). Up to ``steps_per_graph`` steps the window is one
    graph; past that the repeated graph holds whole rotations over the
    replicas, so every replay starts at replica 0 and the window's steps still
    visit the replicas in order."""
    if steps <= steps_per_graph:
        return steps, 1, 0
    per = max(replicas, (steps_per_graph // replicas) * replicas)
    return per, steps // per, steps % per


def time_windows(fn_per_step, reps, steps, steps_per_graph, warmup, min_seconds):
    """Time windows of exactly ``steps`` consecutive steps (rotating over the
    replicas), captured as one HIP graph when ``steps <= steps_per_graph``, else
    in graphs of whole rotations of at most ``steps_per_graph`` steps, and
    replayed back to back until at least ``min_seconds`` of GPU time and
    WINDOWS_MIN windows have run. Returns (median seconds per window, windows,
    total timed seconds)."""
    import torch
    R = len(reps)

    def capture(n, start):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn_per_step(reps[(start + i) % R])
        return g

    per, n_full, rem = window_plan(steps, steps_per_graph, R)
    g_full = capture(per, 0) if n_full else None
    g_rem = capture(rem, 0) if rem else None

    def window():
        for _ in range(n_full):
            g_full.replay()
        if g_rem is not None:
            g_rem.replay()

    torch.cuda.synchronize()
    for _ in range(max(1, -(-warmup // max(1, steps)))):
        window()
    torch.cuda.synchronize()
    # one window to size the run
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    window()
    b.record()
    torch.cuda.synchronize()
    one = max(a.elapsed_time(b) / 1e3, 1e-7)
    nwin = max(WINDOWS_MIN, math.ceil(min_seconds / one))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nwin + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(nwin):
        window()
        ev[i + 1].record()
    torch.cuda.synchronize()
    secs = sorted(ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(nwin))
    total = ev[0].elapsed_time(ev[-1]) / 1e3
    return secs[nwin // 2], nwin, total


class Replica:
    """One independent copy of the workload, resident on the GPU."""

    def __init__(self, step, dev, balanced=False, fuse=True):
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


def build_replicas(W, dev, workload, replicas, mts, batch, mode, fuse, seed=None):
    build, _, _, _ = WORKLOADS[workload]
    seed0 = DEFAULT_SEEDS[workload] if seed is None else seed
    return [Replica(build(W, seed0, mts, batch, r), dev, balanced=mode == "balanced", fuse=fuse)
            for r in range(replicas)]


def check_replays_against_eager(reps, per_step, steps, steps_per_graph):
    """An eager step per replica, then graph replays of the same steps: the
    outputs must agree bit for bit (a NaN from an unwritten pool row fails
    the comparison too)."""
    import torch
    for r in reps:
        per_step(r)
    torch.cuda.synchronize()
    eager = [(r.out.clone(), r.lse.clone()) for r in reps]
    for r in reps:
        r.out.fill_(float("nan"))
        r.lse.fill_(float("nan"))
    time_windows(per_step, reps, max(len(reps), min(steps, steps_per_graph)), steps_per_graph, 0, 0.0)
    for r, (eo, el) in zip(reps, eager):
        if not (torch.equal(r.out, eo) and torch.equal(r.lse, el)):
            raise RuntimeError("graph replay output differs from the eager step")


def stream_reference(nbytes: int, min_seconds: float):
    """A read-only stream over the same number of bytes as one decode launch
    reads (pkv_stream_read: 16-byte non-temporal loads and nothing else),
    rotated over enough buffers (>= 1 GiB in all) that every launch reads
    from HBM, graph-replayed like the decode: what a kernel that only reads
    these bytes reaches on this machine, launch and drain included."""
    import torch

    import paged_kv_attention_19_amd as pkv
    nb = max(16, (int(nbytes) // 16) * 16)
    copies = max(1, min(16, math.ceil((1 << 30) / nb)))
    bufs = []
    for _ in range(copies):
        src = torch.randint(-128, 127, (nb,), dtype=torch.int8, device="cuda:0")
        sink = torch.zeros(max(1, int(pkv.lib().pkv_stream_read_workgroups(nb))), dtype=torch.int32, device="cuda:0")
        bufs.append((src, sink))
    steps = max(copies, 64 * copies if nb < (64 << 20) else 4 * copies)
    sec, nwin, _ = time_windows(lambda b: pkv.stream_read(b[0], b[1]), bufs, steps, 256, steps, min_seconds)
    per = sec / steps
    return {"kernel": "stream_read_kernel", "bytes": nb, "buffers": copies, "us": round(per * 1e6, 3),
            "GB/s": round(nb / per / 1e9, 1), "frac_of_peak": round(nb / per / 1e9 / HBM_PEAK_GBS, 4)}


def decode_figures(reps, args, per_step_time, n_steps):
    """Per-step figures of a decode configuration from its median window."""
    R = len(reps)
    kv = sum(reps[i % R].kv_bytes for i in range(n_steps)) / n_steps
    seqs = sum(reps[i % R].batch for i in range(n_steps)) / n_steps
    gbs = kv / per_step_time / 1e9
    return kv, seqs, gbs


def measure_other(W, dev, workload, min_seconds):
    """One of the other decode configurations, in its default mode and split
    plan: one replica (each reads 0.6-1.7 GB of KV per step, far past the
    Infinity Cache), the step timed in windows like the headline one."""
    import torch
    mode = DEFAULT_MODES[workload]
    mts = WORKLOADS[workload][2]
    t0 = time.time()
    reps = build_replicas(W, dev, workload, 1, mts, 32, mode, True)
    torch.cuda.synchronize()
    log(f"  built {workload} in {time.time() - t0:.1f}s")
    check_replays_against_eager(reps, lambda r: r.step_once(), 4, 4)
    steps = 64
    sec, nwin, _ = time_windows(lambda r: r.step_once(), reps, steps, 16, 16, min_seconds)
    per = sec / steps
    kv, seqs, gbs = decode_figures(reps, None, per, steps)
    r = reps[0]
    res = {
        "config": WORKLOADS[workload][3]["workload"],
        "decode_mode": mode,
        "max_tokens_per_split": None if mode == "balanced" else mts,
        "append": "in the decode pass" if r.fused else "separate reshape_and_cache launch",
        "kv_dtype": r.step.kv_dtype,
        "batch": r.batch,
        "kv_bytes_per_step": int(kv),
        "us_per_step": round(per * 1e6, 2),
        "GB/s": round(gbs, 1),
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "seq_steps_per_s": round(seqs / per, 1),
        "windows": nwin,
    }
    res["stream_ceiling"] = stream_reference(int(kv), min_seconds)
    res["frac_of_stream"] = round(gbs / res["stream_ceiling"]["GB/s"], 4)
    del reps
    torch.cuda.empty_cache()
    return res


def chunked_flops(step) -> int:
    """Algorithmic FLOPs of the chunked pass: every unmasked (row, key) pair of
    every query head costs 2 D for q.k and 2 D for p v."""
    _, cu, _, ctx = step.chunk_batch()
    total = 0
    for i in range(len(ctx)):
        L, n = int(cu[i + 1] - cu[i]), int(ctx[i])
        total += L * (n - L) + L * (L + 1) // 2
    return total * step.num_q_heads * 4 * step.head_dim


def _dt(a, kind, dev):
    import numpy as np
    import torch
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


# Replicas of the mixed step for the chunked measurement: separate caches and
# queries (about 600 MB each, 4.8 GB in all), the calls rotating over them, so
# that no call finds its bytes in the caches from the one before (measured on
# MI355X: 55.6 us per chunked call over 8 replicas against 54.2 us over one).
CHUNKED_REPLICAS = 8


def measure_chunked(dev, min_seconds, kv_dtype: str = "i8", replicas: int = CHUNKED_REPLICAS):
    """The mixed int8 (or fp8, bf16) step: 4 x 512-row causal chunks over a
    1536-token cached prefix plus 124 decode rows. Times the chunked (MFMA)
    pass alone, and the whole step (cache write of 2172 rows, chunked pass,
    decode pass), each rotating over ``replicas`` copies of the step (the same
    shapes and tables, other values)."""
    import types

    import numpy as np
    import torch

    import paged_kv_attention_19_amd as pkv
    import workloads as W
    reps = []
    for r in range(replicas):
        step = W.mixed_int8(kv_dtype=kv_dtype, max_tokens_per_split=MIXED_SPLIT, values_seed=1905 + 1000 * r)
        code = {"i8": pkv.I8, "fp8": pkv.FP8, "bf16": pkv.BF16}[kv_dtype]
        x = types.SimpleNamespace()
        x.cache = pkv.KVCache.allocate(step.num_blocks, 8, 128, code, dev)
        pkv.reshape_and_cache(_dt(step.prefix_k, "bf16", dev), _dt(step.prefix_v, "bf16", dev),
                              _dt(step.prefix_slots.astype(np.int64), "i64", dev), x.cache)
        x.new_k, x.new_v = _dt(step.new_k, "bf16", dev), _dt(step.new_v, "bf16", dev)
        x.new_s = _dt(step.new_slots.astype(np.int64), "i64", dev)
        # the step's new rows (the chunks' own K/V and the decode tokens) are
        # in the cache before any pass reads it; the whole-step timing writes
        # them again (the same bytes)
        pkv.reshape_and_cache(x.new_k, x.new_v, x.new_s, x.cache)
        qc_h, cu_h, tc_h, cc_h = step.chunk_batch()
        x.qc, x.cu, x.tc, x.cc = _dt(qc_h, "bf16", dev), _dt(cu_h, "i32", dev), _dt(tc_h, "i32", dev), _dt(cc_h, "i32", dev)
        x.max_q = int(np.diff(cu_h).max())
        qd, td, ctxd, nsd = step.decode_batch()
        x.max_ns = int(nsd.max())   # the decode rows: ceil(n / MIXED_SPLIT) splits each
        x.qd, x.td, x.ctxd, x.nsd = _dt(qd, "bf16", dev), _dt(td, "i32", dev), _dt(ctxd, "i32", dev), _dt(nsd, "i32", dev)
        x.out_c = torch.empty((x.qc.shape[0], 16, 128), dtype=torch.float32, device=dev)
        x.out_d = torch.empty((x.qd.shape[0], 16, 128), dtype=torch.float32, device=dev)
        x.ws = torch.zeros(max(256, pkv.decode_workspace_bytes(x.qd.shape[0], 16, 128, x.max_ns)), dtype=torch.uint8,
                           device=dev)
        x.scale = float(step.scale)
        reps.append(x)

    def chunked(x):
        pkv.paged_attention_chunked(x.qc, x.cu, x.max_q, x.cache, x.tc, x.cc, x.scale, out=x.out_c)

    def whole(x):
        pkv.reshape_and_cache(x.new_k, x.new_v, x.new_s, x.cache)
        chunked(x)
        pkv.paged_attention_decode(x.qd, x.cache, x.td, x.ctxd, x.nsd, x.max_ns, x.scale, out=x.out_d, workspace=x.ws)

    def check(fn, outs):
        """An eager call per replica, then graph replays of the same calls: the
        outputs must agree bit for bit."""
        for x in reps:
            fn(x)
        torch.cuda.synchronize()
        eager = [[o.clone() for o in outs(x)] for x in reps]
        for x in reps:
            for o in outs(x):
                o.fill_(float("nan"))
        time_windows(fn, reps, len(reps), len(reps), 0, 0.0)
        for x, e in zip(reps, eager):
            if not all(torch.equal(o, eo) for o, eo in zip(outs(x), e)):
                raise RuntimeError("the graph replay differs from the eager call")

    calls = 4 * replicas   # calls per timed window
    check(chunked, lambda x: (x.out_c,))
    s_chunked, nwin, _ = time_windows(chunked, reps, calls, calls, calls, min_seconds)
    check(whole, lambda x: (x.out_c, x.out_d))
    s_step, _, _ = time_windows(whole, reps, calls, calls, calls, min_seconds)
    t_chunked, t_step = s_chunked / calls, s_step / calls
    flops = chunked_flops(step)   # every replica has the same shapes
    tflops = flops / t_chunked / 1e12
    kv_name = {"i8": "int8", "fp8": "fp8", "bf16": "bf16"}[kv_dtype]
    prof = profile_figures(CHUNKED_PROFILE, CHUNKED_FILES, kv_dtype=kv_dtype)
    return {
        "workload": f"4 x 512-row causal chunks over 1536-token {kv_name} prefixes (16q/8kv/128), "
                    f"plus 124 {kv_name} decode rows in the whole step",
        "kernel": "chunked_kernel",
        "chunked_us": round(t_chunked * 1e6, 3),
        "algorithmic_gflop": round(flops / 1e9, 3),
        "tflops": round(tflops, 2),
        "mfma_util": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "whole_step_us": round(t_step * 1e6, 3),
        "windows": nwin,
        "replicas": replicas,
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": prof.get("hbm_bytes_per_launch") if prof else None,
            "trace_us": prof.get("kernel_trace_us") if prof else None,
        },
    }


def measure_spec_verify(dev, min_seconds):
    """Speculative verification: 32 sequences, each checking 4 draft rows at
    positions n - 4 .. n - 1 over its paged history (n uniform in [128, 384],
    the Qwen3 heads, bf16), through the chunked entry point whose offset-causal
    mask is the verification rule. 16 replicas (layers) are rotated so the KV
    comes from HBM; reported as KV GB/s like the decode."""
    import numpy as np
    import torch

    import paged_kv_attention_19_amd as pkv
    import workloads as W
    reps = []
    for r in range(16):
        rng = np.random.default_rng(np.random.SeedSequence([1906, 7]))
        ctx = rng.integers(128, 384, size=32, endpoint=True)
        step = W.make_step("spec_verify", ctx, np.full(32, 4), num_q_heads=16, num_kv_heads=8, head_dim=128,
                           num_blocks=4096, seed=1906, values_seed=1906 + 1000 * r)
        cache = pkv.KVCache.allocate(step.num_blocks, 8, 128, pkv.BF16, dev)
        for k, v, s in ((step.prefix_k, step.prefix_v, step.prefix_slots), (step.new_k, step.new_v, step.new_slots)):
            pkv.reshape_and_cache(_dt(k, "bf16", dev), _dt(v, "bf16", dev), _dt(s.astype(np.int64), "i64", dev), cache)
        q, cu, tab, cc = step.chunk_batch()
        reps.append(dict(q=_dt(q, "bf16", dev), cu=_dt(cu, "i32", dev), tab=_dt(tab, "i32", dev),
                         ctx=_dt(cc, "i32", dev), cache=cache, scale=float(step.scale),
                         out=torch.empty((q.shape[0], 16, 128), dtype=torch.float32, device=dev),
                         kv=int(cc.sum()) * kv_bytes_per_token(8, 128, 2)))

    def call(r):
        pkv.paged_attention_chunked(r["q"], r["cu"], 4, r["cache"], r["tab"], r["ctx"], r["scale"], out=r["out"])

    steps = 512
    sec, nwin, _ = time_windows(call, reps, steps, 256, 64, min_seconds)
    per = sec / steps
    kv = sum(r["kv"] for r in reps) / len(reps)
    return {"config": "spec_verify_b32_q4", "entry_point": "pkv_paged_attention_chunked",
            "kernel": "rows_mfma_kernel (8 rows per kv head)", "rows_per_seq": 4, "context_lens": "uniform[128,384]",
            "kv_bytes_per_step": int(kv),
            "us_per_step": round(per * 1e6, 2), "GB/s": round(kv / per / 1e9, 1),
            "hbm_peak_frac": round(kv / per / 1e9 / HBM_PEAK_GBS, 4), "seq_steps_per_s": round(32 / per, 1),
            "windows": nwin}


# ---------------------------------------------------------------------------
# the oracle on the host (run before the GPU is touched: the all-core timing
# forks worker processes, which must not inherit an initialised GPU runtime)
# ---------------------------------------------------------------------------

_CPU = {}


def _cpu_setup(step):
    import oracle
    pool = oracle.OraclePool(step.num_blocks, step.num_kv_heads, step.block_size, step.head_dim, step.kv_dtype)
    oracle.reshape_and_cache(pool, step.prefix_k, step.prefix_v, step.src_dtype, step.prefix_slots)
    oracle.reshape_and_cache(pool, step.new_k, step.new_v, step.src_dtype, step.new_slots)
    q, tables, ctx, _ = step.decode_batch()
    eb, sb = {"f32": (4, 0), "bf16": (2, 0), "i8": (1, 4), "fp8": (1, 4)}[step.kv_dtype]
    _CPU.update(pool=pool, q64=oracle.decode_rows(q, step.q_dtype), tables=tables, ctx=ctx, scale=step.scale,
                per_tok=kv_bytes_per_token(step.num_kv_heads, step.head_dim, eb, sb))


def _cpu_worker(args):
    """Decode sequences start, start + stride, ... (cycling) for `seconds`
    with BLAS on one thread; returns (KV bytes, sequences, seconds)."""
    start, stride, seconds = args
    from threadpoolctl import threadpool_limits

    import oracle
    c = _CPU
    done = seqs = 0
    B = len(c["ctx"])
    with threadpool_limits(1):
        t0 = time.perf_counter()
        b = start
        while True:
            i = b % B
            oracle.paged_decode(c["q64"][i:i + 1], c["pool"], c["tables"][i:i + 1], c["ctx"][i:i + 1], c["scale"])
            done += int(c["ctx"][i]) * c["per_tok"]
            seqs += 1
            b += stride
            el = time.perf_counter() - t0
            if el >= seconds:
                return done, seqs, el


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(step, seconds):
    """The oracle as it stands, on the host: decode sequences of the step one at
    a time (gather through the block table + float64 attention for every query
    head), on one core, then on every core the process may use (at most 16) in
    worker processes, each on its own share of the batch."""
    import multiprocessing as mp
    _cpu_setup(step)
    B = len(_CPU["ctx"])
    done, seqs, el = _cpu_worker((0, 1, seconds))
    one = {"value": round(done / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{seqs} sequence decodes ({min(seqs, B)} distinct of the step's {B}; "
                     f"{done / 1e6:.1f} MB of KV) in {el:.1f} s, float64 NumPy, BLAS on 1 thread"}
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        avail = os.cpu_count() or 1
    n = max(1, min(16, avail))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(n) as pool:
        res = pool.map(_cpu_worker, [(i, n, seconds) for i in range(n)])
    wall = time.perf_counter() - t0
    done_all = sum(r[0] for r in res)
    seqs_all = sum(r[1] for r in res)
    one["all_cores"] = {"value": round(done_all / wall / 1e9, 4), "unit": "GB/s", "cores": n,
                        "sample": f"{seqs_all} sequence decodes ({done_all / 1e6:.1f} MB of KV) over {n} worker "
                                  f"processes (one per core, BLAS on 1 thread each) in {wall:.1f} s of wall time"}
    one["cpu_model"] = cpu_model()
    one["cpus_visible"] = avail
    return one


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

    import workloads as W
    build, default_reps, default_mts, cfg_text = WORKLOADS[args.workload]
    if args.decode_mode is None:
        args.decode_mode = DEFAULT_MODES[args.workload]
    if args.max_tokens_per_split is None:
        args.max_tokens_per_split = default_mts
    if args.replicas is None:
        args.replicas = default_reps

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        seed0 = DEFAULT_SEEDS[args.workload] if args.seed is None else args.seed
        cpu = cpu_baseline(build(W, seed0, args.max_tokens_per_split, args.batch, 0), args.cpu_seconds)

    import torch

    import paged_kv_attention_19_amd as pkv
    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    pkv.lib()
    t0 = time.time()
    reps = build_replicas(W, dev, args.workload, args.replicas, args.max_tokens_per_split, args.batch,
                          args.decode_mode, not args.no_fuse, seed=args.seed)
    torch.cuda.synchronize()
    log(f"built {len(reps)} replicas in {time.time() - t0:.1f}s; max_ns={[r.max_ns for r in reps][:4]}...")
    check_replays_against_eager(reps, lambda r: r.step_once(), args.steps, args.steps_per_graph)

    steps = args.steps
    sec, nwin, timed = time_windows(lambda r: r.step_once(), reps, steps, args.steps_per_graph, args.warmup,
                                    args.min_seconds)
    per_step = sec / steps
    R = len(reps)
    kv_step, seqs_step, value = decode_figures(reps, args, per_step, steps)

    # per-kernel launch durations: graphs holding one kind of launch, timed
    # in windows the same way, of 4096 launches whatever --steps is (so that
    # a graph's own launch is spread over enough kernel launches)
    per_kernel = {}
    n_k = 4096
    fused = reps[0].fused
    dom = "decode_balanced" if reps[0].balanced else ("decode_append" if fused else "decode_partial")
    sp, _, _ = time_windows(lambda r: r.partials(), reps, n_k, args.steps_per_graph, 64, args.min_seconds)
    per_kernel[dom] = sp / n_k
    if reps[0].max_ns > 1:
        sc, _, _ = time_windows(lambda r: r.combine(), reps, n_k, args.steps_per_graph, 64, args.min_seconds)
        per_kernel["lse_combine"] = sc / n_k
    sr, _, _ = time_windows(lambda r: r.reshape(), reps, n_k, args.steps_per_graph, 64, args.min_seconds)
    per_kernel["reshape_and_cache"] = sr / n_k
    partial_bytes = sum(reps[i % R].kv_bytes for i in range(n_k)) / n_k
    # algorithmic bytes of the dominant launch: the KV it reads, plus, when it
    # appends, the new rows it reads and writes
    launch_bytes = partial_bytes + (sum(reps[i % R].append_bytes for i in range(n_k)) / n_k if fused else 0)
    achieved = launch_bytes / per_kernel[dom] / 1e9
    prof = profile_figures(DECODE_PROFILE, DECODE_FILES, workload=args.workload, decode_mode=args.decode_mode,
                           append=fused, max_tokens_per_split=args.max_tokens_per_split)
    trace_us = prof.get("kernel_trace_us") if prof else None

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(per_step * 1e3, 6),
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
            "replicas": R, "kv_bytes_per_step": int(kv_step),
            "parallelism": "none",
        }),
        "timing": {"steps_per_window": steps, "windows": nwin, "stat": "median window", "timed_s": round(timed, 3)},
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "seq_steps_per_s": round(seqs_step / per_step, 1),
        "kernel_us": {k: round(v * 1e6, 3) for k, v in per_kernel.items()},
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_balanced_kernel" if reps[0].balanced else "decode_partial_kernel",
            "algorithmic_bytes": int(launch_bytes),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": prof.get("hbm_bytes_per_launch") if prof else None,
            "trace_us": trace_us,
            "trace_frac": round(launch_bytes / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if trace_us else None,
        },
    }
    del reps
    torch.cuda.empty_cache()
    log("timing the read-only stream ceiling ...")
    line["stream_ceiling"] = stream_reference(int(partial_bytes), args.min_seconds)
    line["frac_of_stream"] = round(value / line["stream_ceiling"]["GB/s"], 4)
    line["roofline"]["frac_of_stream"] = round(achieved / line["stream_ceiling"]["GB/s"], 4)
    if not args.no_chunked:
        log("timing the chunked prefill ...")
        line["chunked_prefill"] = measure_chunked(dev, args.min_seconds, kv_dtype=args.chunked_kv)
    if not args.no_others:
        line["other_configs"] = {}
        for wl in OTHER_CONFIGS:
            if wl == args.workload:
                continue
            log(f"timing {wl} ...")
            r = measure_other(W, dev, wl, args.min_seconds)
            line["other_configs"][r.pop("config")] = r
        log("timing the speculative-verify shape ...")
        line["spec_verify"] = measure_spec_verify(dev, args.min_seconds)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
