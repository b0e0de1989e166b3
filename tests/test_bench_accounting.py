"""The bench's algorithmic KV-byte accounting, pinned to the memory figures
the pages print (tests/golden/kv_cache_memory.txt): with 8 KV heads the
per-token bytes reproduce "about 50 MB" at batch 1 and "nearly 12 GB" at
batch 256; the 16-KV-head reading of "16H" does not."""

import os

import bench

GOLD = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_memory.txt")


def load():
    vals = {}
    for line in open(GOLD):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


def cache_bytes(batch, kv_heads, g):
    tokens = g["prompt_tokens"] + g["generated_tokens"]
    return batch * tokens * bench.kv_bytes_per_token(kv_heads, int(g["head_dim"]), int(g["elem_bytes"]),
                                                     layers=int(g["layers"]))


def test_eight_kv_heads_reproduce_the_printed_cache_sizes():
    g = load()
    b1 = cache_bytes(1, 8, g)
    b256 = cache_bytes(256, 8, g)
    assert 0.8 * g["batch_1_about_bytes"] <= b1 <= 1.2 * g["batch_1_about_bytes"]
    assert 0.9 * g["batch_256_nearly_bytes"] <= b256 <= g["batch_256_nearly_bytes"]


def test_sixteen_kv_heads_would_not():
    g = load()
    assert cache_bytes(1, 16, g) > 1.2 * g["batch_1_about_bytes"]
    assert cache_bytes(256, 16, g) > g["batch_256_nearly_bytes"]


def test_int8_bytes_include_the_scales():
    assert bench.kv_bytes_per_token(8, 128, 1, 4) == 2 * 8 * (128 + 4)
    assert bench.kv_bytes_per_token(8, 128, 2) == 4096
