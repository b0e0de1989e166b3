"""Plain CPU oracle for paged-KV attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything under ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. The oracle shares no code
with the HIP path (no kernels, headers, helpers, tables or pre/post-processing);
the two meet only in the seeded input generators of ``workloads/``, which hold
none of the method's arithmetic.

What it computes is the plain definition of the operation: softmax attention
of each new query row over the sequence's KV history, gathered into contiguous
arrays through the per-request block table, in float64. The paged, online and
split-K machinery of the HIP path reaches that same result by another route;
the pages state that these variants agree with the plain definition (course
README "Build an LLM Inference Engine From Scratch", section "The code asserts
its own claims", claims s06 and s12).

Every function is pinned by ``tests/test_oracle_*.py`` against things other
than itself: brute force on tiny inputs, closed forms, a library routine
(``torch.nn.functional.scaled_dot_product_attention`` in float64 on CPU),
invariants the pages state, and planted-mistake tests. Functions with no such
pin would say "parity unpinned" here; there are none.
"""

from .paged_attention import (  # noqa: F401
    BF16,
    F32,
    FP8,
    I8,
    NAN_BF16_BITS,
    NAN_FP8_CODE,
    OraclePool,
    attend_direct,
    bf16_bits_to_f64,
    decode_rows,
    fp8_e4m3_value,
    gather_kv,
    kv_head_of,
    lse_combine,
    online_softmax_attend,
    paged_chunked,
    paged_decode,
    quantize_rows_fp8,
    quantize_rows_int8,
    reshape_and_cache,
    split_bounds,
    split_k_decode,
)
