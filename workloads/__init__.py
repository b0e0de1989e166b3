"""Seeded synthetic inputs for paged-KV attention.

This module is shared by the tests, the bench and the oracle's callers. It
holds none of the method's arithmetic: it draws random values, rounds them to
their storage dtype, and lays out block tables and slot lists the way an
engine's block allocator would. The attention, the scatter, the quantizer and
the split rule live on each side separately (``oracle/`` and the HIP library).
"""

from .synth import (  # noqa: F401
    Step,
    f32_to_bf16_bits,
    long_decode,
    make_step,
    mixed_int8,
    qwen3_decode,
    ragged_decode,
    tiny_decode,
)
