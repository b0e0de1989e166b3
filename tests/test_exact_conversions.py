"""CPU pins of the exactness facts the 8-bit cache paths rely on, checked
over every code:

- an int8 code c, with its sign bit flipped (u = c + 128) and placed as the
  low byte under the high byte 0x64, is the fp16 number 1024 + u; subtracting
  1152 in fp16 leaves exactly c;
- every finite OCP E4M3 value is exactly representable in fp16 and in bf16;
- every int8 code is exactly representable in bf16 and in fp16.

These are properties of the number formats, so the checks use numpy and
torch's CPU dtypes only."""

from __future__ import annotations

import numpy as np
import torch


def test_int8_to_fp16_by_byte_placement_is_exact():
    c = np.arange(-128, 128, dtype=np.int16)
    u = (c.astype(np.int32) & 0xFF) ^ 0x80                     # sign bit flipped: c + 128
    assert np.array_equal(u, c + 128)
    bits = (0x6400 | u).astype(np.uint16)
    h = bits.view(np.float16)
    assert np.array_equal(h.astype(np.float64), 1024.0 + u)   # the fp16 numbers 1024 .. 1279, spacing 1
    back = (h - np.float16(1152.0)).astype(np.float16)        # one fp16 subtraction (exact: integers < 2048)
    assert np.array_equal(back.astype(np.float64), c.astype(np.float64))


def test_int8_codes_are_exact_in_bf16_and_fp16():
    c = torch.arange(-127, 128, dtype=torch.float32)
    assert torch.equal(c.to(torch.bfloat16).to(torch.float32), c)
    assert torch.equal(c.to(torch.float16).to(torch.float32), c)


def test_e4m3_values_are_exact_in_fp16_and_bf16():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    v = codes.view(torch.float8_e4m3fn).to(torch.float32)
    fin = torch.isfinite(v)
    assert int(fin.sum()) == 254                               # S.1111.111 is NaN, for both signs
    f = v[fin]
    assert torch.equal(f.to(torch.float16).to(torch.float32), f)
    assert torch.equal(f.to(torch.bfloat16).to(torch.float32), f)
