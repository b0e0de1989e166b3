"""Pins of the float64 oracle against things other than itself.

Each check here ties the oracle to a fact fixed by the pages or by mathematics:
the bfloat16 format, exact rational arithmetic for the quantizer, brute force
in pure Python on tiny inputs, closed forms, a library routine
(``scaled_dot_product_attention`` in float64 on CPU), and the invariants the
course README states in its section "The code asserts its own claims" (s05,
s06, s11, s12). ``test_oracle_mutants.py`` plants mistakes in the oracle and
checks that these pins catch them.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import BF16, F32, FP8, I8, OraclePool
from workloads import f32_to_bf16_bits, make_step, tiny_decode

# --------------------------------------------------------------------------
# helpers: build an oracle pool from a generated step (prefix + new rows)
# --------------------------------------------------------------------------


def oracle_pool(step, with_new=True):
    pool = OraclePool(step.num_blocks, step.num_kv_heads, step.block_size, step.head_dim, step.kv_dtype)
    oracle.reshape_and_cache(pool, step.prefix_k, step.prefix_v, step.src_dtype, step.prefix_slots)
    if with_new:
        oracle.reshape_and_cache(pool, step.new_k, step.new_v, step.src_dtype, step.new_slots)
    return pool


def q64(step):
    return oracle.decode_rows(step.q, step.q_dtype)


# --------------------------------------------------------------------------
# pin helpers, reused by the mutant tests
# --------------------------------------------------------------------------


def brute_force_rows(q, K, V, scale, positions):
    """Pure-Python softmax attention (math.exp, math.fsum), GQA by contiguous
    groups written out as an explicit head loop with integer division."""
    L, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(K[0])
    g = Hq // Hkv
    s32 = float(np.float32(scale))
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(L)]
    lse = [[-math.inf] * Hq for _ in range(L)]
    for r in range(L):
        for h in range(Hq):
            kh = h // g
            keys = range(0, positions[r] + 1)
            sc = [s32 * math.fsum(q[r][h][d] * K[t][kh][d] for d in range(D)) for t in keys]
            if not sc:
                continue
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            den = math.fsum(w)
            for d in range(D):
                out[r][h][d] = math.fsum(w[i] * V[t][kh][d] for i, t in enumerate(keys)) / den
            lse[r][h] = m + math.log(den)
    return np.array(out), np.array(lse)


def check_brute_force(seed=3, L=3, n=7, Hq=4, Hkv=2, D=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, Hq, D))
    K = rng.standard_normal((n, Hkv, D))
    V = rng.standard_normal((n, Hkv, D))
    pos = n - L + np.arange(L)
    scale = 0.37
    o, l = oracle.attend_direct(q, K, V, scale, pos)
    ob, lb = brute_force_rows(q.tolist(), K.tolist(), V.tolist(), scale, pos.tolist())
    np.testing.assert_allclose(o, ob, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l, lb, rtol=1e-13, atol=1e-14)


def sdpa_reference(q, K, V, scale, positions):
    """torch scaled_dot_product_attention, float64 on CPU, KV heads repeated to
    the query heads and an explicit boolean mask ``t <= position``."""
    import torch
    Hq = q.shape[1]
    Hkv = K.shape[1]
    g = Hq // Hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))          # [Hq][L][D]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2))).repeat_interleave(g, 0)
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2))).repeat_interleave(g, 0)
    mask = torch.from_numpy(np.arange(K.shape[0])[None, :] <= np.asarray(positions)[:, None])
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=float(np.float32(scale)))
    return o.numpy().transpose(1, 0, 2)


def check_sdpa_chunked(seed=11):
    """Chunked + decode rows through the paged oracle vs SDPA on the contiguous KV."""
    step = make_step("sdpa", [37, 50, 23, 64], [1, 9, 23, 1], num_q_heads=8, num_kv_heads=2,
                     head_dim=32, q_dtype=F32, kv_dtype=F32, seed=seed, num_blocks=30)
    pool = oracle_pool(step)
    cu = step.cu_q_lens
    out, _ = oracle.paged_chunked(q64(step), cu, pool, step.block_tables, step.context_lens, step.scale)
    for i in range(len(step.context_lens)):
        K, V = (oracle.decode_rows(x, F32) for x in step.kv_contiguous(i))
        n, L = int(step.context_lens[i]), int(step.q_lens[i])
        ref = sdpa_reference(q64(step)[cu[i]:cu[i + 1]], K, V, step.scale, n - L + np.arange(L))
        np.testing.assert_allclose(out[cu[i]:cu[i + 1]], ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# value decoding
# --------------------------------------------------------------------------


def test_bf16_decoding_matches_format():
    """bfloat16 = sign | 8-bit exponent (bias 127) | 7 fraction bits."""
    bits = np.array([0x3F80, 0xC000, 0x3FC0, 0x0001, 0x8000, 0x7F80, 0x4049, 0x3E00], np.uint16)
    want = [1.0, -2.0, 1.5, 2.0 ** -133, -0.0, math.inf, 3.140625, 0.125]
    got = oracle.bf16_bits_to_f64(bits)
    assert got.tolist() == want
    assert math.copysign(1.0, got[4]) == -1.0


def test_int8_decoding_is_code_times_scale():
    codes = np.array([[[-127, 0, 5, 127]]], np.int8)
    scale = np.array([[0.25]], np.float32)
    assert oracle.decode_rows(codes, I8, scale).tolist() == [[[-31.75, 0.0, 1.25, 31.75]]]


def test_generator_bf16_rounding_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties to the even (1.0)
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6 (even)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -1.0], np.float32)
    got = oracle.bf16_bits_to_f64(f32_to_bf16_bits(x)).tolist()
    assert got == [1.0, 1 + 2 ** -6, 1 + 2 ** -7, -1.0]


# --------------------------------------------------------------------------
# int8 quantizer
# --------------------------------------------------------------------------


def _f32_round(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) float32 of an exact rational."""
    approx = np.float32(float(fr))
    lo = approx if Fraction(float(approx)) <= fr else np.nextafter(approx, np.float32(-np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    dlo, dhi = fr - Fraction(float(lo)), Fraction(float(hi)) - fr
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi
    return lo if (lo.view(np.uint32) & 1) == 0 else hi


def _round_half_even(fr: Fraction) -> int:
    f = math.floor(fr)
    rem = fr - f
    if rem > Fraction(1, 2):
        return f + 1
    if rem < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def test_quantizer_against_exact_rational_arithmetic():
    """scale = fl32(amax/127); code = clamp(round_half_even(fl32(x/scale)), +-127),
    recomputed with exact fractions and explicit float32 rounding."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 16)) * rng.choice([1e-3, 1.0, 300.0], size=(40, 1))).astype(np.float32)
    codes, scale = oracle.quantize_rows_int8(x)
    for r in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in x[r])
        sc = _f32_round(amax / 127)
        assert scale[r] == sc
        for c in range(x.shape[1]):
            quot = _f32_round(Fraction(float(x[r, c])) / Fraction(float(sc)))
            want = max(-127, min(127, _round_half_even(Fraction(float(quot)))))
            assert int(codes[r, c]) == want


def test_quantizer_near_half_way_quotients():
    """Quotients placed within a few ulps of k + 1/2, where a float32 division
    and a multiplication by a rounded reciprocal can land on different sides:
    the codes must follow the correctly rounded division (exact rationals)."""
    rng = np.random.default_rng(7)
    rows = []
    for _ in range(64):
        s = np.float32(1.0 + rng.integers(1, 1 << 10) / 1024.0) * np.float32(2.0 ** rng.integers(-8, 4))
        k = rng.integers(-126, 126, size=31)
        x = ((k + 0.5) * np.float64(s)).astype(np.float32)
        x = np.nextafter(x, x + np.sign(x) * rng.integers(-3, 4, size=31)).astype(np.float32)
        rows.append(np.concatenate([[np.float32(127.0) * s], x]))   # amax 127 s -> scale s exactly
    x = np.array(rows, np.float32)
    codes, scale = oracle.quantize_rows_int8(x)
    for r in range(x.shape[0]):
        sc = Fraction(float(scale[r]))
        assert sc == Fraction(float(x[r, 0])) / 127
        for c in range(x.shape[1]):
            quot = _f32_round(Fraction(float(x[r, c])) / sc)
            assert int(codes[r, c]) == max(-127, min(127, _round_half_even(Fraction(float(quot)))))


def test_quantizer_bounds_and_special_cases():
    rng = np.random.default_rng(6)
    x = f32_to_bf16_bits(rng.standard_normal((500, 128), dtype=np.float32))
    x32 = oracle.bf16_bits_to_f64(x).astype(np.float32)
    codes, scale = oracle.quantize_rows_int8(x32)
    assert codes.min() >= -127 and codes.max() <= 127
    err = np.abs(x32.astype(np.float64) - codes.astype(np.float64) * scale[:, None].astype(np.float64))
    # |x/scale| <= 127 (1 + 2^-23), so the float32 quotient is off by at most
    # 2^-24 * 128 = 2^-17 before rounding to an integer moves it by <= 1/2
    assert (err <= (0.5 + 2.0 ** -17) * scale[:, None].astype(np.float64)).all()
    # the element of largest magnitude maps to +-127 with its sign
    j = np.argmax(np.abs(x32), axis=1)
    assert (np.abs(codes[np.arange(500), j]) == 127).all()
    assert (np.sign(codes[np.arange(500), j]) == np.sign(x32[np.arange(500), j])).all()
    # all-zero row -> scale 1, codes 0
    c0, s0 = oracle.quantize_rows_int8(np.zeros((1, 8), np.float32))
    assert s0[0] == 1.0 and (c0 == 0).all()
    # ties go to even: amax 127 -> scale exactly 1
    c1, s1 = oracle.quantize_rows_int8(np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -2.5, -3.5, 126.5]], np.float32))
    assert s1[0] == 1.0
    assert c1[0].tolist() == [127, 0, 2, 2, 0, -2, -4, 126]


# --------------------------------------------------------------------------
# fp8 (OCP E4M3) decoding and quantizer
# --------------------------------------------------------------------------

# E4M3 values worked out by hand from the format: sign | exponent (4 bits,
# bias 7) | mantissa (3 bits); exponent 0 -> m * 2^-9.
FP8_WORKED = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
              0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x1D: 0.1015625, 0x77: 240.0, 0x7E: 448.0,
              0xB8: -1.0, 0xC4: -3.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}


def test_fp8_decoding_matches_format():
    v = oracle.fp8_e4m3_value(np.arange(256))
    for c, want in FP8_WORKED.items():
        assert v[c] == want, hex(c)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and int(np.isnan(v).sum()) == 2
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) == -1.0
    assert (np.diff(v[:0x7F]) > 0).all()                        # codes 0 .. 0x7E increase
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])              # the sign bit negates
    # spacing: 2^-9 below 2^-6 (subnormals and the first binade), then 2^(e-10)
    assert np.allclose(np.diff(v[:0x10]), 2.0 ** -9)


def test_fp8_decoding_matches_library():
    """torch's float8_e4m3fn (the same OCP format) decodes all 256 codes alike."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.fp8_e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    fin = ~np.isnan(ours)
    assert np.array_equal(lib[fin], ours[fin]) and np.array_equal(np.signbit(lib[fin]), np.signbit(ours[fin]))


def _fp8_codes_with_unit_scale(x: np.ndarray) -> np.ndarray:
    """Quantize values with |x| <= 448 through rows led by 448 (scale exactly 1)."""
    rows = np.concatenate([np.full((len(x), 1), 448.0, np.float32), np.asarray(x, np.float32)[:, None]], axis=1)
    codes, scale = oracle.quantize_rows_fp8(rows)
    assert (scale == 1.0).all()
    return codes[:, 1]


def test_fp8_encoder_matches_library_rounding():
    """torch rounds float32 to float8_e4m3fn to nearest, ties to even: on every
    value of magnitude <= 448 the oracle's table search must give its codes,
    including exact midpoints between neighbours and the float32 values next to
    them."""
    import torch
    rng = np.random.default_rng(12)
    mags = np.exp2(rng.uniform(-13, np.log2(448.0), 20000))
    x = (mags * rng.choice([-1.0, 1.0], 20000)).astype(np.float32)
    pos = oracle.fp8_e4m3_value(np.arange(0x7F))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)        # exact in float32
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    x = np.concatenate([x, near, -near, [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(_fp8_codes_with_unit_scale(x), lib)


def test_fp8_quantizer_bounds_and_special_cases():
    rng = np.random.default_rng(13)
    x = f32_to_bf16_bits(rng.standard_normal((500, 128), dtype=np.float32))
    x32 = oracle.bf16_bits_to_f64(x).astype(np.float32)
    codes, scale = oracle.quantize_rows_fp8(x32)
    assert not np.isnan(oracle.fp8_e4m3_value(codes)).any()
    y = x32.astype(np.float64) / scale[:, None].astype(np.float64)      # exact quotient
    err = np.abs(y - oracle.fp8_e4m3_value(codes))
    # half a step of the format (relative 2^-4 from 2^-6 up, absolute 2^-10 below),
    # plus the float32 rounding of the quotient (2^-24 relative)
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 2.0 ** -20)
    assert (err <= bound).all()
    # the element of largest magnitude maps to +-448 with its sign
    j = np.argmax(np.abs(x32), axis=1)
    r = np.arange(500)
    assert (codes[r, j] & 0x7F == 0x7E).all()
    assert ((codes[r, j] >> 7) == (x32[r, j] < 0)).all()
    # all-zero row -> scale 1, codes 0
    c0, s0 = oracle.quantize_rows_fp8(np.zeros((1, 8), np.float32))
    assert s0[0] == 1.0 and (c0 == 0).all()
    # worked values at scale 1: 0.1 -> 1.625 * 2^-4 (0x1D); 2^-10 ties to 0; 3 * 2^-11
    # -> 2^-9; 432 (between 416 and 448) ties to the even code 0x7E
    got = _fp8_codes_with_unit_scale(np.array([0.1, 2.0 ** -10, 3 * 2.0 ** -11, 432.0, -432.0, 1.0], np.float32))
    assert got.tolist() == [0x1D, 0x00, 0x01, 0x7E, 0xFE, 0x38]


def test_fp8_scatter_stores_quantized_rows():
    step = make_step("f8", [20, 33], [4, 1], num_q_heads=4, num_kv_heads=2, head_dim=16,
                     q_dtype=BF16, kv_dtype=FP8, src_dtype=BF16, seed=14)
    pool = oracle_pool(step)
    for i, n in enumerate(step.context_lens):
        K, V = oracle.gather_kv(pool, step.block_tables[i], int(n))
        Kc, Vc = (oracle.decode_rows(x, BF16) for x in step.kv_contiguous(i))
        kc, ks = oracle.quantize_rows_fp8(Kc.astype(np.float32))
        assert np.array_equal(K, oracle.fp8_e4m3_value(kc) * ks.astype(np.float64)[..., None])
        # dequantized rows are within half a step of the source
        tol = np.maximum(np.abs(Vc) * 2.0 ** -4, 2.0 ** -10 * np.abs(Vc).max(axis=-1, keepdims=True) / 448)
        assert (np.abs(V - Vc) <= tol * (1 + 2.0 ** -16)).all()


# --------------------------------------------------------------------------
# scatter / gather (claims s06 and s11)
# --------------------------------------------------------------------------


@pytest.mark.parametrize("kv_dtype", [F32, BF16])
def test_gather_of_scatter_is_identity(kv_dtype):
    step = make_step("rt", [5, 17, 40, 16, 1], [1, 1, 1, 1, 1], num_q_heads=4, num_kv_heads=2,
                     head_dim=64, q_dtype=kv_dtype, kv_dtype=kv_dtype, seed=2, num_blocks=12)
    pool = oracle_pool(step)
    for i, n in enumerate(step.context_lens):
        K, V = oracle.gather_kv(pool, step.block_tables[i], int(n))
        Kc, Vc = (oracle.decode_rows(x, kv_dtype) for x in step.kv_contiguous(i))
        assert np.array_equal(K, Kc) and np.array_equal(V, Vc)
    # exactly the written slots hold numbers; every other row is NaN
    written = np.zeros(pool.num_slots, bool)
    written[np.concatenate([step.prefix_slots, step.new_slots])] = True
    dk = oracle.decode_rows(pool.k, kv_dtype).transpose(0, 2, 1, 3).reshape(pool.num_slots, -1)
    assert np.isfinite(dk[written]).all() and np.isnan(dk[~written]).all()


def test_int8_scatter_stores_quantized_rows():
    step = make_step("q8", [20, 33], [4, 1], num_q_heads=4, num_kv_heads=2, head_dim=16,
                     q_dtype=BF16, kv_dtype=I8, src_dtype=BF16, seed=8)
    pool = oracle_pool(step)
    for i, n in enumerate(step.context_lens):
        K, V = oracle.gather_kv(pool, step.block_tables[i], int(n))
        Kc, Vc = (oracle.decode_rows(x, BF16) for x in step.kv_contiguous(i))
        kc, ks = oracle.quantize_rows_int8(Kc.astype(np.float32))
        assert np.array_equal(K, kc.astype(np.float64) * ks.astype(np.float64)[..., None])
        # dequantized rows are within half a step of the source
        assert (np.abs(K - Kc) <= (0.5 + 2.0 ** -17) * ks[..., None]).all()
        vs = np.abs(Vc).max(axis=-1, keepdims=True) / 127
        assert (np.abs(V - Vc) <= (0.5 + 2.0 ** -16) * vs).all()


@pytest.mark.parametrize("kv_dtype", [BF16, I8, FP8])
def test_piecewise_chunk_writes_equal_one_shot(kv_dtype):
    """Claim s11: writing a chunk's K/V in pieces yields a bit-identical cache."""
    step = make_step("pieces", [300, 77], [300, 77], num_q_heads=4, num_kv_heads=2, head_dim=32,
                     q_dtype=BF16, kv_dtype=kv_dtype, seed=9, num_blocks=40)
    one = oracle_pool(step)
    piece = OraclePool(step.num_blocks, 2, 16, 32, kv_dtype)
    rng = np.random.default_rng(0)
    cuts = np.sort(rng.choice(np.arange(1, len(step.new_slots)), 6, replace=False))
    for a, e in zip(np.r_[0, cuts], np.r_[cuts, len(step.new_slots)]):
        oracle.reshape_and_cache(piece, step.new_k[a:e], step.new_v[a:e], step.src_dtype, step.new_slots[a:e])
    for name in ("k", "v", "k_scale", "v_scale"):
        a, b = getattr(one, name), getattr(piece, name)
        if a is not None:
            assert a.tobytes() == b.tobytes(), name


def test_negative_slots_are_skipped_and_bad_slots_raise():
    pool = OraclePool(2, 1, 4, 2, F32)
    k = np.arange(6, dtype=np.float32).reshape(3, 1, 2)
    oracle.reshape_and_cache(pool, k, k, F32, np.array([-1, 5, -7]))
    assert pool.k[1, 0, 1].tolist() == [2.0, 3.0]
    assert int(np.isfinite(pool.k).sum()) == 2
    with pytest.raises(AssertionError):
        oracle.reshape_and_cache(pool, k, k, F32, np.array([1, 1, 2]))
    with pytest.raises(AssertionError):
        oracle.reshape_and_cache(pool, k, k, F32, np.array([0, 1, 8]))
    with pytest.raises(AssertionError):
        oracle.gather_kv(pool, np.array([0, 2]), 5)       # block id 2 of a 2-block pool
    with pytest.raises(AssertionError):
        oracle.gather_kv(pool, np.array([0]), 5)          # 5 tokens in one 4-slot block


@pytest.mark.parametrize("kv_dtype", [F32, I8, FP8])
def test_output_invariant_under_block_placement(kv_dtype):
    """Claim s06: the result does not depend on where blocks sit in the pool."""
    kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=32, q_dtype=F32 if kv_dtype == F32 else BF16,
              kv_dtype=kv_dtype, num_blocks=20)
    a = make_step("pa", [45, 19, 64], [1, 1, 1], seed=4, **kw)
    pa = oracle_pool(a)
    oa, la = oracle.paged_decode(q64(a), pa, a.block_tables, a.context_lens, a.scale)
    # same values, another placement: move every block through a fixed permutation
    perm = np.random.default_rng(99).permutation(a.num_blocks)
    pb = OraclePool(a.num_blocks, 2, 16, 32, kv_dtype)
    for name in ("k", "v", "k_scale", "v_scale"):
        if getattr(pa, name) is not None:
            arr = getattr(pb, name)
            arr[perm] = getattr(pa, name)
    tb = np.where(a.block_tables >= 0, perm[np.maximum(a.block_tables, 0)], -1)
    ob, lb = oracle.paged_decode(q64(a), pb, tb, a.context_lens, a.scale)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------


def test_direct_matches_brute_force():
    check_brute_force()
    check_brute_force(seed=4, L=1, n=1, Hq=2, Hkv=2, D=3)
    check_brute_force(seed=5, L=4, n=4, Hq=6, Hkv=3, D=2)


def test_paged_matches_library_sdpa_on_contiguous_kv():
    check_sdpa_chunked()


def test_tiny_decode_config_against_sdpa():
    step = tiny_decode()
    pool = oracle_pool(step)
    out, lse = oracle.paged_decode(q64(step), pool, step.block_tables, step.context_lens, step.scale)
    for i, n in enumerate(step.context_lens):
        K, V = (oracle.decode_rows(x, F32) for x in step.kv_contiguous(i))
        ref = sdpa_reference(q64(step)[i:i + 1], K, V, step.scale, [int(n) - 1])
        np.testing.assert_allclose(out[i:i + 1], ref, rtol=1e-12, atol=1e-13)
        # lse = log sum_t exp(s_t), against numpy's logaddexp reduction
        for h in range(step.num_q_heads):
            s = float(step.scale) * (K[:, h // 2, :] @ q64(step)[i, h])
            assert abs(lse[i, h] - np.logaddexp.reduce(s)) <= 1e-13 * max(1.0, abs(lse[i, h]))


def test_closed_forms():
    rng = np.random.default_rng(12)
    V = rng.standard_normal((9, 2, 6))
    K = rng.standard_normal((9, 2, 6))
    # one key: the output is that key's value, exactly
    o, l = oracle.attend_direct(rng.standard_normal((1, 4, 6)), K[:1], V[:1], 0.5, [0])
    assert np.array_equal(o[0, :2], np.repeat(V[0, :1], 2, 0)) and np.array_equal(o[0, 2:], np.repeat(V[0, 1:], 2, 0))
    # zero query: uniform weights -> the mean of the values; lse = log n
    o, l = oracle.attend_direct(np.zeros((1, 2, 6)), K, V, 0.5, [8])
    np.testing.assert_allclose(o[0], V.mean(axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(l[0], math.log(9), rtol=0, atol=1e-15)
    # all keys equal: uniform weights as well
    Ke = np.repeat(K[:1], 9, 0)
    o, _ = oracle.attend_direct(rng.standard_normal((1, 2, 6)), Ke, V, 0.5, [8])
    np.testing.assert_allclose(o[0], V.mean(axis=0), rtol=0, atol=1e-15)
    # causal: a row at position p ignores keys after p, whatever they hold
    Kn, Vn = K.copy(), V.copy()
    Kn[5:], Vn[5:] = np.nan, np.nan
    q = rng.standard_normal((1, 2, 6))
    o1, _ = oracle.attend_direct(q, Kn, Vn, 0.5, [4])
    o2, _ = oracle.attend_direct(q, K[:5], V[:5], 0.5, [4])
    assert np.array_equal(o1, o2)
    # no key at all: zero output, -inf lse
    o, l = oracle.attend_direct(q, K[:0], V[:0], 0.5, [-1])
    assert (o == 0).all() and (l == -np.inf).all()


def test_one_hot_key_selects_its_value_exactly():
    """A key much closer to q than all others takes all the weight: every other
    exp underflows to 0 and the output is that key's value bit for bit."""
    rng = np.random.default_rng(13)
    D, n = 16, 33
    q = rng.standard_normal((1, 1, D))
    K = np.zeros((n, 1, D))
    V = rng.standard_normal((n, 1, D))
    for j in (0, 7, 32):
        Kj = K.copy()
        Kj[j, 0] = q[0, 0] * (2000.0 / float(q[0, 0] @ q[0, 0]))
        o, _ = oracle.attend_direct(q, Kj, V, 1.0, [n - 1])
        assert np.array_equal(o[0, 0], V[j, 0])


def test_decode_equals_last_row_of_full_causal_attention():
    """Claim s05 analogue: attending the cached history with the last token's q
    equals the last row of attention over the whole sequence at once."""
    n = 41
    dec = make_step("d", [n], [1], num_q_heads=4, num_kv_heads=1, head_dim=8, q_dtype=F32, kv_dtype=F32, seed=21)
    full = make_step("f", [n], [n], num_q_heads=4, num_kv_heads=1, head_dim=8, q_dtype=F32, kv_dtype=F32, seed=21)
    # the two steps share K/V (same child stream); use the full step's last q row for both
    assert np.array_equal(dec.kv_contiguous(0)[0], full.kv_contiguous(0)[0])
    pf = oracle_pool(full)
    of, lf = oracle.paged_chunked(q64(full), full.cu_q_lens, pf, full.block_tables, full.context_lens, full.scale)
    pd = oracle_pool(dec)
    od, ld = oracle.paged_decode(q64(full)[-1:], pd, dec.block_tables, dec.context_lens, dec.scale)
    np.testing.assert_allclose(od[0], of[-1], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(ld[0], lf[-1], rtol=1e-14, atol=1e-15)


def test_chunk_row_equals_decode_at_its_position():
    step = make_step("c", [70], [20], num_q_heads=4, num_kv_heads=2, head_dim=16, q_dtype=F32,
                     kv_dtype=F32, seed=22)
    pool = oracle_pool(step)
    oc, _ = oracle.paged_chunked(q64(step), step.cu_q_lens, pool, step.block_tables, step.context_lens, step.scale)
    for r in (0, 7, 19):
        p = 70 - 20 + r
        od, _ = oracle.paged_decode(q64(step)[r:r + 1], pool, step.block_tables, np.array([p + 1]), step.scale)
        np.testing.assert_allclose(od[0], oc[r], rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------------------
# online softmax and split-K (claim s12: exact; agree to 1e-15)
# --------------------------------------------------------------------------


@pytest.mark.parametrize("n", [1, 15, 16, 17, 40, 129])
def test_online_and_split_k_agree_with_direct(n):
    rng = np.random.default_rng(n)
    D = 32
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    scale = float(np.float32(1 / math.sqrt(D)))
    od, ld = oracle.attend_direct(q[None, None], K[:, None], V[:, None], scale, [n - 1])
    oo, lo = oracle.online_softmax_attend(q, K, V, scale)
    assert np.abs(oo - od[0, 0]).max() <= 1e-15 and abs(lo - ld[0, 0]) <= 1e-15 * max(1, abs(ld[0, 0]))
    for ns in range(1, -(-n // 16) + 3):
        os_, ls = oracle.split_k_decode(q, K, V, scale, ns)
        assert np.abs(os_ - od[0, 0]).max() <= 1e-15, ns
        assert abs(ls - ld[0, 0]) <= 2e-15 * max(1, abs(ld[0, 0])), ns


def test_online_softmax_rescales_when_the_max_grows():
    """Scores that grow along the sequence move the running max at every block,
    so each block must rescale what was accumulated before it."""
    rng = np.random.default_rng(31)
    D, n = 8, 70
    q = rng.standard_normal(D)
    K = np.outer(np.linspace(-3.0, 3.0, n), q) / float(q @ q)
    V = rng.standard_normal((n, D))
    od, ld = oracle.attend_direct(q[None, None], K[:, None], V[:, None], 1.0, [n - 1])
    oo, lo = oracle.online_softmax_attend(q, K, V, 1.0)
    assert np.abs(oo - od[0, 0]).max() <= 1e-15 and abs(lo - ld[0, 0]) <= 1e-15
    for ns in (2, 3, 5):
        os_, ls = oracle.split_k_decode(q, K, V, 1.0, ns)
        assert np.abs(os_ - od[0, 0]).max() <= 1e-15 and abs(ls - ld[0, 0]) <= 2e-15


def test_split_bounds_partition_the_context():
    for n in (1, 5, 16, 17, 40, 511, 512, 513, 8192):
        for ns in (1, 2, 3, 7, 16, 64):
            b = oracle.split_bounds(n, ns, 16)
            assert len(b) == ns and b[0][0] == 0 and b[-1][1] == n
            assert all(b[i][1] == b[i + 1][0] for i in range(ns - 1))
            assert all(a % 16 == 0 or a == n for a, _ in b)
            assert max(e - a for a, e in b) <= 16 * -(-(-(-n // ns)) // 16)


def test_lse_combine_ignores_empty_splits():
    o = np.array([[1.0, 2.0], [5.0, 5.0], [3.0, -1.0]])
    l = np.array([0.5, -np.inf, 0.5])
    out, lse = oracle.lse_combine(o, l)
    assert out.tolist() == [2.0, 0.5] and abs(lse - (0.5 + math.log(2))) < 1e-15
    out, lse = oracle.lse_combine(o[:1] * np.nan, np.array([-np.inf]))
    assert (out == 0).all() and lse == -np.inf
