"""Float64 NumPy oracle: scatter, gather, direct softmax attention, int8 and fp8 quantizers.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the
product path.

Sources on the pages, cited by page title and section:

* Page "S20 · The Complete Engine" (course chapter), section "Core idea":
  step 2 (MEMORY) gives every request a ``block_table``, a list of physical
  block ids from a shared pool. The pool is a set of fixed-size blocks.
* Page "llm-inference" (work-log on shehab-ashraf.github.io), section
  "KV Cache", subsection "The Idea": a decode step computes one new q, k, v,
  appends the new k, v to the cache, and the single q attends over the whole
  history. Hence ``context_len`` counts the new token, and the new K/V are
  written (``reshape_and_cache``) before attention reads them.
* Course README "Build an LLM Inference Engine From Scratch", section "The
  curriculum": S03 names grouped-query attention (GQA); S06 PagedAttention;
  S08 quantization (notation ``q = round(w / scale) + zero`` in section
  "Translating", conventions paragraph); S11 chunked prefill; S12
  FlashAttention (online softmax, split-K).
* Same README, section "The code asserts its own claims": s05 cached and
  uncached generation agree; s06 paged attention equals contiguous attention;
  s11 chunked prefill yields a bit-identical KV cache; s12 online softmax is
  exact and the paged and split-K variants agree.

Readings taken where the pages are silent (each one is listed, with its
reason, in the design notes of the repository):

* GQA: query head ``h`` reads KV head ``h // (Hq // Hkv)`` (contiguous groups).
* Chunked rows are bottom-right aligned: row ``r`` of a length-``L`` chunk of a
  sequence whose cache now holds ``n`` tokens sits at position ``n - L + r``
  and attends keys ``t <= n - L + r``.
* INT8 KV is symmetric per (token, KV head) with zero point 0:
  ``scale = amax / 127`` in float32, ``code = clamp(rint(x / scale), -127, 127)``
  with an IEEE float32 division and round-half-to-even; ``amax == 0`` gives
  ``scale = 1``. The dequantized value is ``code * scale``.
* FP8 KV (the course README's curriculum, S00 "bf16/fp8" with S08
  quantization) is read as the OCP 8-bit floating-point format E4M3 (sign, 4
  exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the subnormals
  ``m * 2^-9``; ``S.1111.111`` is NaN; no infinities; largest finite 448),
  scaled like the int8 cache: per (token, KV head), ``scale = amax / 448`` in
  float32 (``amax == 0`` gives 1) and ``code`` = the E4M3 value nearest to the
  float32 quotient ``x / scale``, ties to the even code, saturating at 448. The
  dequantized value is ``value(code) * scale``.
* Split-K uses block-aligned contiguous ranges:
  ``tps = bs * ceil(ceil(n / ns) / bs)``, split ``s`` covers
  ``[s * tps, min(n, (s + 1) * tps))``; an empty split yields
  ``(o = 0, lse = -inf)`` and carries no weight in the merge.
* Outputs are float32-representable values computed in float64; ``lse`` is the
  natural log of the softmax denominator plus the row max.

Layouts (the same as the library's public header states):
``k, v : [num_blocks][Hkv][block_size][D]`` in the storage dtype;
``k_scale, v_scale : [num_blocks][Hkv][block_size]`` float32 (int8 and fp8 only);
``block_tables : int32 [B][max_blocks]`` (``-1`` past the used entries);
``slot_mapping : int64 [T]``, slot ``s`` is block ``s // bs``, offset ``s % bs``;
a negative slot means "skip this row".
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F32 = "f32"
BF16 = "bf16"
I8 = "i8"
FP8 = "fp8"

# A quiet NaN in bfloat16 storage: unused pool rows are filled with it so that a
# stray read shows up as NaN in the output.
NAN_BF16_BITS = np.uint16(0x7FC0)

_STORAGE = {F32: np.float32, BF16: np.uint16, I8: np.int8, FP8: np.uint8}

# An E4M3 NaN code: unused fp8 pool rows hold it (and NaN scales).
NAN_FP8_CODE = np.uint8(0x7F)


# --------------------------------------------------------------------------
# value decoding (storage -> float64), all exact
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the top half of an IEEE binary32: sign, 8-bit exponent and
    the 7 leading fraction bits. Shifting the 16 stored bits up by 16 gives the
    binary32 with the same value, which widens exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp8_e4m3_value(code) -> np.ndarray:
    """Value of OCP E4M3 codes, float64: sign bit 7, exponent bits 6..3 (bias
    7), mantissa bits 2..0. Exponent 0 holds the subnormals ``m * 2^-9``; a
    nonzero exponent gives ``(1 + m / 8) * 2^(e - 7)``; ``S.1111.111`` is NaN
    and there are no infinities."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.power(2.0, e - 7))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


# the finite non-negative E4M3 values, codes 0x00 .. 0x7E, in increasing order
_FP8_POSITIVE = fp8_e4m3_value(np.arange(0x7F))


def decode_rows(raw: np.ndarray, dtype: str, scale: np.ndarray | None = None) -> np.ndarray:
    """Storage values -> float64.

    int8 and fp8 rows are dequantized as ``value(code) * scale`` with the
    per-(token, head) float32 scale broadcast over the last (head_dim) axis. The
    product of an 8-bit integer (or an E4M3 value) and a float32 needs at most
    24 + 7 significant bits, so it is exact in float64.
    """
    if dtype == F32:
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(raw)
    if dtype == I8:
        assert scale is not None, "int8 rows need their scales"
        return np.asarray(raw, np.int8).astype(np.float64) * np.asarray(scale, np.float32).astype(np.float64)[..., None]
    if dtype == FP8:
        # an E4M3 value has at most 4 significant bits: its product with a
        # float32 scale is exact in float64
        assert scale is not None, "fp8 rows need their scales"
        return fp8_e4m3_value(raw) * np.asarray(scale, np.float32).astype(np.float64)[..., None]
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# int8 quantizer (course README, curriculum S08 and the "q = round(w/scale) +
# zero" notation; symmetric per (token, head) reading, zero = 0)
# --------------------------------------------------------------------------

def quantize_rows_int8(x32: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize float32 rows (last axis = head_dim) to int8 codes + float32 scale.

    Every operation is a float32 NumPy operation: ``|x|`` and ``max`` are exact,
    ``amax / 127`` and ``x / scale`` are IEEE correctly-rounded float32
    divisions, and ``np.rint`` rounds half to even.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    safe = np.where(amax > np.float32(0.0), amax, np.float32(127.0)).astype(np.float32)
    scale = (safe / np.float32(127.0)).astype(np.float32)   # amax == 0 -> scale 1
    quot = (x32 / scale[..., None]).astype(np.float32)
    codes = np.clip(np.rint(quot), -127.0, 127.0).astype(np.int8)
    return codes, scale


def quantize_rows_fp8(x32: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize float32 rows (last axis = head_dim) to OCP E4M3 codes + float32
    scale: ``scale = amax / 448`` (IEEE float32 division; ``amax == 0`` gives
    1), then each float32 quotient ``x / scale`` takes the code of the nearest
    finite E4M3 value, found by search over the value table; an exact tie goes
    to the even code; quotients past 448 take 448. The sign bit is the
    quotient's."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    safe = np.where(amax > np.float32(0.0), amax, np.float32(448.0)).astype(np.float32)
    scale = (safe / np.float32(448.0)).astype(np.float32)   # amax == 0 -> scale 1
    y = (x32 / scale[..., None]).astype(np.float32)
    a = np.abs(y).astype(np.float64)                          # exact
    hi = np.minimum(np.searchsorted(_FP8_POSITIVE, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(a - _FP8_POSITIVE[lo])
    d_hi = np.abs(_FP8_POSITIVE[hi] - a)
    pick = np.where(d_hi < d_lo, hi, np.where(d_lo < d_hi, lo, np.where(hi % 2 == 0, hi, lo)))
    codes = (pick | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)
    return codes, scale


# --------------------------------------------------------------------------
# the block pool and the scatter ("reshape_and_cache")
# --------------------------------------------------------------------------

@dataclass
class OraclePool:
    """KV block pool in storage form. Unused rows hold NaN (or NaN scales)."""

    num_blocks: int
    num_kv_heads: int
    block_size: int
    head_dim: int
    kv_dtype: str
    k: np.ndarray = None
    v: np.ndarray = None
    k_scale: np.ndarray | None = None
    v_scale: np.ndarray | None = None

    def __post_init__(self):
        shape = (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)
        if self.kv_dtype == F32:
            self.k = np.full(shape, np.nan, np.float32)
            self.v = np.full(shape, np.nan, np.float32)
        elif self.kv_dtype == BF16:
            self.k = np.full(shape, NAN_BF16_BITS, np.uint16)
            self.v = np.full(shape, NAN_BF16_BITS, np.uint16)
        elif self.kv_dtype == I8:
            self.k = np.zeros(shape, np.int8)
            self.v = np.zeros(shape, np.int8)
            self.k_scale = np.full(shape[:3], np.nan, np.float32)
            self.v_scale = np.full(shape[:3], np.nan, np.float32)
        elif self.kv_dtype == FP8:
            self.k = np.full(shape, NAN_FP8_CODE, np.uint8)
            self.v = np.full(shape, NAN_FP8_CODE, np.uint8)
            self.k_scale = np.full(shape[:3], np.nan, np.float32)
            self.v_scale = np.full(shape[:3], np.nan, np.float32)
        else:
            raise ValueError(self.kv_dtype)

    @property
    def num_slots(self) -> int:
        return self.num_blocks * self.block_size


def reshape_and_cache(pool: OraclePool, k_new: np.ndarray, v_new: np.ndarray,
                      src_dtype: str, slot_mapping: np.ndarray) -> None:
    """Write new K/V rows ``[T][Hkv][D]`` into the pool at ``slot_mapping``.

    Append-then-attend (page "llm-inference", section "KV Cache"): the rows of
    the new tokens go into the cache before attention reads them. A negative
    slot skips its row. Float caches take the source bytes unchanged (the
    source dtype must match); the int8 and fp8 caches quantize each (token,
    head) row.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    T = slots.shape[0]
    assert k_new.shape == (T, pool.num_kv_heads, pool.head_dim) == v_new.shape
    live = np.nonzero(slots >= 0)[0]
    s = slots[live]
    if s.size:
        assert s.max() < pool.num_slots, "slot out of range"
        assert np.unique(s).size == s.size, "duplicate slots in one call"
    blk = s // pool.block_size
    off = s % pool.block_size
    if pool.kv_dtype in (F32, BF16):
        assert src_dtype == pool.kv_dtype, "float caches copy bytes: dtypes must match"
        store = _STORAGE[src_dtype]
        pool.k[blk, :, off, :] = np.asarray(k_new, store)[live]
        pool.v[blk, :, off, :] = np.asarray(v_new, store)[live]
    else:
        assert src_dtype in (F32, BF16)
        k32 = decode_rows(k_new, src_dtype).astype(np.float32)[live]  # exact: bf16 and f32 fit binary32
        v32 = decode_rows(v_new, src_dtype).astype(np.float32)[live]
        quantize = quantize_rows_int8 if pool.kv_dtype == I8 else quantize_rows_fp8
        kc, ks = quantize(k32)
        vc, vs = quantize(v32)
        pool.k[blk, :, off, :] = kc
        pool.v[blk, :, off, :] = vc
        pool.k_scale[blk, :, off] = ks
        pool.v_scale[blk, :, off] = vs


def gather_kv(pool: OraclePool, table_row: np.ndarray, n: int) -> tuple[np.ndarray, np.ndarray]:
    """Contiguous float64 K, V ``[n][Hkv][D]`` of one sequence.

    Logical token ``t`` lives in physical block ``table_row[t // bs]`` at offset
    ``t % bs`` (page "S20 · The Complete Engine", section "Core idea", the
    per-request ``block_table``).
    """
    t = np.arange(n)
    bs = pool.block_size
    assert n <= len(table_row) * bs, "context longer than its block table"
    blk = np.asarray(table_row, np.int64)[t // bs]
    off = t % bs
    assert ((blk >= 0) & (blk < pool.num_blocks)).all(), "block id out of range"
    # advanced indices on axes 0 and 2 -> result axes [n][Hkv][D]
    if pool.kv_dtype in (I8, FP8):
        K = decode_rows(pool.k[blk, :, off, :], pool.kv_dtype, pool.k_scale[blk, :, off])
        V = decode_rows(pool.v[blk, :, off, :], pool.kv_dtype, pool.v_scale[blk, :, off])
    else:
        K = decode_rows(pool.k[blk, :, off, :], pool.kv_dtype)
        V = decode_rows(pool.v[blk, :, off, :], pool.kv_dtype)
    return K, V


# --------------------------------------------------------------------------
# attention: the plain two-pass definition in float64
# --------------------------------------------------------------------------

def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """GQA (course README, curriculum S03): contiguous groups of
    ``Hq / Hkv`` query heads share one KV head."""
    return h // (num_q_heads // num_kv_heads)


def attend_direct(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                  positions: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """softmax(scale * q K^T) V for query rows at ``positions``, float64.

    ``q [L][Hq][D]``, ``K, V [n][Hkv][D]``; row ``r`` attends keys
    ``t <= positions[r]``. Two passes: row max, then exponentials, sum and the
    weighted sum of values. ``scale`` is taken as the float32 the GPU receives.
    Returns ``out [L][Hq][D]`` and ``lse [L][Hq]`` (natural log). A row with no
    key gives ``out = 0``, ``lse = -inf``.
    """
    q = np.asarray(q, np.float64)
    L, Hq, D = q.shape
    n, Hkv, _ = K.shape
    s64 = float(np.float32(scale))
    out = np.zeros((L, Hq, D), np.float64)
    lse = np.full((L, Hq), -np.inf, np.float64)
    for r in range(L):
        m_keys = max(0, min(n, int(positions[r]) + 1))     # keys t <= position, and t < n
        if m_keys == 0:
            continue
        for h in range(Hq):
            k = kv_head_of(h, Hq, Hkv)
            s = s64 * (K[:m_keys, k, :] @ q[r, h, :])      # [m_keys]
            m = s.max()
            w = np.exp(s - m)
            den = w.sum()
            out[r, h, :] = (w @ V[:m_keys, k, :]) / den
            lse[r, h] = m + math.log(den)
    return out, lse


def paged_decode(q: np.ndarray, pool: OraclePool, block_tables: np.ndarray,
                 context_lens: np.ndarray, scale: float,
                 rows: list[tuple[int, int]] | None = None):
    """Decode: one query row per sequence at position ``n_b - 1``.

    ``q [B][Hq][D]`` float64 values. Returns ``out [B][Hq][D]``, ``lse [B][Hq]``.
    With ``rows = [(b, h), ...]`` only those outputs are computed (the rest stay
    NaN) -- for checking large problems one output at a time.
    """
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    want = {}
    if rows is None:
        want = {b: list(range(Hq)) for b in range(B)}
    else:
        for b, h in rows:
            want.setdefault(b, []).append(h)
    for b, heads in want.items():
        n = int(context_lens[b])
        K, V = gather_kv(pool, block_tables[b], n)
        o, l = attend_direct(q[b:b + 1], K, V, scale, np.array([n - 1]))
        for h in heads:
            out[b, h] = o[0, h]
            lse[b, h] = l[0, h]
    return out, lse


def paged_chunked(q: np.ndarray, cu_q_lens: np.ndarray, pool: OraclePool,
                  block_tables: np.ndarray, context_lens: np.ndarray, scale: float):
    """Chunked prefill: sequence ``i`` has ``L_i = cu[i+1] - cu[i]`` new rows
    whose K/V are already in the cache; its cache holds ``n_i`` tokens, row
    ``r`` sits at ``n_i - L_i + r`` (bottom-right aligned causal mask).

    ``q [sum L][Hq][D]`` -> ``out [sum L][Hq][D]``, ``lse [sum L][Hq]``.
    """
    q = np.asarray(q, np.float64)
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for i in range(len(cu_q_lens) - 1):
        a, e = int(cu_q_lens[i]), int(cu_q_lens[i + 1])
        L, n = e - a, int(context_lens[i])
        if L == 0:
            continue
        assert L <= n, "a chunk cannot be longer than the cached context"
        K, V = gather_kv(pool, block_tables[i], n)
        o, l = attend_direct(q[a:e], K, V, scale, n - L + np.arange(L))
        out[a:e], lse[a:e] = o, l
    return out, lse


# --------------------------------------------------------------------------
# online softmax and split-K: the same quantity by the route the pages name
# (course README, curriculum S12; claim s12). Used only to check the oracle
# against itself and against the pages' claim, never for GPU parity.
# --------------------------------------------------------------------------

def online_softmax_attend(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                          block: int = 16) -> tuple[np.ndarray, float]:
    """One query row (``[D]``) against ``K, V [n][D]`` of one head, one key block
    at a time: keep the running max ``m``, the running denominator ``l`` and the
    running weighted sum ``acc``; when the max grows, rescale ``l`` and ``acc`` by
    ``exp(m_old - m_new)`` (the online normalizer). Returns ``(out, lse)``."""
    s64 = float(np.float32(scale))
    m, l = -np.inf, 0.0
    acc = np.zeros(V.shape[1])
    for t0 in range(0, K.shape[0], block):
        s = s64 * (K[t0:t0 + block] @ q_row)
        m_new = max(m, float(s.max()))
        corr = math.exp(m - m_new) if m != -np.inf else 0.0
        p = np.exp(s - m_new)
        l = l * corr + float(p.sum())
        acc = acc * corr + p @ V[t0:t0 + block]
        m = m_new
    if l == 0.0:
        return np.zeros(V.shape[1]), -np.inf
    return acc / l, m + math.log(l)


def split_bounds(n: int, num_splits: int, block_size: int) -> list[tuple[int, int]]:
    """Block-aligned contiguous split ranges (empty ranges kept as ``(a, a)``)."""
    per = -(-n // num_splits)                       # ceil(n / ns)
    tps = block_size * (-(-per // block_size))      # rounded up to whole blocks
    return [(min(n, s * tps), min(n, (s + 1) * tps)) for s in range(num_splits)]


def lse_combine(o_parts: np.ndarray, lse_parts: np.ndarray) -> tuple[np.ndarray, float]:
    """Merge partial results ``o_s`` (each already normalised by its own
    denominator) with their log-sum-exps: weights ``exp(lse_s - max lse)``.
    Splits with ``lse = -inf`` carry no weight. All empty -> ``(0, -inf)``."""
    lse_parts = np.asarray(lse_parts, np.float64)
    live = np.isfinite(lse_parts)
    if not live.any():
        return np.zeros(o_parts.shape[-1]), -np.inf
    M = lse_parts[live].max()
    w = np.where(live, np.exp(np.where(live, lse_parts, M) - M), 0.0)
    tot = w.sum()
    o = (w[:, None] * np.where(live[:, None], o_parts, 0.0)).sum(axis=0) / tot
    return o, M + math.log(tot)


def split_k_decode(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                   num_splits: int, block_size: int = 16) -> tuple[np.ndarray, float]:
    """Flash-decoding decomposition of one decode row: attend each split range
    separately (online softmax inside it), then merge with :func:`lse_combine`."""
    parts, lses = [], []
    for a, e in split_bounds(K.shape[0], num_splits, block_size):
        if e > a:
            o, l = online_softmax_attend(q_row, K[a:e], V[a:e], scale, block_size)
        else:
            o, l = np.zeros(V.shape[1]), -np.inf
        parts.append(o)
        lses.append(l)
    return lse_combine(np.array(parts), np.array(lses))
