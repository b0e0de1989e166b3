"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad host-side arguments before launching anything.
Every call here fails a host check, so no kernel is ever launched."""

from __future__ import annotations

import ctypes

import pytest

import paged_kv_attention_19_amd as pkv
from paged_kv_attention_19_amd import _Cache

FAKE = 0x10000  # never dereferenced: every call below fails a host check first


def cache(**kw):
    d = dict(num_blocks=8, block_size=16, num_kv_heads=2, head_dim=64, kv_dtype=pkv.BF16, k=FAKE, v=FAKE,
             k_scale=None, v_scale=None)
    d.update(kw)
    return _Cache(d["num_blocks"], d["block_size"], d["num_kv_heads"], d["head_dim"], d["kv_dtype"], d["k"], d["v"],
                  d["k_scale"], d["v_scale"])


def test_library_exports_every_header_function():
    L = pkv.lib()
    names = pkv.exported_symbols()
    assert {"pkv_reshape_and_cache", "pkv_paged_attention_decode", "pkv_paged_attention_decode_append",
            "pkv_paged_attention_chunked", "pkv_lse_combine", "pkv_decode_workspace_bytes", "pkv_last_error",
            "pkv_version", "pkv_decode_default_max_num_splits", "pkv_chunked_kernel_for"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in pkv.version()


def test_default_decode_mode_by_table_width():
    """One split per sequence up to 64-block (1024-token) tables, balanced
    past that; a width below 1 is an error."""
    assert [pkv.decode_default_max_num_splits(w) for w in (1, 24, 64, 65, 512, 2048)] == [1, 1, 1, 0, 0, 0]
    with pytest.raises(pkv.PkvError, match="max_blocks_per_seq=0"):
        pkv.decode_default_max_num_splits(0)


def test_chunked_kernel_by_rows_per_kv_head():
    """R = max_q_len x GQA group rows per kv head: the decode core up to 2
    (head_dim 128) or 4 (head_dim 64), the 16x16 MFMA kernel up to 16 (head_dim
    128 only), the 128-row kernel past that; rejected shapes are errors."""
    D_ROWS, M_ROWS, TILES = pkv.CHUNKED_DECODE_ROWS, pkv.CHUNKED_ROWS_MFMA, pkv.CHUNKED_TILES

    def path(L, hq, hkv, d):
        return pkv.chunked_kernel_for(L, hq, hkv, d)

    assert [path(L, 8, 8, 128) for L in (1, 2, 3, 4, 16, 17, 512)] == [D_ROWS, D_ROWS] + [M_ROWS] * 3 + [TILES] * 2
    assert [path(L, 16, 8, 128) for L in (1, 2, 8, 9)] == [D_ROWS, M_ROWS, M_ROWS, TILES]
    assert [path(1, 8 * g, 8, 128) for g in (1, 2, 4, 8)] == [D_ROWS, D_ROWS, M_ROWS, M_ROWS]
    assert [path(2, 16, 2, 128), path(3, 16, 2, 128)] == [M_ROWS, TILES]      # group 8: 16 and 24 rows
    assert [path(L, 8, 8, 64) for L in (1, 2, 3, 4, 5, 16, 17)] == [D_ROWS] * 4 + [TILES] * 3
    assert [path(1, 8 * g, 8, 64) for g in (1, 2, 4, 8)] == [D_ROWS, D_ROWS, D_ROWS, TILES]
    for args, msg in [((0, 8, 8, 128), "max_q_len=0"), ((1, 8, 0, 128), "num_kv_heads=0"),
                      ((1, 12, 8, 128), "not a multiple"), ((1, 48, 3, 128), "group size 16"),
                      ((1, 8, 8, 96), "head_dim=96")]:
        with pytest.raises(pkv.PkvError, match=msg):
            path(*args)


def test_workspace_bytes():
    assert pkv.decode_workspace_bytes(32, 16, 128, 1) == 0
    assert pkv.decode_workspace_bytes(0, 16, 128, 4) == 0
    b = pkv.decode_workspace_bytes(32, 16, 128, 4)
    assert b >= 32 * 4 * 16 * 129 * 4 and b % 256 == 0


def dec(c, **kw):
    a = dict(q=FAKE, q_dtype=pkv.BF16, batch=3, hq=4, tables=FAKE, maxb=4, ctx=FAKE, ns=FAKE, max_ns=2, scale=0.125,
             out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 20)
    a.update(kw)
    return pkv.lib().pkv_paged_attention_decode(a["q"], a["q_dtype"], a["batch"], a["hq"], ctypes.byref(c), a["tables"],
                                                a["maxb"], a["ctx"], a["ns"], a["max_ns"], a["scale"], a["out"],
                                                a["lse"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("ckw,kw,status", [
    (dict(block_size=32), {}, -2),
    (dict(head_dim=96), {}, -2),
    (dict(num_kv_heads=3), {}, -1),            # 4 q heads not a multiple of 3
    (dict(num_kv_heads=2), dict(hq=6), -2),    # group of 3 not built
    (dict(kv_dtype=7), {}, -1),
    (dict(kv_dtype=pkv.I8), {}, -1),           # int8 without scales
    (dict(k=None), {}, -1),
    (dict(k=FAKE + 4), {}, -1),                # misaligned pool
    (dict(num_blocks=0), {}, -1),
    ({}, dict(q=None), -1),
    ({}, dict(q_dtype=pkv.I8), -1),
    ({}, dict(out=FAKE + 8), -1),
    ({}, dict(maxb=0), -1),
    ({}, dict(max_ns=0), -1),
    ({}, dict(ns=None), -1),
    ({}, dict(ws=None), -3),
    ({}, dict(ws_bytes=100), -3),
    ({}, dict(scale=float("inf")), -1),
    ({}, dict(batch=-1), -1),
])
def test_decode_rejects_bad_arguments(ckw, kw, status):
    assert dec(cache(**ckw), **kw) == status
    assert pkv.lib().pkv_last_error().decode().startswith("pkv_paged_attention_decode")


def test_reshape_rejects_bad_arguments():
    L = pkv.lib()
    c = cache()
    assert L.pkv_reshape_and_cache(FAKE, FAKE, pkv.F32, FAKE, 4, ctypes.byref(c), None) == -1   # bf16 cache, f32 rows
    assert L.pkv_reshape_and_cache(None, FAKE, pkv.BF16, FAKE, 4, ctypes.byref(c), None) == -1
    assert L.pkv_reshape_and_cache(FAKE, FAKE, pkv.BF16, FAKE + 4, 4, ctypes.byref(c), None) == -1
    assert L.pkv_reshape_and_cache(FAKE, FAKE, pkv.BF16, FAKE, -1, ctypes.byref(c), None) == -1
    ci8 = cache(kv_dtype=pkv.I8, k_scale=FAKE, v_scale=FAKE)
    assert L.pkv_reshape_and_cache(FAKE, FAKE, pkv.I8, FAKE, 4, ctypes.byref(ci8), None) == -1
    assert L.pkv_reshape_and_cache(FAKE, FAKE, pkv.BF16, FAKE, 0, ctypes.byref(c), None) == 0  # nothing to do
    assert L.pkv_reshape_and_cache(FAKE, FAKE, pkv.BF16, FAKE, 4, None, None) == -1


def test_decode_append_rejects_bad_arguments():
    """Every call fails a host check (or has nothing to do), so none launches."""
    L = pkv.lib()

    def app(c=None, **kw):
        a = dict(kn=FAKE, vn=FAKE, src=pkv.BF16, slots=FAKE, q=FAKE, q_dtype=pkv.BF16, batch=3, hq=4, maxb=4,
                 max_ns=1, out=FAKE)
        a.update(kw)
        c = c or cache()
        return L.pkv_paged_attention_decode_append(a["kn"], a["vn"], a["src"], a["slots"], a["q"], a["q_dtype"],
                                                   a["batch"], a["hq"], ctypes.byref(c), FAKE, a["maxb"], FAKE, None,
                                                   a["max_ns"], 0.125, a["out"], None, None, 0, None)

    assert app(max_ns=0) == -2               # the balanced mode has no append
    assert app(kn=None) == -1
    assert app(vn=None) == -1
    assert app(slots=None) == -1
    assert app(src=pkv.F32) == -1            # a bf16 cache takes bf16 rows
    assert app(c=cache(kv_dtype=pkv.I8, k_scale=FAKE, v_scale=FAKE), src=pkv.I8) == -1
    assert app(slots=FAKE + 4) == -1         # slot_mapping not 8-byte aligned
    assert app(kn=FAKE + 8) == -1            # rows not 16-byte aligned
    assert app(q=None) == -1                 # the decode checks apply too
    assert app(max_ns=2) == -1               # num_splits NULL with max_num_splits > 1
    assert pkv.lib().pkv_last_error().decode().startswith("pkv_paged_attention_decode_append")
    assert app(batch=0) == 0                 # nothing to do


def test_chunked_and_combine_reject_bad_arguments():
    L = pkv.lib()
    c = cache(head_dim=128)
    args = [FAKE, pkv.BF16, 2, 4, FAKE, 64, ctypes.byref(c), FAKE, 8, FAKE, 0.1, FAKE, None, None]
    bad = list(args); bad[1] = pkv.F32
    assert L.pkv_paged_attention_chunked(*bad) == -2
    bad = list(args); bad[6] = ctypes.byref(cache(head_dim=128, kv_dtype=pkv.F32))
    assert L.pkv_paged_attention_chunked(*bad) == -2
    bad = list(args); bad[5] = 0
    assert L.pkv_paged_attention_chunked(*bad) == -1
    bad = list(args); bad[4] = None
    assert L.pkv_paged_attention_chunked(*bad) == -1
    assert L.pkv_lse_combine(FAKE, FAKE, 2, 4, 96, 2, FAKE, FAKE, None, None) == -2
    assert L.pkv_lse_combine(None, FAKE, 2, 4, 128, 2, FAKE, FAKE, None, None) == -1
    assert L.pkv_lse_combine(FAKE, FAKE, 2, 4, 128, 0, FAKE, FAKE, None, None) == -1


def test_auto_mode_argument_checks():
    """"auto" resolves before anything else and refuses a split plan or the
    partials-only mode (both need an explicit split count)."""
    import torch
    t = torch.zeros(2, 3, dtype=torch.int32)
    with pytest.raises(ValueError, match="auto"):
        pkv.paged_attention_decode(None, None, t, t, t, "auto", 0.1)
    with pytest.raises(ValueError, match="auto"):
        pkv.paged_attention_decode(None, None, t, t, None, "auto", 0.1, partials_only=True)
    with pytest.raises(ValueError, match="GPU"):   # then the tensors are checked as for any mode
        pkv.paged_attention_decode(None, None, t, t, None, "auto", 0.1)


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(2, 4, 64)
    with pytest.raises(ValueError, match="GPU"):
        pkv.paged_attention_decode(q, None, q, q, None, 1, 0.1)


def test_noalloc_decode_rejects_before_any_device_call():
    """The allocation-free decode checks its arguments like the workspace
    decode, then refuses a call whose scratch would not fit the library's
    fixed array (PKV_ERR_WORKSPACE), all before touching the device."""
    L = pkv.lib()

    def na(c, **kw):
        a = dict(batch=3, hq=4, maxb=4, ns=FAKE, max_ns=2, out=FAKE)
        a.update(kw)
        return L.pkv_paged_attention_decode_noalloc(FAKE, pkv.BF16, a["batch"], a["hq"], ctypes.byref(c), FAKE,
                                                    a["maxb"], FAKE, a["ns"], a["max_ns"], 0.125, a["out"], None,
                                                    None)

    c = cache(head_dim=128)
    assert na(c, out=None) == -1
    assert na(c, ns=None) == -1
    assert na(cache(block_size=32)) == -2
    # 4096 x 64 splits x 4 heads x 129 floats = 541 MB > 48 MiB
    assert na(c, batch=4096, max_ns=64) == -3
    assert "needs" in L.pkv_last_error().decode()
    # balanced, group of 8: 65535 x 128 q heads of counters (33.6 MB) + 2048 x 2 x 8 x 129 x 4 (16.9 MB)
    # = 50.4 MB > 48 MiB
    assert na(cache(head_dim=128, num_kv_heads=16), batch=65535, hq=128, ns=None, max_ns=0) == -3
    assert na(c, batch=0) == 0
    assert pkv.NOALLOC_SCRATCH_BYTES == 48 << 20


def test_stream_read_rejects_bad_arguments():
    L = pkv.lib()
    assert L.pkv_stream_read(None, 1024, FAKE, None) == -1
    assert L.pkv_stream_read(FAKE, 1000, FAKE, None) == -1     # not a multiple of 16
    assert L.pkv_stream_read(FAKE + 8, 1024, FAKE, None) == -1
    assert L.pkv_stream_read(FAKE, 0, FAKE, None) == -1
    assert L.pkv_stream_read(FAKE, 1024, None, None) == -1
    assert L.pkv_stream_read_workgroups(0) == 0
    assert L.pkv_stream_read_workgroups(16) == 1
    assert L.pkv_stream_read_workgroups(34 << 20) == 2176      # 2,228,224 chunks / 1,024 per pass
    assert L.pkv_stream_read_workgroups(1 << 30) == 4096


def test_debug_mode_keeps_host_checks_first(monkeypatch):
    """With PKV_DEBUG=1 a call that fails a host check still returns before
    the device validation pass (nothing is launched here)."""
    monkeypatch.setenv("PKV_DEBUG", "1")
    assert dec(cache(), q=None) == -1
    assert "PKV_DEBUG" not in pkv.lib().pkv_last_error().decode()
    assert dec(cache(), ws=None) == -3
