"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, sizes its buffers as documented and
rejects bad arguments before touching the device."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def g():
    import chunked_lzss_coder_amd as g
    if not os.path.exists(g.LIB_PATH):
        from chunked_lzss_coder_amd import build
        build.build()
    return g


def declared_symbols():
    txt = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"GPULZ_API\s+\w+\s+(gpulz_\w+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == sorted(["gpulz_decode", "gpulz_decode_workspace_size", "gpulz_encode",
                                         "gpulz_encode_workspace_size", "gpulz_max_compressed_size",
                                         "gpulz_stream_info", "gpulz_encode_timed", "gpulz_decode_timed",
                                         "gpulz_split_bounds", "gpulz_encode_split_workspace_size",
                                         "gpulz_encode_split", "gpulz_decode_split_workspace_size",
                                         "gpulz_decode_split", "gpulz_decode_one_thread_per_chunk",
                                         "gpulz_lorenzo_quant", "gpulz_encode_window",
                                         "gpulz_encode_advancing_search", "gpulz_split_info",
                                         "gpulz_decode_noalloc"])


def test_library_exports_every_declared_symbol(g):
    lib = g.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert sorted(g.SYMBOLS) == declared_symbols()
    # nothing else with C linkage leaks out
    out = os.popen(f"nm -D --defined-only {g.LIB_PATH}").read()
    exported = sorted(set(re.findall(r"\bT (gpulz_\w+)", out)))
    assert exported == declared_symbols()


@pytest.mark.parametrize("cs", [1024, 2048, 4096])
def test_max_compressed_size(g, cs):
    for n in [0, 1, cs - 1, cs, cs + 1, 26_214_400, 2 << 30]:
        chunks = -(-n // cs)
        assert g.max_compressed_size(n, cs) == 32 + 8 * chunks + n
    assert g.max_compressed_size(100, 3000) == 0
    assert g.max_compressed_size(100, 512) == 0


def test_workspace_sizes(g):
    assert g.encode_workspace_size(1 << 20, 2048) >= 512 * 8
    assert g.encode_workspace_size(1 << 20, 777) == 0
    assert g.decode_workspace_size(32 + 8 * 1000) >= 1000 * 4  # one u32 tile offset per chunk
    assert g.decode_workspace_size(0) > 0


def test_stream_info_matches_oracle_streams(g, oracle_mod):
    rng = np.random.default_rng(0)
    for cs, ws, n in [(2048, 4, 5000), (1024, 1, 0), (4096, 2, 9000)]:
        a = rng.integers(0, 4, size=n, dtype=np.uint8)
        s = oracle_mod.encode(a, cs, ws, 0)
        assert g.stream_info(s[:32].tobytes()) == (n, s.size, cs, ws)
        assert g.stream_info(s[:31].tobytes()) is None
        bad = s[:32].copy()
        bad[0] ^= 1
        assert g.stream_info(bad.tobytes()) is None


def test_split_info_matches_oracle_meta(g, oracle_mod):
    rng = np.random.default_rng(1)
    for cs, ws, n in [(2048, 4, 5000), (1024, 1, 0), (4096, 2, 9000), (2048, 4, 40 * 2048)]:
        a = rng.integers(0, 4, size=n, dtype=np.uint8)
        meta = oracle_mod.encode_split(a, cs, ws, 1)[3]
        assert g.split_info(meta[:32].tobytes()) == (n, meta.size, cs, ws)
        assert g.split_info(meta[:31].tobytes()) is None
        # a one-stream header is not a meta port, and vice versa
        s = oracle_mod.encode(a, cs, ws, 0)
        assert g.split_info(s[:32].tobytes()) is None
        assert g.stream_info(meta[:32].tobytes()) is None
        for i, v in ((0, 1), (6, 1), (12, 1)):
            bad = meta[:32].copy()
            bad[i] ^= v
            assert g.split_info(bad.tobytes()) is None, i
        # more flag bytes than the chunks can hold
        bad = meta[:32].copy()
        nc = -(-n // cs)
        too_many = nc * ((cs // ws + 7) // 8) + 1
        bad[24:32] = np.frombuffer(np.uint64(too_many).astype("<u8").tobytes(), dtype=np.uint8)
        assert g.split_info(bad.tobytes()) is None


def _call_encode(g, ptr_in, n, cs, ws, level, ptr_out, cap, ptr_nb, ptr_ws, wsb):
    return g.lib().gpulz_encode(ptr_in, n, cs, ws, level, ptr_out, cap, ptr_nb, ptr_ws, wsb, None)


def test_encode_rejects_bad_arguments_before_launch(g):
    # fake non-null pointers: every call below must return before using them
    p = ctypes.c_void_p(0x1000)
    big = 1 << 40
    assert _call_encode(g, p, 100, 3000, 4, 0, p, big, p, p, big) == g.ERR_INVALID_ARG
    assert _call_encode(g, p, 100, 2048, 3, 0, p, big, p, p, big) == g.ERR_INVALID_ARG
    assert _call_encode(g, p, 100, 2048, 4, 2, p, big, p, p, big) == g.ERR_INVALID_ARG
    assert _call_encode(g, None, 100, 2048, 4, 0, p, big, p, p, big) == g.ERR_INVALID_ARG
    assert _call_encode(g, p, 100, 2048, 4, 0, None, big, p, p, big) == g.ERR_INVALID_ARG
    assert _call_encode(g, p, 100, 2048, 4, 0, p, big, None, p, big) == g.ERR_INVALID_ARG
    assert _call_encode(g, p, 100, 2048, 4, 0, p, big, p, None, big) == g.ERR_INVALID_ARG
    need = g.max_compressed_size(100, 2048)
    assert _call_encode(g, p, 100, 2048, 4, 0, p, need - 1, p, p, big) == g.ERR_CAPACITY
    wsn = g.encode_workspace_size(100, 2048)
    assert _call_encode(g, p, 100, 2048, 4, 0, p, need, p, p, wsn - 1) == g.ERR_CAPACITY


def test_decode_rejects_bad_arguments_before_launch(g):
    p = ctypes.c_void_p(0x1000)
    big = 1 << 40
    dec = g.lib().gpulz_decode
    assert dec(None, 100, p, big, p, p, p, big, None) == g.ERR_INVALID_ARG
    assert dec(p, 100, p, big, None, p, p, big, None) == g.ERR_INVALID_ARG
    assert dec(p, 100, p, big, p, None, p, big, None) == g.ERR_INVALID_ARG
    assert dec(p, 100, p, big, p, p, None, big, None) == g.ERR_INVALID_ARG
    assert dec(p, 100, None, 10, p, p, p, big, None) == g.ERR_INVALID_ARG
    assert dec(p, 31, p, big, p, p, p, big, None) == g.ERR_CORRUPT
    need = g.decode_workspace_size(1000)
    assert dec(p, 1000, p, big, p, p, p, need - 1, None) == g.ERR_CAPACITY


def test_decode_noalloc_rejects_bad_arguments_before_launch(g):
    # every call below fails a host check before the device is touched
    p = ctypes.c_void_p(0x1000)
    dec = g.lib().gpulz_decode_noalloc
    big = 1 << 40
    assert dec(None, 100, p, big, p, p, None) == g.ERR_INVALID_ARG
    assert dec(p, 100, p, big, None, p, None) == g.ERR_INVALID_ARG
    assert dec(p, 100, p, big, p, None, None) == g.ERR_INVALID_ARG
    assert dec(p, 100, None, 10, p, p, None) == g.ERR_INVALID_ARG
    assert dec(p, 31, p, big, p, p, None) == g.ERR_CORRUPT
    mx = g.DECODE_NOALLOC_MAX_CHUNKS
    # chunk bound = min((in_bytes - 32) / 8, ceil(out_capacity / 1024)) above the limit
    assert dec(p, 32 + 8 * (mx + 1), p, 1024 * (mx + 1), p, p, None) == g.ERR_CAPACITY
    assert dec(p, big, p, big, p, p, None) == g.ERR_CAPACITY
    hdr = open(os.path.join(ROOT, "include", "gpulz.h")).read()
    assert re.search(r"#define GPULZ_DECODE_NOALLOC_MAX_CHUNKS \(1ull << 22\)", hdr)
    assert mx == 1 << 22


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "chunked_lzss_coder_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "gpulz_oracle" not in txt and "liboracle" not in txt, f


@pytest.mark.parametrize("cs,ws", [(1024, 1), (2048, 4), (4096, 2)])
def test_split_bounds_match_the_oracle(g, oracle_mod, cs, ws):
    for n in [0, 1, cs, 3 * cs + 5, 26_214_400]:
        assert g.split_bounds(n, cs, ws) == oracle_mod.split_bounds(n, cs, ws)
    with pytest.raises(g.GpulzError):
        g.split_bounds(10, 3000, 4)


def test_split_rejects_bad_arguments_before_launch(g):
    p = ctypes.c_void_p(0x1000)
    big = 1 << 40
    enc = g.lib().gpulz_encode_split
    bl, bt, bm = g.split_bounds(100, 2048, 4)
    wsn = g.encode_split_workspace_size(100, 2048)
    args = [p, 100, 2048, 4, 0, p, bl, p, p, bt, p, bm, p, p, wsn, None]
    for i, bad in [(2, 3000), (3, 3), (4, 2), (0, None), (5, None), (7, None), (8, None), (10, None), (12, None),
                   (13, None)]:
        a = list(args); a[i] = bad
        assert enc(*a) == g.ERR_INVALID_ARG, i
    for i in (6, 9, 11, 14):
        a = list(args); a[i] = args[i] - 1
        assert enc(*a) == g.ERR_CAPACITY, i
    dec = g.lib().gpulz_decode_split
    need = g.decode_split_workspace_size(1000)
    dargs = [p, 10, p, p, 10, p, 1000, p, big, p, p, p, need, None]
    for i in (5, 9, 10, 11):
        a = list(dargs); a[i] = None
        assert dec(*a) == g.ERR_INVALID_ARG, i
    a = list(dargs); a[0] = None
    assert dec(*a) == g.ERR_INVALID_ARG
    a = list(dargs); a[6] = 31
    assert dec(*a) == g.ERR_CORRUPT
    a = list(dargs); a[12] = need - 1
    assert dec(*a) == g.ERR_CAPACITY


def test_lorenzo_quant_rejects_bad_arguments(g):
    # every call below fails a host check, so nothing is enqueued (the
    # pointers are never dereferenced)
    lib = g.lib()
    p = ctypes.c_void_p(0x1000)
    q = lambda f, nx, ny, nz, eb, c, k: lib.gpulz_lorenzo_quant(f, nx, ny, nz, eb, c, k, None)
    assert q(None, 4, 4, 1, 0.1, p, p) == g.ERR_INVALID_ARG
    assert q(p, 4, 4, 1, 0.1, None, p) == g.ERR_INVALID_ARG
    assert q(p, 4, 4, 1, 0.1, p, None) == g.ERR_INVALID_ARG
    for dims in [(0, 4, 1), (4, 0, 1), (4, 4, 0), (1 << 16, 1 << 16, 1), (1 << 11, 1 << 11, 1 << 10)]:
        assert q(p, *dims, 0.1, p, p) == g.ERR_INVALID_ARG
    for eb in [0.0, -1.0, float("nan"), float("inf"), 1e308]:
        assert q(p, 4, 4, 1, eb, p, p) == g.ERR_INVALID_ARG
    assert q(ctypes.c_void_p(0x1002), 4, 4, 1, 0.1, p, p) == g.ERR_INVALID_ARG
    assert q(p, 4, 4, 1, 0.1, ctypes.c_void_p(0x1001), p) == g.ERR_INVALID_ARG
    assert q(p, 4, 4, 1, 0.1, p, ctypes.c_void_p(0x1004)) == g.ERR_INVALID_ARG


def test_encode_window_rejects_bad_windows(g):
    lib = g.lib()
    p = ctypes.c_void_p(0x1000)
    for window in (0, 16, 31, 33, 40, 96, 128):
        # a bad window fails before any launch (pointers never dereferenced)
        assert lib.gpulz_encode_window(p, 4096, 2048, 4, 0, window, p, 1 << 20, p, p, 1 << 30, None) \
            == g.ERR_INVALID_ARG


def test_encode_advancing_search_rejects_bad_arguments(g):
    lib = g.lib()
    p = ctypes.c_void_p(0x1000)
    big = 1 << 40
    # fails before any launch: pointers never dereferenced
    for cs, ws in ((3000, 4), (2048, 3), (512, 1)):
        assert lib.gpulz_encode_advancing_search(p, 100, cs, ws, p, big, p, p, big, None, None, None) \
            == g.ERR_INVALID_ARG
    assert lib.gpulz_encode_advancing_search(None, 100, 2048, 4, p, big, p, p, big, None, None, None) \
        == g.ERR_INVALID_ARG
    need = g.max_compressed_size(100, 2048)
    assert lib.gpulz_encode_advancing_search(p, 100, 2048, 4, p, need - 1, p, p, big, None, None, None) \
        == g.ERR_CAPACITY
    wsn = g.encode_workspace_size(100, 2048)
    assert lib.gpulz_encode_advancing_search(p, 100, 2048, 4, p, need, p, p, wsn - 1, None, None, None) \
        == g.ERR_CAPACITY


def test_missing_library_fails_loudly(monkeypatch):
    # no CPU fallback: without the built library every entry point raises
    import chunked_lzss_coder_amd as gl
    monkeypatch.setattr(gl, "_lib", None)
    monkeypatch.setattr(gl, "LIB_PATH", gl.LIB_PATH + ".absent")
    with pytest.raises(gl.GpulzError):
        gl.lib()
    with pytest.raises(gl.GpulzError):
        gl.max_compressed_size(100, 2048)
