"""CPU oracle of the chunked LZSS coder (FZGPUModules "fz::GPULZStage" page).

TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers allowed.  The product
package never imports this module, and this module imports nothing from the
product package: the two share no code.

The arithmetic lives in ``gpulz_oracle.c`` (plain single-threaded C, built
with gcc into ``liboracle.so`` next to it).  This file only marshals numpy
buffers through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gpulz_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A separately built copy (the sanitizer test builds one with ASan/UBSan) may
# be named here; it is loaded instead of liboracle.so and never rebuilt.
_LIB_OVERRIDE = os.environ.get("GPULZ_ORACLE_LIB")
_lib = None

OK, EINVAL, ECAP, ECORRUPT = 0, -1, -2, -3
HEADER_BYTES = 32
ENTRY_BYTES = 8
RAW_BIT = 0x80000000


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (always recompiles)."""
    tmp = f"{_LIB_PATH}.{os.getpid()}.tmp"  # one per process: concurrent builds do not collide
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    global _lib
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    u8p = ctypes.c_void_p
    lib.oracle_max_stream_size.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
    lib.oracle_max_stream_size.restype = ctypes.c_uint64
    lib.oracle_hash.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
    lib.oracle_hash.restype = ctypes.c_uint32
    lib.oracle_near_match.argtypes = [u8p, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
    lib.oracle_near_match.restype = None
    lib.oracle_level1_candidates.argtypes = [u8p, ctypes.c_uint32, u8p, u8p]
    lib.oracle_level1_candidates.restype = None
    lib.oracle_encode_chunk.argtypes = [u8p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                        ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32),
                                        ctypes.POINTER(ctypes.c_uint32), u8p,
                                        ctypes.POINTER(ctypes.c_uint32)]
    lib.oracle_encode_chunk.restype = ctypes.c_int
    lib.oracle_encode.argtypes = [u8p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                  ctypes.c_uint32, u8p, ctypes.c_uint64]
    lib.oracle_encode.restype = ctypes.c_int64
    lib.oracle_decode.argtypes = [u8p, ctypes.c_uint64, u8p, ctypes.c_uint64]
    lib.oracle_decode.restype = ctypes.c_int64
    lib.oracle_stream_info.argtypes = [u8p, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64),
                                       ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint32),
                                       ctypes.POINTER(ctypes.c_uint32)]
    lib.oracle_stream_info.restype = ctypes.c_int
    u64 = ctypes.c_uint64
    lib.oracle_split_bounds.argtypes = [u64, ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(u64),
                                        ctypes.POINTER(u64), ctypes.POINTER(u64)]
    lib.oracle_split_bounds.restype = None
    lib.oracle_encode_split.argtypes = [u8p, u64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                        u8p, u64, u8p, u8p, u64, u8p, u64, ctypes.POINTER(u64)]
    lib.oracle_encode_split.restype = ctypes.c_int
    lib.oracle_decode_split.argtypes = [u8p, u64, u8p, u8p, u64, u8p, u64, u8p, u64]
    lib.oracle_decode_split.restype = ctypes.c_int64
    lib.oracle_near_match_w.argtypes = [u8p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                        ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
    lib.oracle_near_match_w.restype = None
    lib.oracle_encode_w.argtypes = [u8p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                    ctypes.c_uint32, u8p, ctypes.c_uint64]
    lib.oracle_encode_w.restype = ctypes.c_int64
    lib.oracle_lorenzo_quant.argtypes = [u8p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_double, u8p]
    lib.oracle_lorenzo_quant.restype = ctypes.c_uint64
    lib.oracle_advancing_match.argtypes = [u8p, ctypes.c_uint32, ctypes.c_uint32,
                                           ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
    lib.oracle_advancing_match.restype = None
    lib.oracle_encode_advancing.argtypes = [u8p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, u8p,
                                            ctypes.c_uint64]
    lib.oracle_encode_advancing.restype = ctypes.c_int64
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


def _bytes(buf) -> np.ndarray:
    a = np.ascontiguousarray(np.frombuffer(buf, dtype=np.uint8) if isinstance(buf, (bytes, bytearray))
                             else np.asarray(buf))
    return a.view(np.uint8).reshape(-1)


def max_stream_size(n: int, chunk_size: int) -> int:
    return int(_load().oracle_max_stream_size(n, chunk_size))


def hash2(w0: int, w1: int) -> int:
    return int(_load().oracle_hash(w0, w1))


def near_match(x: np.ndarray, p: int, window: int = 32) -> tuple[int, int]:
    """(L, O) of the exact near-window search (offsets 1..window) at element p
    of chunk x (uint32)."""
    x = np.ascontiguousarray(x, dtype=np.uint32)
    L, O = ctypes.c_uint32(), ctypes.c_uint32()
    if window == 32:
        _load().oracle_near_match(_ptr(x), x.size, p, ctypes.byref(L), ctypes.byref(O))
    else:
        _load().oracle_near_match_w(_ptr(x), x.size, p, window, ctypes.byref(L), ctypes.byref(O))
    return L.value, O.value


def advancing_match(x: np.ndarray, p: int) -> tuple[int, int]:
    """(L, O) of the upstream-style advancing-window search at element p of
    chunk x (uint32): the reading in oracle_advancing_match."""
    x = np.ascontiguousarray(x, dtype=np.uint32)
    L, O = ctypes.c_uint32(), ctypes.c_uint32()
    _load().oracle_advancing_match(_ptr(x), x.size, p, ctypes.byref(L), ctypes.byref(O))
    return L.value, O.value


def encode_advancing(data, chunk_size: int, word_size: int) -> np.ndarray:
    """Level-0 stream with the advancing-window search in place of the exact
    one; returns the stream as a uint8 array."""
    a = _bytes(data)
    cap = max_stream_size(a.size, chunk_size)
    if cap == 0:
        raise ValueError("unsupported chunk_size")
    out = np.empty(cap, dtype=np.uint8)
    r = _load().oracle_encode_advancing(_ptr(a), a.size, chunk_size, word_size, _ptr(out), cap)
    if r < 0:
        raise ValueError(f"oracle_encode_advancing status {r}")
    return out[:r]


def level1_candidates(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-position level-1 candidate offsets (0 = none) and the final table."""
    x = np.ascontiguousarray(x, dtype=np.uint32)
    cand = np.zeros(x.size, dtype=np.uint32)
    table = np.zeros(2048, dtype=np.uint32)
    _load().oracle_level1_candidates(_ptr(x), x.size, _ptr(cand), _ptr(table))
    return cand, table


def encode_chunk(chunk: bytes | np.ndarray, chunk_size: int, word_size: int, level: int):
    """Encode one chunk -> (flag_size, data_size, payload bytes)."""
    a = _bytes(chunk)
    f, d, pb = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint32()
    pay = np.zeros(chunk_size, dtype=np.uint8)
    st = _load().oracle_encode_chunk(_ptr(a), a.size, chunk_size, word_size, level,
                                     ctypes.byref(f), ctypes.byref(d), _ptr(pay), ctypes.byref(pb))
    if st != OK:
        raise ValueError(f"oracle_encode_chunk status {st}")
    return f.value, d.value, pay[:pb.value].tobytes()


def encode(data, chunk_size: int, word_size: int, level: int, window: int = 32) -> np.ndarray:
    """Encode a whole buffer (near window of `window` offsets: 32, 48 or 64);
    returns the stream as a uint8 array."""
    a = _bytes(data)
    cap = max_stream_size(a.size, chunk_size)
    if cap == 0:
        raise ValueError("unsupported chunk_size")
    out = np.empty(cap, dtype=np.uint8)
    if window == 32:
        r = _load().oracle_encode(_ptr(a), a.size, chunk_size, word_size, level, _ptr(out), cap)
    else:
        r = _load().oracle_encode_w(_ptr(a), a.size, chunk_size, word_size, level, window, _ptr(out), cap)
    if r < 0:
        raise ValueError(f"oracle_encode status {r}")
    return out[:r]


def decode_status(stream, cap: int | None = None) -> tuple[int, np.ndarray]:
    """Decode; returns (status_or_size, output array).  Never raises on corruption."""
    s = _bytes(stream)
    if cap is None:
        info = stream_info(s)
        cap = info[0] if info is not None else 0
    out = np.zeros(max(cap, 1), dtype=np.uint8)
    r = int(_load().oracle_decode(_ptr(s) if s.size else ctypes.c_void_p(1), s.size, _ptr(out), cap))
    return r, out[: max(r, 0)]


def decode(stream) -> np.ndarray:
    r, out = decode_status(stream)
    if r < 0:
        raise ValueError(f"oracle_decode status {r}")
    return out


def stream_info(stream):
    """(original_size, stream_bytes, chunk_size, word_size) or None if the header is invalid."""
    s = _bytes(stream)
    n, t = ctypes.c_uint64(), ctypes.c_uint64()
    cs, ws = ctypes.c_uint32(), ctypes.c_uint32()
    st = _load().oracle_stream_info(_ptr(s) if s.size else ctypes.c_void_p(1), s.size, ctypes.byref(n),
                                    ctypes.byref(t), ctypes.byref(cs), ctypes.byref(ws))
    if st != OK:
        return None
    return n.value, t.value, cs.value, ws.value


# ---- split mode: literals / lengths / offsets / meta ports ----------------

def split_bounds(n: int, chunk_size: int, word_size: int) -> tuple[int, int, int]:
    """Port capacities that always suffice: (literals, lengths = offsets, meta)."""
    a, b, c = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _load().oracle_split_bounds(n, chunk_size, word_size, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return a.value, b.value, c.value


def encode_split(data, chunk_size: int, word_size: int, level: int):
    """Encode into four ports; returns (literals, lengths, offsets, meta) uint8 arrays."""
    a = _bytes(data)
    bl, bt, bm = split_bounds(a.size, chunk_size, word_size)
    lit = np.empty(max(bl, 1), dtype=np.uint8)
    lens = np.empty(max(bt, 1), dtype=np.uint8)
    offs = np.empty(max(bt, 1), dtype=np.uint8)
    meta = np.empty(max(bm, 1), dtype=np.uint8)
    sizes = (ctypes.c_uint64 * 4)()
    st = _load().oracle_encode_split(_ptr(a), a.size, chunk_size, word_size, level, _ptr(lit), bl, _ptr(lens),
                                     _ptr(offs), bt, _ptr(meta), bm, sizes)
    if st != OK:
        raise ValueError(f"oracle_encode_split status {st}")
    return lit[:sizes[0]], lens[:sizes[1]], offs[:sizes[2]], meta[:sizes[3]]


def decode_split_status(lit, lens, offs, meta, cap: int | None = None) -> tuple[int, np.ndarray]:
    """Decode four ports; returns (status_or_size, output).  Never raises on corruption.
    lens and offs must have the same length (one byte per match each)."""
    lit, lens, offs, meta = (_bytes(v) for v in (lit, lens, offs, meta))
    if lens.size != offs.size:
        raise ValueError("lengths and offsets ports differ in length")
    if cap is None:
        cap = int(np.frombuffer(meta[16:24].tobytes(), dtype="<u8")[0]) if meta.size >= 32 else 0
    out = np.zeros(max(cap, 1), dtype=np.uint8)
    one = ctypes.c_void_p(1)
    r = int(_load().oracle_decode_split(_ptr(lit) or one, lit.size, _ptr(lens) or one, _ptr(offs) or one,
                                        lens.size, _ptr(meta) or one, meta.size, _ptr(out), cap))
    return r, out[: max(r, 0)]


def decode_split(lit, lens, offs, meta) -> np.ndarray:
    r, out = decode_split_status(lit, lens, offs, meta)
    if r < 0:
        raise ValueError(f"oracle_decode_split status {r}")
    return out


def lorenzo_quant(field, eb: float) -> tuple[np.ndarray, int]:
    """Lorenzo-quantizer front end: a float32 field of shape (nx,), (ny, nx)
    or (nz, ny, nx), x fastest, and an absolute error bound -> (u32 codes of
    the same shape, number of clamped cells)."""
    f = np.ascontiguousarray(field, dtype=np.float32)
    if f.ndim not in (1, 2, 3) or f.size == 0:
        raise ValueError("field must be a non-empty 1-D, 2-D or 3-D array")
    dims = (1,) * (3 - f.ndim) + f.shape  # (nz, ny, nx)
    codes = np.empty(f.shape, dtype=np.uint32)
    clamped = _load().oracle_lorenzo_quant(_ptr(f), dims[2], dims[1], dims[0], float(eb), _ptr(codes))
    return codes, int(clamped)


# ---- whole streams on several host threads -----------------------------------
# Chunks are coded independently (GPULZStage page, introduction: every chunk is
# compressed on its own), so the oracle run over contiguous whole-chunk ranges
# of the input, one call per range, yields the size-table rows and payloads of
# exactly those chunks; concatenated in range order they are the rows and
# payloads of the whole buffer.  Only the header's whole-buffer fields (chunk
# count, original size, payload or flag-byte total) are rewritten.  The
# per-range calls are the plain single-threaded oracle; the C calls release
# the interpreter lock, so the ranges run side by side.

def _ranges(n: int, chunk_size: int, parts: int) -> list[tuple[int, int]]:
    nch = -(-n // chunk_size)
    parts = max(1, min(parts, nch))
    per = -(-nch // parts)
    out = []
    for i in range(parts):
        c0, c1 = i * per, min(nch, (i + 1) * per)
        if c0 < c1:
            out.append((c0 * chunk_size, min(n, c1 * chunk_size)))
    return out


def _map_ranges(fn, a: np.ndarray, chunk_size: int, threads: int):
    from concurrent.futures import ThreadPoolExecutor
    rngs = _ranges(a.size, chunk_size, threads)
    with ThreadPoolExecutor(max_workers=max(1, len(rngs))) as ex:
        return list(ex.map(lambda r: fn(a[r[0]:r[1]]), rngs)), rngs


def encode_parallel(data, chunk_size: int, word_size: int, level: int, threads: int | None = None,
                    window: int = 32) -> np.ndarray:
    """The stream encode() returns, built from the oracle run on `threads`
    contiguous whole-chunk ranges at once (default: the host's CPUs, at most
    16)."""
    a = _bytes(data)
    threads = threads or max(1, min(16, os.cpu_count() or 1))
    if a.size <= chunk_size or threads == 1:
        return encode(a, chunk_size, word_size, level, window)
    parts, rngs = _map_ranges(lambda q: encode(q, chunk_size, word_size, level, window), a, chunk_size, threads)
    nch = -(-a.size // chunk_size)
    tables, pays = [], []
    for (lo, hi), s in zip(rngs, parts):
        k = -(-(hi - lo) // chunk_size)
        tables.append(s[HEADER_BYTES:HEADER_BYTES + ENTRY_BYTES * k])
        pays.append(s[HEADER_BYTES + ENTRY_BYTES * k:])
    payload = sum(int(p.size) for p in pays)
    head = parts[0][:HEADER_BYTES].copy()
    head[12:16] = np.frombuffer(np.uint32(nch).astype("<u4").tobytes(), dtype=np.uint8)
    head[16:24] = np.frombuffer(np.uint64(a.size).astype("<u8").tobytes(), dtype=np.uint8)
    head[24:32] = np.frombuffer(np.uint64(payload).astype("<u8").tobytes(), dtype=np.uint8)
    return np.concatenate([head, *tables, *pays])


def encode_split_parallel(data, chunk_size: int, word_size: int, level: int, threads: int | None = None):
    """The four ports encode_split() returns, built from the oracle run on
    `threads` contiguous whole-chunk ranges at once.  Ports concatenate in
    range order; meta = header | every range's rows | every range's flag
    bytes, with the header's chunk count, size and flag-byte total rewritten."""
    a = _bytes(data)
    threads = threads or max(1, min(16, os.cpu_count() or 1))
    if a.size <= chunk_size or threads == 1:
        return encode_split(a, chunk_size, word_size, level)
    parts, rngs = _map_ranges(lambda q: encode_split(q, chunk_size, word_size, level), a, chunk_size, threads)
    nch = -(-a.size // chunk_size)
    rows, flags = [], []
    for (lo, hi), (_, _, _, m) in zip(rngs, parts):
        k = -(-(hi - lo) // chunk_size)
        rows.append(m[HEADER_BYTES:HEADER_BYTES + ENTRY_BYTES * k])
        flags.append(m[HEADER_BYTES + ENTRY_BYTES * k:])
    nflag = sum(int(f.size) for f in flags)
    head = parts[0][3][:HEADER_BYTES].copy()
    head[12:16] = np.frombuffer(np.uint32(nch).astype("<u4").tobytes(), dtype=np.uint8)
    head[16:24] = np.frombuffer(np.uint64(a.size).astype("<u8").tobytes(), dtype=np.uint8)
    head[24:32] = np.frombuffer(np.uint64(nflag).astype("<u8").tobytes(), dtype=np.uint8)
    lit = np.concatenate([p[0] for p in parts])
    lens = np.concatenate([p[1] for p in parts])
    offs = np.concatenate([p[2] for p in parts])
    meta = np.concatenate([head, *rows, *flags])
    return lit, lens, offs, meta
