"""The oracle run on contiguous whole-chunk ranges across threads, stitched,
gives exactly the single-threaded oracle's stream and ports.

Chunks are coded independently (GPULZStage page, introduction), so the only
whole-buffer fields are the header's chunk count, original size and payload
(or flag-byte) total; everything else is the per-range output concatenated.
These checks pin the stitching against the plain single call on inputs with
ragged tails, more threads than chunks, zero and raw chunks, both levels,
every word size and the wider near windows.
"""
from __future__ import annotations

import numpy as np
import pytest


def mixed(rng, n):
    parts = [np.zeros(0, dtype=np.uint8)]
    while sum(p.size for p in parts) < n:
        k = int(rng.integers(0, 4))
        ln = int(rng.integers(64, 6000))
        if k == 0:
            parts.append(np.zeros(ln, dtype=np.uint8))
        elif k == 1:
            parts.append(rng.integers(0, 256, size=ln, dtype=np.uint8))
        elif k == 2:
            parts.append(np.resize(rng.integers(0, 256, size=int(rng.integers(1, 90)), dtype=np.uint8), ln))
        else:
            parts.append(rng.integers(0, 3, size=ln, dtype=np.uint8))
    return np.concatenate(parts)[:n]


@pytest.mark.parametrize("cs", [1024, 4096])
@pytest.mark.parametrize("ws", [1, 2, 4])
@pytest.mark.parametrize("level", [0, 1])
def test_encode_parallel_equals_single_call(oracle_mod, cs, ws, level):
    rng = np.random.default_rng(cs + 10 * ws + level)
    for n in (0, 1, cs - 3, cs, 5 * cs + 17, 37 * cs, 37 * cs + 1):
        data = mixed(rng, n)
        ref = oracle_mod.encode(data, cs, ws, level)
        for threads in (1, 2, 3, 8, 64):
            got = oracle_mod.encode_parallel(data, cs, ws, level, threads=threads)
            assert got.dtype == np.uint8 and np.array_equal(got, ref), (n, threads)


@pytest.mark.parametrize("window", [48, 64])
def test_encode_parallel_windows(oracle_mod, window):
    rng = np.random.default_rng(window)
    data = mixed(rng, 19 * 2048 + 5)
    ref = oracle_mod.encode(data, 2048, 4, 1, window=window)
    assert np.array_equal(oracle_mod.encode_parallel(data, 2048, 4, 1, threads=5, window=window), ref)


@pytest.mark.parametrize("ws", [1, 4])
@pytest.mark.parametrize("level", [0, 1])
def test_encode_split_parallel_equals_single_call(oracle_mod, ws, level):
    rng = np.random.default_rng(100 + ws + level)
    cs = 2048
    for n in (0, 7, cs, 3 * cs + 9, 29 * cs + 1001):
        data = mixed(rng, n)
        ref = oracle_mod.encode_split(data, cs, ws, level)
        for threads in (1, 2, 7, 40):
            got = oracle_mod.encode_split_parallel(data, cs, ws, level, threads=threads)
            for a, b in zip(got, ref):
                assert np.array_equal(a, b), (n, threads)


def test_parallel_header_fields_rewritten(oracle_mod):
    """A planted stitch that keeps the first range's header would differ:
    with several ranges the header's chunk count, size and payload total are
    the whole buffer's, as the stream walker reads them."""
    rng = np.random.default_rng(3)
    data = mixed(rng, 40 * 4096 + 3)
    s = oracle_mod.encode_parallel(data, 4096, 4, 0, threads=4)
    nc = int(np.frombuffer(s[12:16].tobytes(), "<u4")[0])
    n = int(np.frombuffer(s[16:24].tobytes(), "<u8")[0])
    pb = int(np.frombuffer(s[24:32].tobytes(), "<u8")[0])
    assert (nc, n) == (41, data.size)
    assert 32 + 8 * nc + pb == s.size
    assert np.array_equal(oracle_mod.decode(s), data)
