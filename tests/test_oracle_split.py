"""Pins of the oracle's split mode (four ports: literals, lengths, offsets,
meta) against things other than itself:

* hand-worked ports (tests/golden/split_examples.txt), restating the
  hand-worked single-stream examples in the split layout;
* an independent Python restriper of the oracle's single stream: the split
  ports must be exactly the single stream's items dealt out in order;
* decoding: round trips, agreement with the single-stream decoder when the
  same data byte is corrupted in both forms, and rejection of broken ports.
"""
from __future__ import annotations

import struct

import numpy as np
import pytest

from golden_cases import load_split

SPLIT_CASES = load_split()


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c["name"] for c in SPLIT_CASES])
def test_split_hand_examples(oracle_mod, case):
    lit, lens, offs, meta = oracle_mod.encode_split(case["input"], case["cs"], case["ws"], case["level"])
    assert lit.tobytes() == case["lit"]
    assert lens.tobytes() == case["lens"]
    assert offs.tobytes() == case["offs"]
    assert meta.tobytes() == case["meta"]
    back = oracle_mod.decode_split(case["lit"], case["lens"], case["offs"], case["meta"])
    assert back.tobytes() == case["input"]


def restripe(stream: bytes):
    """Independent restriper: walks a single stream's header, size table and
    payloads and deals every item into the four ports.  Also returns, for
    each byte of the literals / lengths / offsets ports, its position in the
    single stream."""
    magic, ver, ws, r0, r1, cs, nc, n, pb = struct.unpack_from("<IBBBBIIQQ", stream, 0)
    table = 32
    pay = 32 + 8 * nc
    lit, lens, offs, flags, entries = bytearray(), bytearray(), bytearray(), bytearray(), []
    lit_pos, len_pos, off_pos = [], [], []
    off = pay
    for c in range(nc):
        f, d = struct.unpack_from("<II", stream, table + 8 * c)
        if f == 0:
            size = d & 0x7FFFFFFF if d & 0x80000000 else 0
            lit += stream[off:off + size]
            lit_pos += list(range(off, off + size))
            entries.append((0, d))
            off += size
            continue
        fl = stream[off:off + f]
        dp = off + f
        used = k = m = 0
        while used < d:
            if (fl[k >> 3] >> (k & 7)) & 1:
                lens.append(stream[dp + used]); len_pos.append(dp + used)
                offs.append(stream[dp + used + 1]); off_pos.append(dp + used + 1)
                used += 2
                m += 1
            else:
                lit += stream[dp + used:dp + used + ws]
                lit_pos += list(range(dp + used, dp + used + ws))
                used += ws
            k += 1
        entries.append((k, m))
        flags += fl
        off += f + d
    meta = struct.pack("<IBBBBIIQQ", magic, 2, ws, 0, 0, cs, nc, n, len(flags))
    meta += b"".join(struct.pack("<II", a, b) for a, b in entries) + bytes(flags)
    return (bytes(lit), bytes(lens), bytes(offs), meta), (lit_pos, len_pos, off_pos)


def _inputs(rng, cs, ws):
    n = 5 * cs + int(rng.integers(1, cs))
    words = (rng.integers(0, 5, size=n // 4 + 1) * (rng.random(n // 4 + 1) < 0.7)).astype("<u4")
    data = bytearray(words.tobytes()[:n])
    data[cs:2 * cs] = bytes(cs)                      # an all-zero chunk
    data[2 * cs:3 * cs] = rng.integers(0, 256, size=cs, dtype=np.uint8).tobytes()  # a raw chunk
    return bytes(data)


@pytest.mark.parametrize("cs,ws,level", [(2048, 4, 0), (2048, 4, 1), (1024, 1, 0), (1024, 1, 1), (4096, 2, 0),
                                         (4096, 2, 1), (1024, 4, 1), (2048, 2, 0)])
def test_split_equals_restriped_single_stream(oracle_mod, cs, ws, level):
    rng = np.random.default_rng(cs * 10 + ws + level)
    data = _inputs(rng, cs, ws)
    single = oracle_mod.encode(data, cs, ws, level).tobytes()
    want, _ = restripe(single)
    got = tuple(p.tobytes() for p in oracle_mod.encode_split(data, cs, ws, level))
    assert got == want
    assert oracle_mod.decode_split(*got).tobytes() == data


def test_split_corruption_agrees_with_single_stream(oracle_mod):
    """A byte changed in the literals, lengths or offsets port decodes exactly
    as the same byte changed in the single stream (or both are rejected)."""
    rng = np.random.default_rng(11)
    for cs, ws, level in [(2048, 4, 0), (1024, 1, 1), (2048, 2, 1)]:
        data = _inputs(rng, cs, ws)
        single = bytearray(oracle_mod.encode(data, cs, ws, level).tobytes())
        ports, pos = restripe(bytes(single))
        for _ in range(60):
            which = int(rng.integers(0, 3))
            if len(ports[which]) == 0:
                continue
            i = int(rng.integers(0, len(ports[which])))
            v = int(rng.integers(1, 256))
            mod = [bytearray(p) for p in ports]
            mod[which][i] ^= v
            if which == 1:    # a length byte: the same token byte in both forms
                pass
            s2 = bytearray(single)
            s2[pos[which][i]] ^= v
            r1, o1 = oracle_mod.decode_split_status(*(bytes(m) for m in mod))
            r2, o2 = oracle_mod.decode_status(bytes(s2))
            assert (r1 < 0) == (r2 < 0), (cs, ws, level, which, i)
            if r1 >= 0:
                assert o1.tobytes() == o2.tobytes()


def test_split_rejects_broken_ports(oracle_mod):
    data = (np.arange(3000, dtype="<u4") % 7).tobytes()
    lit, lens, offs, meta = (p.tobytes() for p in oracle_mod.encode_split(data, 2048, 4, 0))
    ok, out = oracle_mod.decode_split_status(lit, lens, offs, meta)
    assert ok == len(data) and out.tobytes() == data
    bad = []
    m = bytearray(meta); m[4] = 1; bad.append((lit, lens, offs, bytes(m)))            # single-stream version
    m = bytearray(meta); m[0] ^= 1; bad.append((lit, lens, offs, bytes(m)))           # magic
    bad.append((lit[:-1], lens, offs, meta))                                           # literals too short
    bad.append((lit, lens[:-1], offs[:-1], meta))                                      # tokens too short
    bad.append((lit, lens, offs, meta[:-1]))                                           # flags cut
    m = bytearray(meta); struct.pack_into("<Q", m, 24, struct.unpack_from("<Q", m, 24)[0] + 1)
    bad.append((lit, lens, offs, bytes(m) + b"\0"))                                    # flag total wrong
    m = bytearray(meta); k, mm = struct.unpack_from("<II", m, 32)
    struct.pack_into("<II", m, 32, k, k + 1); bad.append((lit, lens, offs, bytes(m)))  # M > K
    m = bytearray(meta); struct.pack_into("<II", m, 32, 513, 0); bad.append((lit, lens, offs, bytes(m)))  # K > E
    m = bytearray(meta); m[-1] |= 0x80; bad.append((lit, lens, offs, bytes(m)))        # flag beyond the items / type change
    for b in bad:
        r, _ = oracle_mod.decode_split_status(*b, cap=len(data))
        assert r < 0


def test_split_zero_length_input(oracle_mod):
    lit, lens, offs, meta = oracle_mod.encode_split(b"", 2048, 4, 0)
    assert lit.size == lens.size == offs.size == 0 and meta.size == 32
    assert meta.tobytes()[:6] == bytes.fromhex("474C5A310204")
    r, out = oracle_mod.decode_split_status(lit, lens, offs, meta)
    assert r == 0
