"""Pins for the CPU oracle, against facts fixed outside the oracle itself.

* hand-worked streams derived from the page's rules (tests/golden/);
* brute-force longest match on every short sequence over tiny alphabets,
  using slice equality (not the oracle's element loop);
* the page's own search method (omask equality masks AND-ed until empty),
  written independently here, agreeing with the oracle at every position;
* the level-1 table in closed form (latest earlier-sub-block position with the
  same bucket) and its independence from insertion order;
* an independent Python encoder built from those two pieces, checked stream
  for stream against the oracle on small inputs;
* round trips, the worst-case bound, and corrupted-stream rejection.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import golden_cases

HASH_MUL = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1


def py_hash(w0: int, w1: int) -> int:
    """Bucket of a two-word key: top 11 bits of (w0 | w1<<32) * golden-ratio constant mod 2^64."""
    return (((w0 | (w1 << 32)) * HASH_MUL) & MASK64) >> 53


# ---------------------------------------------------------------- golden ---

CASES = golden_cases.load()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_examples_encode(oracle_mod, case):
    if case["name"] == "B5_period40_level1":
        # precondition of the hand derivation: no later colliding key in the
        # two buckets it relies on
        x = np.frombuffer(case["input"], dtype="<u4").astype(np.int64)
        b_a = py_hash(25, 26)
        assert all(py_hash(int(x[p]), int(x[p + 1])) != b_a for p in range(25, 64))
        b_b = py_hash(40, 1)
        assert all(py_hash(int(x[p]), int(x[p + 1])) != b_b for p in range(240, 256))
    got = oracle_mod.encode(case["input"], case["cs"], case["ws"], case["level"]).tobytes()
    assert got == case["stream"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_examples_decode(oracle_mod, case):
    out = oracle_mod.decode(case["stream"])
    assert out.tobytes() == case["input"]


def test_hash_matches_definition(oracle_mod):
    rng = np.random.default_rng(5)
    for _ in range(2000):
        a, b = (int(v) for v in rng.integers(0, 1 << 32, size=2, dtype=np.uint64))
        assert oracle_mod.hash2(a, b) == py_hash(a, b)
    assert oracle_mod.hash2(0, 0) == 0


# ------------------------------------------------------ near-window search ---

def brute_near(x, p):
    """Longest L <= 255 with x[p:p+L] == x[p-o:p-o+L] for some 1 <= o <= min(32, p);
    smallest such o."""
    E = len(x)
    best, bo = 0, 0
    for o in range(1, min(32, p) + 1):
        L = 0
        for k in range(min(255, E - p), 0, -1):
            if list(x[p:p + k]) == list(x[p - o:p - o + k]):
                L = k
                break
        if L > best:
            best, bo = L, o
    return best, bo


@pytest.mark.parametrize("alphabet,length", [(3, 7), (2, 10)])
def test_near_match_exhaustive(oracle_mod, alphabet, length):
    for seq in itertools.product(range(alphabet), repeat=length):
        x = np.array(seq, dtype=np.uint32)
        for p in range(length):
            assert oracle_mod.near_match(x, p) == brute_near(seq, p), (seq, p)


def omask_array(x: np.ndarray) -> np.ndarray:
    """omask[i]: bit o-1 set iff x[i] == x[i-o], o = 1..32 (page: search paragraph)."""
    E = x.size
    om = np.zeros(E, dtype=np.uint64)
    for o in range(1, 33):
        eq = np.zeros(E, dtype=bool)
        eq[o:] = x[o:] == x[:-o]
        om |= eq.astype(np.uint64) << np.uint64(o - 1)
    return om


def and_extension(om: np.ndarray, p: int) -> tuple[int, int]:
    """The page's extension: AND successive masks until no offset survives, cap 255."""
    s = int(om[p])
    if s == 0:
        return 0, 0
    L = 1
    while L < 255 and p + L < om.size:
        t = s & int(om[p + L])
        if t == 0:
            break
        s = t
        L += 1
    return L, (s & -s).bit_length()


def structured_chunk(rng, E):
    """Runs, short periods, copies at short distances and noise, small alphabet."""
    x = np.empty(E, dtype=np.uint32)
    i = 0
    while i < E:
        k = rng.integers(0, 4)
        ln = int(rng.integers(1, 300))
        ln = min(ln, E - i)
        if k == 0:
            x[i:i + ln] = rng.integers(0, 3)
        elif k == 1:
            per = int(rng.integers(1, 40))
            x[i:i + ln] = np.resize(rng.integers(0, 4, size=per), ln)
        elif k == 2 and i > 0:
            d = int(rng.integers(1, min(i, 64) + 1))
            for j in range(ln):
                x[i + j] = x[i + j - d]
        else:
            x[i:i + ln] = rng.integers(0, 5, size=ln)
        i += ln
    return x


@pytest.mark.parametrize("E", [256, 512, 1024])
def test_near_match_vs_omask_and(oracle_mod, E):
    rng = np.random.default_rng(E)
    for _ in range(6):
        x = structured_chunk(rng, E)
        om = omask_array(x)
        for p in range(E):
            assert oracle_mod.near_match(x, p) == and_extension(om, p), p


def test_near_match_cap_and_window(oracle_mod):
    # constant run: offset 1 reaches the cap, far beyond the 32-element window
    x = np.full(600, 9, dtype=np.uint32)
    assert oracle_mod.near_match(x, 1) == (255, 1)
    assert oracle_mod.near_match(x, 400) == (200, 1)
    # equal capped lengths at several offsets -> smallest offset
    y = np.resize(np.array([1, 2], dtype=np.uint32), 700)
    assert oracle_mod.near_match(y, 2) == (255, 2)
    # period 33 is outside the window
    z = np.resize(np.arange(33, dtype=np.uint32), 300)
    assert oracle_mod.near_match(z, 100) == (0, 0)
    # period 32 is the widest reachable
    w = np.resize(np.arange(32, dtype=np.uint32), 300)
    assert oracle_mod.near_match(w, 100) == (200, 32)
    for p in range(0, 300, 7):
        assert oracle_mod.near_match(x[:300], p) == brute_near(list(x[:300]), p)


# ------------------------------------------------ wider near windows ------

def brute_near_w(x, p, window):
    """brute_near with offsets 1..window."""
    E = len(x)
    best, bo = 0, 0
    for o in range(1, min(window, p) + 1):
        L = 0
        while L < 255 and p + L < E and x[p + L] == x[p + L - o]:
            L += 1
        if L > best:
            best, bo = L, o
    return best, bo


@pytest.mark.parametrize("window", [48, 64])
def test_near_match_window_brute_force(oracle_mod, window):
    rng = np.random.default_rng(window)
    for _ in range(20):
        x = rng.integers(0, 3, size=int(rng.integers(60, 200))).astype(np.uint32)
        seq = x.tolist()
        for p in range(x.size):
            assert oracle_mod.near_match(x, p, window) == brute_near_w(seq, p, window), (window, p)


@pytest.mark.parametrize("window", [48, 64])
def test_near_match_window_periods(oracle_mod, window):
    # a period is reachable exactly when it is at most the window
    for per, want in [(window, window), (window + 1, 0), (33, 33), (32, 32)]:
        z = np.resize(np.arange(per, dtype=np.uint32), 400)
        L, O = oracle_mod.near_match(z, 150, window)
        assert O == want and (L == 0) == (want == 0), (per, L, O)
    # window 32 still behaves as the stage's own search
    z = np.resize(np.arange(40, dtype=np.uint32), 300)
    assert oracle_mod.near_match(z, 100, 32) == oracle_mod.near_match(z, 100) == (0, 0)


@pytest.mark.parametrize("window", [32, 48, 64])
def test_encode_window_round_trip(oracle_mod, window):
    rng = np.random.default_rng(window + 1)
    base = rng.integers(0, 1000, size=60).astype(np.uint32)
    x = np.concatenate([np.resize(base[:per], 1000) for per in (20, 40, 50, 60, 70)]).astype("<u4")
    data = x.view(np.uint8)
    s = oracle_mod.encode(data, 2048, 4, 0, window)
    assert np.array_equal(oracle_mod.decode(s), data)
    if window == 32:
        assert np.array_equal(s, oracle_mod.encode(data, 2048, 4, 0))
    # wider windows never code the periodic segments worse
    assert s.size <= oracle_mod.encode(data, 2048, 4, 0, 32).size


# ----------------------------------------------------------- level 1 ------

def closed_form_candidates(x: np.ndarray):
    """cand[p] = p - c, c = the latest position before p's sub-block (and <= E-2)
    whose key has the same bucket, when 1 <= p - c <= 255; table[h] = 1 + the
    latest position <= E-2 with bucket h."""
    E = x.size
    sub = E // 8
    h = [py_hash(int(x[p]), int(x[p + 1])) if p + 1 < E else -1 for p in range(E)]
    cand = np.zeros(E, dtype=np.uint32)
    for p in range(E - 1):
        lo = (p // sub) * sub
        c = None
        for q in range(lo - 1, -1, -1):
            if h[q] == h[p]:
                c = q
                break
        if c is not None and 1 <= p - c <= 255:
            cand[p] = p - c
    table = np.zeros(2048, dtype=np.uint32)
    for p in range(E - 1):
        table[h[p]] = max(table[h[p]], p + 1)
    return cand, table


@pytest.mark.parametrize("E", [256, 512, 1024, 4096])
def test_level1_candidates_closed_form(oracle_mod, E):
    rng = np.random.default_rng(100 + E)
    xs = [structured_chunk(rng, E),
          rng.integers(0, 1 << 32, size=E, dtype=np.uint64).astype(np.uint32),
          np.resize(rng.integers(0, 50, size=int(rng.integers(33, 256))), E).astype(np.uint32)]
    for x in xs:
        cand, table = oracle_mod.level1_candidates(x)
        ec, et = closed_form_candidates(x)
        np.testing.assert_array_equal(cand, ec)
        np.testing.assert_array_equal(table, et)


def test_level1_insert_order_independent():
    # the max-insert makes the table independent of the order inserts land in
    rng = np.random.default_rng(3)
    x = rng.integers(0, 8, size=512).astype(np.uint32)
    pos = list(range(511))
    ref = {}
    for p in pos:
        b = py_hash(int(x[p]), int(x[p + 1]))
        ref[b] = max(ref.get(b, 0), p + 1)
    for _ in range(5):
        rng.shuffle(pos)
        t = {}
        for p in pos:
            b = py_hash(int(x[p]), int(x[p + 1]))
            t[b] = max(t.get(b, 0), p + 1)
        assert t == ref


# --------------------------------------------- independent Python encoder --

def py_encode_chunk(chunk: bytes, cs: int, ws: int, level: int):
    """Encoder built only from the omask-AND search and the closed-form table."""
    bc = len(chunk)
    padded = chunk + bytes(cs - bc)
    x = np.frombuffer(padded, dtype={1: "<u1", 2: "<u2", 4: "<u4"}[ws]).astype(np.uint32)
    E = x.size
    if not x.any():
        return 0, 0, b""
    om = omask_array(x)
    cand = closed_form_candidates(x)[0] if level == 1 else None
    mm = {1: 3, 2: 2, 4: 1}[ws]
    items = []
    p = 0
    while p < E:
        L, O = and_extension(om, p)
        if cand is not None and cand[p]:
            o = int(cand[p])
            r = 0
            while r < 255 and p + r < E and x[p + r] == x[p + r - o]:
                r += 1
            if r > L:
                L, O = r, o
        if L * ws > 2 and L >= mm:
            items.append((1, L, O))
            p += L
        else:
            items.append((0, p, 0))
            p += 1
    F = (len(items) + 7) // 8
    flags = bytearray(F)
    data = bytearray()
    for k, (m, a, b) in enumerate(items):
        if m:
            flags[k >> 3] |= 1 << (k & 7)
            data += bytes([a, b])
        else:
            data += padded[a * ws:(a + 1) * ws]
    if F + len(data) >= bc:
        return 0, 0x80000000 | bc, chunk
    return F, len(data), bytes(flags) + bytes(data)


@pytest.mark.parametrize("cs,ws", [(1024, 4), (2048, 4), (4096, 4), (1024, 2), (2048, 1), (1024, 1)])
@pytest.mark.parametrize("level", [0, 1])
def test_oracle_chunks_vs_independent_encoder(oracle_mod, cs, ws, level):
    rng = np.random.default_rng(cs * 10 + ws + level)
    E = cs // ws
    for t in range(4):
        if t == 0:
            x = structured_chunk(rng, E)
        elif t == 1:
            x = np.resize(rng.integers(0, 1 << (8 * ws), size=int(rng.integers(33, 120)), dtype=np.uint64), E)
        elif t == 2:
            x = rng.integers(0, 3, size=E)
        else:
            x = np.repeat(rng.integers(0, 4, size=E // 16), 16)
        raw = np.asarray(x, dtype={1: "<u1", 2: "<u2", 4: "<u4"}[ws]).tobytes()
        bc = cs if t != 3 else int(rng.integers(1, cs))
        chunk = raw[:bc]
        assert oracle_mod.encode_chunk(chunk, cs, ws, level) == py_encode_chunk(chunk, cs, ws, level)


# ------------------------------------------------ round trip and bounds ---

def random_inputs(rng, cs):
    sizes = [0, 1, 3, 7, cs - 1, cs, cs + 1, 2 * cs + 5, 3 * cs + 7]
    for n in sizes:
        yield rng.integers(0, 256, size=n, dtype=np.uint8)                      # incompressible
        yield np.zeros(n, dtype=np.uint8)                                        # zero chunks
        yield np.repeat(rng.integers(0, 3, size=n // 37 + 1, dtype=np.uint8), 37)[:n]  # runs
        yield np.resize(rng.integers(0, 256, size=int(rng.integers(1, 300)), dtype=np.uint8), n)


@pytest.mark.parametrize("cs", [1024, 2048, 4096])
@pytest.mark.parametrize("ws", [1, 2, 4])
@pytest.mark.parametrize("level", [0, 1])
def test_roundtrip_and_bound(oracle_mod, cs, ws, level):
    rng = np.random.default_rng(cs + 7 * ws + level)
    for a in random_inputs(rng, cs):
        s = oracle_mod.encode(a, cs, ws, level)
        chunks = (a.size + cs - 1) // cs
        assert s.size <= 32 + 8 * chunks + a.size
        assert oracle_mod.stream_info(s) == (a.size, s.size, cs, ws)
        np.testing.assert_array_equal(oracle_mod.decode(s), a)


def test_zero_chunks_cost_only_their_entry(oracle_mod):
    a = np.zeros(5 * 2048 + 100, dtype=np.uint8)
    s = oracle_mod.encode(a, 2048, 4, 0)
    assert s.size == 32 + 8 * 6
    a[3 * 2048 + 5] = 1
    s = oracle_mod.encode(a, 2048, 4, 0)
    e = s[32:32 + 48].view("<u4").reshape(6, 2)
    assert (e[[0, 1, 2, 4, 5]] == 0).all() and e[3, 0] > 0


def test_cross_level_streams_decode_identically(oracle_mod):
    import workloads as synth
    w = synth.workload(0)
    s0 = oracle_mod.encode(w.data, w.chunk_size, w.word_size, 0)
    s1 = oracle_mod.encode(w.data, w.chunk_size, w.word_size, 1)
    np.testing.assert_array_equal(oracle_mod.decode(s0), w.data)
    np.testing.assert_array_equal(oracle_mod.decode(s1), w.data)


# --------------------------------------------------------- corruption -----

def _good_stream(oracle_mod):
    a = np.tile(np.array([1, 2, 3, 4, 1, 2, 3, 4, 9], dtype="<u4"), 700).view(np.uint8)
    return oracle_mod.encode(a, 2048, 4, 0).copy(), a


def test_corrupt_headers_rejected(oracle_mod):
    s, a = _good_stream(oracle_mod)
    ECORRUPT = oracle_mod.ECORRUPT
    for off, val in [(0, 0x48), (4, 2), (5, 3), (6, 1), (8, 0xFF), (12, 0x77), (24, 0xFF)]:
        t = s.copy()
        t[off] = val
        assert oracle_mod.decode_status(t, a.size)[0] == ECORRUPT, off
    assert oracle_mod.decode_status(s[:20], a.size)[0] == ECORRUPT
    assert oracle_mod.decode_status(s[:-1], a.size)[0] == ECORRUPT
    assert oracle_mod.decode_status(s, a.size - 1)[0] == oracle_mod.ECAP


def test_corrupt_tokens_rejected(oracle_mod):
    # one chunk, constant run: payload = flags 0x0E, literal, (255,1), (255,1), (1,1)
    a = np.full(512, 7, dtype="<u4").view(np.uint8)
    s = oracle_mod.encode(a, 2048, 4, 0).copy()
    pay = 32 + 8
    assert s[pay] == 0x0E
    for idx, val in [(pay + 5, 0), (pay + 6, 2), (pay + 10, 0), (pay + 9, 0), (pay + 0, 0x1E),
                     (pay + 0, 0x0F), (pay + 6, 0)]:
        t = s.copy()
        t[idx] = val
        assert oracle_mod.decode_status(t, a.size)[0] == oracle_mod.ECORRUPT, (idx, val)
    # entry sizes that disagree with the payload
    for field_off, val in [(32, 2), (36, 11), (36, 9), (36, 0x80000000 | 2048)]:
        t = s.copy()
        t[field_off:field_off + 4] = np.frombuffer(np.uint32(val).tobytes(), np.uint8)
        assert oracle_mod.decode_status(t, a.size)[0] == oracle_mod.ECORRUPT, (field_off, val)


def test_random_bit_flips_never_misbehave(oracle_mod):
    s, a = _good_stream(oracle_mod)
    rng = np.random.default_rng(11)
    for _ in range(3000):
        t = s.copy()
        i = int(rng.integers(0, t.size))
        t[i] ^= np.uint8(1 << int(rng.integers(0, 8)))
        r, out = oracle_mod.decode_status(t, a.size + 64)
        assert r < 0 or r == out.size


def test_raw_threshold_at_equality(oracle_mod):
    # cs 1024, ws 4 (256 elements): distinct words except 16 positions that
    # repeat their left neighbour once -> 240 literals + 16 one-element matches
    # = 256 items: F = 32, D = 240*4 + 16*2 = 992, F + D = 1024 = chunk -> raw.
    x = np.arange(1, 257, dtype="<u4")
    for p in range(8, 256, 16):
        x[p] = x[p - 1]
    f, d, pay = oracle_mod.encode_chunk(x.tobytes(), 1024, 4, 0)
    assert (f, d) == (0, 0x80000000 | 1024) and pay == x.tobytes()
    # one more one-element match: F + D = 32 + 956 + 34 = 1022 < 1024 -> coded
    x[4] = x[3]
    f, d, pay = oracle_mod.encode_chunk(x.tobytes(), 1024, 4, 0)
    assert (f, d) == (32, 990)
