"""Pins of the oracle's upstream-style advancing-window search (CPU only).

Per the GPULZStage page (exact longest-match search paragraph), upstream's
search moves its candidate pointer forward with each comparison, so while a
match is being extended the starts it passes are never tried, and its
matches come out shorter than the exact search's.  The oracle's reading: the pointer w
walks the 32 elements before p, one comparison per step of x[w] against the
element the partial match needs next; a mismatch drops the partial match and
spends that w; the longest partial match seen wins (the first on ties).

These tests fix that reading by values worked out by hand, a closed form on
constant chunks, a whole hand-built stream, and properties any correct
implementation of it has (every result is a real match inside the window,
never longer than the exact search's).
"""
import numpy as np
import pytest

import oracle

# x = 5 6 5 6 5 6 7 5 6 7, worked by hand step by step:
#   p=2: w=0 5=5 len 1 (start 0); w=1 6=6 len 2           -> (2, 2)   exact (4, 2)
#   p=4: w=0,1 grow to 2 (start 0); w=2 5 vs x[6]=7 drop;
#        w=3 6 vs x[4]=5 no                                -> (2, 4)   exact (2, 2)
#   p=5: w=1 6=6 len 1 (start 1); w=2 drop; w=3 len 1 again (not longer) -> (1, 4)
#   p=7: w=0,1 grow to 2 (start 0); w=2 drop; w=3 no; w=4,5,6 grow to 3
#        (start 4)                                         -> (3, 3)
HAND = np.array([5, 6, 5, 6, 5, 6, 7, 5, 6, 7], np.uint32)
HAND_WANT = {0: (0, 0), 1: (0, 0), 2: (2, 2), 3: (2, 2), 4: (2, 4), 5: (1, 4), 6: (0, 0),
             7: (3, 3), 8: (2, 3), 9: (1, 3)}


@pytest.mark.parametrize("p", sorted(HAND_WANT))
def test_hand_worked(p):
    assert oracle.advancing_match(HAND, p) == HAND_WANT[p]


@pytest.mark.parametrize("E", [40, 256, 1024])
def test_constant_chunk_closed_form(E):
    # every window element equals x[p]: the partial match started at the
    # window's first element grows on every step until it reaches p or the
    # chunk end, so L = min(p, 32, E - p) and O = min(p, 32)
    x = np.full(E, 9, np.uint32)
    for p in range(E):
        L, O = oracle.advancing_match(x, p)
        if p == 0:
            assert (L, O) == (0, 0)
        else:
            assert L == min(p, 32, E - p)
            assert O == min(p, 32)


def test_no_repeat_in_window():
    x = np.arange(1, 200, dtype=np.uint32)
    for p in range(x.size):
        assert oracle.advancing_match(x, p) == (0, 0)


@pytest.mark.parametrize("alphabet", [2, 3, 5])
def test_results_are_window_matches_never_longer_than_exact(alphabet):
    rng = np.random.default_rng(alphabet)
    x = rng.integers(0, alphabet, size=300).astype(np.uint32)
    shorter = 0
    for p in range(x.size):
        L, O = oracle.advancing_match(x, p)
        Le, _ = oracle.near_match(x, p)
        if L == 0:
            assert O == 0
            continue
        # a real match, inside the 32-element window, its source before p
        assert 1 <= O <= 32 and O <= p and L <= O
        assert all(x[p + k] == x[p + k - O] for k in range(L))
        assert p + L <= x.size
        assert L <= Le
        shorter += L < Le
    assert shorter > 0  # the approximation does settle for shorter matches


def test_whole_stream_by_hand():
    # 256 words of 7 (chunk 1024, word 4).  Items: a literal at 0, then
    # matches (1,1) (2,2) (4,4) (8,8) (16,16) at 1, 2, 4, 8, 16, then seven
    # (32,32) from 32 to 256: 13 items, 12 of them matches.
    # flags: bit 0 clear, bits 1-12 set -> FE 1F (F = 2); data: the literal's
    # 4 bytes, then length, offset per match (D = 4 + 24 = 28).
    data = np.full(256, 7, np.uint32).view(np.uint8)
    s = oracle.encode_advancing(data, 1024, 4)
    payload = bytes([0xFE, 0x1F, 7, 0, 0, 0, 1, 1, 2, 2, 4, 4, 8, 8, 16, 16] + [32, 32] * 7)
    header = (b"GLZ1" + bytes([1, 4, 0, 0]) + (1024).to_bytes(4, "little") + (1).to_bytes(4, "little")
              + (1024).to_bytes(8, "little") + len(payload).to_bytes(8, "little"))
    table = (2).to_bytes(4, "little") + (28).to_bytes(4, "little")
    assert s.tobytes() == header + table + payload
    assert oracle.decode(s).tobytes() == data.tobytes()


@pytest.mark.parametrize("cs,ws", [(1024, 1), (2048, 2), (4096, 4), (1024, 4)])
def test_round_trip_and_only_the_search_differs(cs, ws):
    # same stream rules as the exact coder: decodes with the same decoder; on
    # data without repeats both searches find nothing and the streams agree
    rng = np.random.default_rng(cs + ws)
    a = rng.integers(0, 4, size=3 * cs + 77).astype(np.uint8)
    s = oracle.encode_advancing(a, cs, ws)
    assert oracle.decode(s).tobytes() == a.tobytes()
    u = rng.permutation(np.arange(2 * cs // 4, dtype=np.uint32) * 2654435761).astype(np.uint32).view(np.uint8)
    assert oracle.encode_advancing(u, cs, ws).tobytes() == oracle.encode(u, cs, ws, 0).tobytes()


def test_exact_search_compresses_better_on_structured_data():
    # the page's claim, on repeats longer than the window and on short periods
    a = np.concatenate([np.full(3000, 3, np.uint32), np.tile(np.arange(1, 8, dtype=np.uint32), 400)])
    b = a.view(np.uint8)
    assert oracle.encode(b, 2048, 4, 0).size < oracle.encode_advancing(b, 2048, 4).size
