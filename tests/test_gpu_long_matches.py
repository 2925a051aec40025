"""GPU parity of streams whose chunks hold several long near matches (16
words or more) inside one 64-position word of the parse, through the C ABI
against the oracle.

Level 0 with chunks of up to 1024 elements finds a long match's exact length
only where the parse starts an item on it; the parse then goes on after the
match, possibly inside the same word, and each word's item-start bits are
rebuilt from the lengths found.  These chunks put one to three long matches
in the same word (starting and ending mid-word), matches that cross one or
more word boundaries, matches that run to the 255 cap, literals between
them, and a ragged tail; level 1 and the larger chunks (exact lengths
everywhere) take the same inputs.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunked_lzss_coder_amd as g
    g.lib()
    return g


def long_match_words(rng, n_words: int, top: int) -> np.ndarray:
    """Random words (top: exclusive bound) with copies of earlier stretches
    pasted in: offset 1..32, length 16..70 (often several per 64 words),
    now and then 200..300 (past the length cap)."""
    a = rng.integers(1, top, size=n_words, dtype=np.uint64)
    p = 40
    while p < n_words - 16:
        p += int(rng.integers(0, 20))  # literals before the copy
        o = int(rng.integers(1, 33))
        ln = int(rng.integers(200, 300)) if rng.random() < 0.08 else int(rng.integers(16, 71))
        ln = min(ln, n_words - p)
        for k in range(ln):  # element by element: overlapping copies repeat
            a[p + k] = a[p + k - o]
        p += ln
    return a


@pytest.mark.parametrize("cs,ws", [(2048, 4), (4096, 4), (1024, 1), (2048, 2), (1024, 2), (4096, 1)])
@pytest.mark.parametrize("level", [0, 1])
def test_long_matches_within_words(g, oracle_mod, cs, ws, level):
    rng = np.random.default_rng(cs * 10 + ws + 100 * level)
    dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[ws]
    n_words = (cs // ws) * 24 + 333  # 24 chunks and a ragged tail
    words = long_match_words(rng, n_words, 1 << (8 * ws) if ws < 4 else 1 << 32).astype(dt)
    data = words.view(np.uint8)
    x = torch.from_numpy(np.ascontiguousarray(data)).to("cuda:0")
    out, nb = g.encode(x, cs, ws, level)
    torch.cuda.synchronize()
    k = int(nb.item())
    want = oracle_mod.encode(data, cs, ws, level)
    got = out[:k].cpu().numpy()
    assert got.size == want.size and np.array_equal(got, want), (cs, ws, level)
    dec, _, st = g.decode(out, k)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and np.array_equal(dec.cpu().numpy(), data)
