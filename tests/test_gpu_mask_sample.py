"""GPU parity of the level-0 offset-mask pass's shortcut for chunks without
near matches (word size 4, window 32), through the C ABI against the oracle.

The pass computes the masks of every lane's last position first; when none
has a near match it tests the remaining positions by compares alone and
leaves a chunk with no match at all raw.  These inputs drive each route:
words with no repeats (raw), matches only at positions the first step never
looks at (the compares find them, the masks are then computed), zero words
among the first 32 positions (compared against the zeros ahead of the chunk,
a false hit that must only cost time), and all of them in one stream.
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


def unique_words(rng, n):
    """n distinct nonzero u32 words (no near match anywhere)."""
    v = rng.choice(np.arange(1, 1 << 31, dtype=np.uint64), size=n, replace=False) * 2 + 1
    return v.astype(np.uint32)


def off_sample_matches(rng, e, ppass):
    """Distinct words, except that inside every group of ppass positions the
    words before the group's last one repeat their left neighbour: many near
    matches, none at a group's last position."""
    w = unique_words(rng, e)
    for p in range(e):
        q = p % ppass
        if 1 <= q < ppass - 1:
            w[p] = w[p - 1]
    return w


def encode_gpu(g, data, cs, level=0):
    x = torch.from_numpy(np.ascontiguousarray(data).view(np.uint8)).to("cuda:0")
    out, nb = g.encode(x, cs, 4, level)
    torch.cuda.synchronize()
    k = int(nb.item())
    assert k > 0
    return out[:k].cpu().numpy()


@pytest.mark.parametrize("cs", [1024, 2048, 4096])
def test_mask_shortcut_routes_match_oracle(g, oracle_mod, cs):
    e = cs // 4
    ppass = 4 if e == 256 else 8
    rng = np.random.default_rng(cs)
    chunks = []
    chunks.append(unique_words(rng, e))                       # no match: raw
    chunks.append(off_sample_matches(rng, e, ppass))          # matches off the sampled positions
    zs = unique_words(rng, e)
    zs[[3, 17, 30]] = 0                                        # zeros among the first 32 words
    chunks.append(zs)
    zr = unique_words(rng, e)
    zr[5] = 0
    zr[200 % e] = 0                                            # one real repeat (zero twice, far apart)
    chunks.append(zr)
    chunks.append(np.full(e, 7, dtype=np.uint32))              # constant: matched at sampled positions
    for i, c in enumerate(chunks):
        data = c.astype("<u4").view(np.uint8)
        got = encode_gpu(g, data, cs)
        want = oracle_mod.encode(data, cs, 4, 0)
        assert np.array_equal(got, want), (cs, i)
    # all of them in one stream, twice over, with a ragged tail
    whole = np.concatenate(chunks + chunks).astype("<u4").view(np.uint8)
    whole = np.concatenate([whole, unique_words(rng, 37).astype("<u4").view(np.uint8)])
    got = encode_gpu(g, whole, cs)
    want = oracle_mod.encode(whole, cs, 4, 0)
    assert np.array_equal(got, want)
    # and the stream decodes back
    st = torch.from_numpy(got.copy()).to("cuda:0")
    dec, dnb, status = g.decode(st, got.size)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and np.array_equal(dec[: whole.size].cpu().numpy(), whole)
