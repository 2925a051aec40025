"""GPU parity of chunks made of one repeated nonzero word, through the C ABI
against the oracle.

Such a chunk's greedy parse is fixed (a literal, then matches at offset 1 of
length min(255, remaining) while at least the minimum match remains, then the
remaining words as literals), and the chunk kernel writes that payload
without searching.  These streams mix such chunks (several word values,
including ones whose bytes differ, so byte order matters) with chunks that
must not take that route: a zero chunk, one word changed at the start, at the
end or in the middle, and a ragged constant tail (its padding is zeros).
Every chunk size, word size and level; windows 48 and 64; split mode; and the
decode of every stream.
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


def constant_mix(cs: int, ws: int, seed: int) -> np.ndarray:
    """Chunks in a fixed order: constants of several values, a zero chunk, a
    constant with its first / last / middle word changed, more constants, and
    a ragged tail of a constant word."""
    rng = np.random.default_rng(seed)
    e = cs // ws
    dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[ws]
    top = 1 << (8 * ws)
    vals = [1, top - 1, int(rng.integers(1, top)), 0x01020304 % top or 1, 0x80 % top or 1]
    chunks = []
    for v in vals:
        chunks.append(np.full(e, v, dtype=dt))
    chunks.append(np.zeros(e, dtype=dt))
    for where in (0, e - 1, e // 2):
        c = np.full(e, vals[2], dtype=dt)
        c[where] = (vals[2] + 1) % top
        chunks.append(c)
    for v in vals[:2]:
        chunks.append(np.full(e, v, dtype=dt))
    chunks.append(np.full(e // 3 + 1, vals[3], dtype=dt))  # ragged tail
    return np.concatenate(chunks).view(np.uint8)


def to_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


@pytest.mark.parametrize("cs", [1024, 2048, 4096])
@pytest.mark.parametrize("ws", [1, 2, 4])
def test_constant_chunks_match_oracle(g, oracle_mod, cs, ws):
    data = constant_mix(cs, ws, cs + ws)
    x = to_dev(data)
    for level in (0, 1):
        out, nb = g.encode(x, cs, ws, level)
        torch.cuda.synchronize()
        k = int(nb.item())
        got = out[:k].cpu().numpy()
        want = oracle_mod.encode(data, cs, ws, level)
        assert got.size == want.size and np.array_equal(got, want), (cs, ws, level)
        dec, _, st = g.decode(out, k)
        torch.cuda.synchronize()
        assert int(st.item()) == 0 and np.array_equal(dec.cpu().numpy(), data), (cs, ws, level)


@pytest.mark.parametrize("window", [48, 64])
def test_constant_chunks_wider_windows(g, oracle_mod, window):
    cs, ws = 2048, 4
    data = constant_mix(cs, ws, window)
    x = to_dev(data)
    cap = g.max_compressed_size(data.size, cs)
    out = torch.zeros(cap, dtype=torch.uint8, device="cuda:0")
    nb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
    wsp = torch.empty(g.encode_workspace_size(data.size, cs), dtype=torch.uint8, device="cuda:0")
    for level in (0, 1):
        g.encode_window_into(x, cs, ws, level, window, out, nb, wsp)
        torch.cuda.synchronize()
        k = int(nb.item())
        want = oracle_mod.encode(data, cs, ws, level, window)
        assert np.array_equal(out[:k].cpu().numpy(), want), (window, level)


@pytest.mark.parametrize("ws", [1, 4])
def test_constant_chunks_split_mode(g, oracle_mod, ws):
    cs = 4096
    data = constant_mix(cs, ws, 7 * ws)
    x = to_dev(data)
    lit, lens, offs, meta, pb = g.encode_split(x, cs, ws, 0)
    torch.cuda.synchronize()
    sizes = [int(v) for v in pb.cpu().tolist()]
    ref = oracle_mod.encode_split(data, cs, ws, 0)
    for t, n_, r in zip((lit, lens, offs, meta), sizes, ref):
        assert np.array_equal(t[:n_].cpu().numpy(), r)
    dec, _, st = g.decode_split(lit, lens, offs, meta, port_bytes=pb)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and np.array_equal(dec.cpu().numpy(), data)
