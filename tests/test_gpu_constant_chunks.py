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
decode of every stream.  The one-wave decoder of 1024-element chunks fills a
payload in exactly that form directly; a stream long enough for that layout
checks it, beside the same payload re-coded validly in another form and one
with an invalid offset.
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


def test_one_word_route_of_the_one_wave_decoder(g, oracle_mod):
    """2100 chunks of 4096 bytes at word size 4 (enough for one wave per
    chunk, the layout whose decoder fills a payload in the encoder's one-word
    form directly): one-word chunks among Lorenzo chunks decode exactly; the
    same payload re-coded with other match lengths (still valid, so no longer
    the form) decodes to the oracle's output; a match offset turned invalid
    in such a payload gives the oracle's status."""
    import workloads
    cs, ws = 4096, 4
    e = cs // ws
    lor = workloads.lorenzo2d(99, 512, 512, 1e-3, noise=0.01)[0].astype(np.uint32)
    rng = np.random.default_rng(3)
    chunks = []
    for i in range(2100):
        if i % 3 == 0:
            chunks.append(np.full(e, int(rng.integers(1, 1 << 32)), dtype=np.uint32))
        else:
            st = int(rng.integers(0, lor.size - e))
            chunks.append(lor[st:st + e])
    data = np.concatenate(chunks).view(np.uint8)
    stream = oracle_mod.encode(data, cs, ws, 0)

    def gpu_decode(s):
        x = to_dev(s)
        out = torch.zeros(data.size, dtype=torch.uint8, device="cuda:0")
        nb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
        st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        dws = torch.empty(g.decode_workspace_size(s.size), dtype=torch.uint8, device="cuda:0")
        g.decode_into(x, s.size, out, nb, st, dws)
        torch.cuda.synchronize()
        return int(st.item()), int(nb.item()), out.cpu().numpy()

    st, nb, out = gpu_decode(stream)
    assert st == 0 and nb == data.size and np.array_equal(out, data)
    # the one-word payloads: literal (4 bytes), tokens (255,1) x 4, (3,1)
    nc = data.size // cs
    table = stream[32:32 + 8 * nc].view("<u4").reshape(nc, 2).astype(np.int64)
    f, d = table[:, 0], table[:, 1]
    sizes = np.where(f > 0, f + d, np.where(d & 0x80000000, d & 0x7FFFFFFF, 0))
    offs = 32 + 8 * nc + np.concatenate([[0], np.cumsum(sizes)])
    assert (f[::3] == 1).all() and (d[::3] == 14).all()
    c = 3 * 500
    p0 = int(offs[c]) + 1 + 4  # first token
    assert list(stream[p0:p0 + 10]) == [255, 1, 255, 1, 255, 1, 255, 1, 3, 1]
    # still valid, no longer the form: lengths 254, 255, 255, 255, 4
    other = stream.copy()
    other[p0] = 254
    other[p0 + 8] = 4
    r, ref = oracle_mod.decode_status(other, data.size)
    assert r == data.size and np.array_equal(ref, data)
    st, nb, out = gpu_decode(other)
    assert st == 0 and nb == data.size and np.array_equal(out, ref)
    # an offset of 2 at the first match (position 1) reaches before the chunk
    bad = stream.copy()
    bad[p0 + 1] = 2
    want, _ = oracle_mod.decode_status(bad, data.size)
    assert want == oracle_mod.ECORRUPT
    st, nb, _ = gpu_decode(bad)
    assert st == g.STATUS_CORRUPT and nb == 0
