"""A seeded random sweep across the whole parameter space: chunk size, word
size, match level, near window, input length (ragged, up to a few dozen
chunks) and data shape (runs, short and long periods, small alphabets,
noise, zero and raw chunks).  Every case's GPU stream must equal the
oracle's byte for byte and decode back to the input; some cases also run
split mode and the advancing-search baseline against their oracle
counterparts.  Complements the targeted parity tests with combinations
they do not enumerate."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = 40


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunked_lzss_coder_amd as g
    g.lib()
    return g


def shaped(rng, n, ws):
    words = n // ws + 1
    a = np.empty(words, dtype=np.uint32)
    i = 0
    while i < words:
        ln = int(rng.integers(8, 900))
        kind = int(rng.integers(0, 6))
        if kind == 0:
            seg = np.full(ln, rng.integers(0, 6))                                  # run
        elif kind == 1:
            seg = np.resize(rng.integers(0, 1 << 24, size=int(rng.integers(1, 33))), ln)   # near period
        elif kind == 2:
            seg = np.resize(rng.integers(0, 1 << 24, size=int(rng.integers(33, 300))), ln)  # far period
        elif kind == 3:
            seg = rng.integers(0, int(rng.integers(2, 5)), size=ln)               # small alphabet
        elif kind == 4:
            seg = np.zeros(ln, dtype=np.int64)                                     # zeros
        else:
            seg = rng.integers(0, 1 << 31, size=ln)                                # noise
        a[i:i + ln] = seg[: words - i]
        i += ln
    return a.astype({1: np.uint8, 2: "<u2", 4: "<u4"}[ws]).view(np.uint8)[:n].copy()


def params(i):
    rng = np.random.default_rng(1000 + i)
    cs = int(rng.choice([1024, 2048, 4096]))
    ws = int(rng.choice([1, 2, 4]))
    level = int(rng.integers(0, 2))
    window = int(rng.choice([32, 32, 48, 64]))
    n = int(rng.integers(1, 36 * cs))
    return rng, cs, ws, level, window, n


def gpu_encode(g, data, cs, ws, level, window):
    x = torch.from_numpy(data).to("cuda:0")
    out = torch.zeros(g.max_compressed_size(data.size, cs), dtype=torch.uint8, device="cuda:0")
    nb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
    wsp = torch.empty(max(g.encode_workspace_size(data.size, cs), 1), dtype=torch.uint8, device="cuda:0")
    if window == 32:
        g.encode_into(x, cs, ws, level, out, nb, wsp)
    else:
        g.encode_window_into(x, cs, ws, level, window, out, nb, wsp)
    torch.cuda.synchronize()
    return out, int(nb.item())


@pytest.mark.parametrize("i", range(CASES))
def test_random_case(g, oracle_mod, i):
    rng, cs, ws, level, window, n = params(i)
    data = shaped(rng, n, ws)
    if n > 6 * cs and rng.random() < 0.5:
        c = int(rng.integers(1, n // cs - 1))
        data[c * cs:(c + 1) * cs] = rng.integers(0, 256, size=cs, dtype=np.uint8)  # a raw chunk
    out, nb = gpu_encode(g, data, cs, ws, level, window)
    want = oracle_mod.encode(data, cs, ws, level, window)
    assert nb == want.size and out[:nb].cpu().numpy().tobytes() == want.tobytes(), (cs, ws, level, window, n)
    y, yb, st = g.decode(out, nb, n)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(yb.item()) == n
    assert y[:n].cpu().numpy().tobytes() == data.tobytes()
    if i % 4 == 0:  # split mode, same input
        lit, lens, offs, meta, pb = g.encode_split(torch.from_numpy(data).to("cuda:0"), cs, ws, level)
        torch.cuda.synchronize()
        v = [int(x) for x in pb.cpu().tolist()]
        got = (lit[:v[0]].cpu().numpy().tobytes(), lens[:v[1]].cpu().numpy().tobytes(),
               offs[:v[2]].cpu().numpy().tobytes(), meta[:v[3]].cpu().numpy().tobytes())
        assert got == tuple(p.tobytes() for p in oracle_mod.encode_split(data, cs, ws, level))
    if i % 4 == 1:  # the advancing-search baseline, same input
        x = torch.from_numpy(data).to("cuda:0")
        aout = torch.zeros(g.max_compressed_size(n, cs), dtype=torch.uint8, device="cuda:0")
        anb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
        wsp = torch.empty(max(g.encode_workspace_size(n, cs), 1), dtype=torch.uint8, device="cuda:0")
        g.encode_advancing_into(x, cs, ws, aout, anb, wsp)
        torch.cuda.synchronize()
        want_a = oracle_mod.encode_advancing(data, cs, ws)
        assert aout[: int(anb.item())].cpu().numpy().tobytes() == want_a.tobytes()
