"""GPU parity of the wider near windows (gpulz_encode_window): byte-identical
streams against the oracle's encode at windows 32, 48 and 64, every chunk
size and word size, both match levels, ragged tails; the streams decode
with the ordinary decoder; window 32 is gpulz_encode."""
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


def periodic(rng, n, ws):
    """Segments of periods 1..80 (inside and beyond each window), runs and noise."""
    words = n // ws + 1
    a = np.empty(words, dtype=np.uint32)
    i = 0
    while i < words:
        ln = int(rng.integers(50, 700))
        kind = int(rng.integers(0, 4))
        per = int(rng.integers(1, 81))
        if kind == 0:
            seg = np.resize(rng.integers(0, 1 << 20, size=per), ln)
        elif kind == 1:
            seg = np.full(ln, rng.integers(0, 5))
        elif kind == 2:
            seg = np.resize(rng.integers(0, 4, size=per), ln)
        else:
            seg = rng.integers(0, 1 << 30, size=ln)
        a[i:i + ln] = seg[: words - i]
        i += ln
    return a.astype({1: np.uint8, 2: "<u2", 4: "<u4"}[ws]).view(np.uint8)[:n].copy()


def gpu_encode_window(g, data: np.ndarray, cs, ws, level, window):
    x = torch.from_numpy(data).to("cuda:0")
    cap = g.max_compressed_size(data.size, cs)
    out = torch.zeros(cap, dtype=torch.uint8, device="cuda:0")
    nb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
    wsp = torch.empty(max(g.encode_workspace_size(data.size, cs), 1), dtype=torch.uint8, device="cuda:0")
    g.encode_window_into(x, cs, ws, level, window, out, nb, wsp)
    torch.cuda.synchronize()
    return out[: int(nb.item())].cpu().numpy().tobytes()


@pytest.mark.parametrize("cs", [1024, 2048, 4096])
@pytest.mark.parametrize("ws", [1, 2, 4])
@pytest.mark.parametrize("window", [48, 64])
def test_window_parity(g, oracle_mod, cs, ws, window):
    rng = np.random.default_rng(cs + 10 * ws + window)
    for level in (0, 1):
        for n in [1, cs + 5, 7 * cs + int(rng.integers(1, cs))]:
            data = periodic(rng, n, ws)
            got = gpu_encode_window(g, data, cs, ws, level, window)
            want = oracle_mod.encode(data, cs, ws, level, window).tobytes()
            assert got == want, (cs, ws, level, window, n)
            assert np.array_equal(oracle_mod.decode(np.frombuffer(got, np.uint8)), data)


def test_window_32_is_the_default_encode(g, oracle_mod):
    rng = np.random.default_rng(3)
    data = periodic(rng, 20 * 2048 + 17, 4)
    got = gpu_encode_window(g, data, 2048, 4, 1, 32)
    assert got == oracle_mod.encode(data, 2048, 4, 1).tobytes()


def test_window_streams_decode_on_the_gpu(g, oracle_mod):
    rng = np.random.default_rng(4)
    data = periodic(rng, 40 * 4096 + 3, 4)
    for window in (48, 64):
        s = gpu_encode_window(g, data, 4096, 4, 0, window)
        st = torch.from_numpy(np.frombuffer(s, np.uint8).copy()).to("cuda:0")
        out, nb, status = g.decode(st, len(s))
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert np.array_equal(out[: int(nb.item())].cpu().numpy(), data)
