"""gpulz_decode_noalloc (the decode entry point that allocates nothing, its
workspace a static device array) against gpulz_decode with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller
stream, then corrupted and too-small-output cases; every result equals the
allocating decode's (status, length, output bytes) and the input."""
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


def _both(g, stream: np.ndarray, cap: int, poison: int):
    """Decode with gpulz_decode (its own workspace) and gpulz_decode_noalloc;
    returns ((status, length, bytes), (status, length, bytes))."""
    dev = torch.device("cuda:0")
    xs = torch.from_numpy(stream.copy()).to(dev)
    res = []
    for noalloc in (False, True):
        out = torch.full((max(cap, 1),), poison, dtype=torch.uint8, device=dev)[:cap]
        nb = torch.full((1,), 77, dtype=torch.uint64, device=dev)
        st = torch.full((1,), 99, dtype=torch.int32, device=dev)
        print(f"decode {'noalloc' if noalloc else 'workspace'}: {stream.size} stream bytes, cap {cap}", flush=True)
        if noalloc:
            g.decode_noalloc_into(xs, stream.size, out, nb, st)
        else:
            wsb = torch.full((g.decode_workspace_size(stream.size),), poison ^ 0x5A, dtype=torch.uint8, device=dev)
            g.decode_into(xs, stream.size, out, nb, st, wsb)
        torch.cuda.synchronize()
        res.append((int(st.item()), int(nb.item()), out.cpu().numpy()))
    return res


def test_noalloc_matches_workspace_decode_twice_then_smaller(g, oracle_mod):
    import workloads
    big = workloads.workload(1)  # 1800x3600 field, chunk 2048, word 4
    rng = np.random.default_rng(21)
    small = np.resize(rng.integers(0, 7, size=3001, dtype=np.uint8), 37 * 4096 + 999)
    cases = [(big.data, 2048, 4, 0), (small, 4096, 1, 1)]
    for k, (data, cs, ws, level) in enumerate(cases):
        s = oracle_mod.encode(data, cs, ws, level)
        a, b = _both(g, s, data.size, poison=0x11 * (k + 1))
        assert a[0] == 0 and a[1] == data.size and np.array_equal(a[2], data)
        assert b[0] == a[0] and b[1] == a[1] and np.array_equal(b[2], a[2])


def test_noalloc_error_statuses_match(g, oracle_mod):
    data = np.tile(np.array([1, 2, 3, 4, 1, 2, 3, 4, 9], dtype="<u4"), 2000).view(np.uint8)
    s = oracle_mod.encode(data, 2048, 4, 0)
    rng = np.random.default_rng(8)
    trials = [s[:-1].copy(), s[:40].copy()]
    for _ in range(40):
        t = s.copy()
        i = int(rng.integers(0, t.size))
        t[i] ^= np.uint8(1 << int(rng.integers(0, 8)))
        trials.append(t)
    for t in trials:
        a, b = _both(g, t, data.size + 64, poison=0x3C)
        assert (b[0], b[1]) == (a[0], a[1])
        if a[0] == 0:
            assert np.array_equal(b[2][:a[1]], a[2][:a[1]])
    # output smaller than the stream's original size: capacity status, nothing written
    a, b = _both(g, s, data.size - 1, poison=0x6B)
    assert a[0] == b[0] == g.STATUS_CAPACITY and a[1] == b[1] == 0
    assert (b[2] == 0x6B).all()
