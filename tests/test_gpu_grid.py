"""GPU checks of the chunk kernels' grid striding: streams with more chunks
than the decode grid has workgroups, for chunks decoded by a whole
workgroup (word size 1 or 2 at chunk 4096: up to 16384 workgroups, one
chunk each) and for chunks shared by waves (word size 4 at chunk 2048:
8192 workgroups of four waves), so that workgroups and waves take several
chunks each.  A sample of size-table rows and payloads equals the oracle's
chunk encoder, the table is consistent, and the decode is bit-exact."""
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


def data_of(rng, n):
    """Segments of 1-64 KiB: short periods, a small alphabet, noise, zeros."""
    a = np.empty(n, np.uint8)
    i = 0
    while i < n:
        ln = int(rng.integers(1 << 10, 1 << 16))
        k = int(rng.integers(0, 4))
        if k == 0:
            seg = np.resize(rng.integers(0, 256, size=int(rng.integers(1, 300)), dtype=np.uint8), ln)
        elif k == 1:
            seg = rng.integers(0, 3, size=ln, dtype=np.uint8)
        elif k == 2:
            seg = rng.integers(0, 256, size=ln, dtype=np.uint8)
        else:
            seg = np.zeros(ln, np.uint8)
        a[i:i + ln] = seg[: n - i]
        i += ln
    return a


@pytest.mark.parametrize("cs,ws,chunks,level", [(4096, 1, 16384 + 3111, 0), (4096, 2, 16384 + 517, 1),
                                                (2048, 4, 8192 * 4 * 2 + 77, 0)])
def test_more_chunks_than_workgroups(g, oracle_mod, cs, ws, chunks, level):
    rng = np.random.default_rng(chunks)
    n = (chunks - 1) * cs + 1 + int(rng.integers(0, cs - 1))
    data = data_of(rng, n)
    x = torch.from_numpy(data).to("cuda:0")
    out, nb = g.encode(x, cs, ws, level)
    torch.cuda.synchronize()
    total = int(nb.item())
    assert g.stream_info(out[:32].cpu().numpy().tobytes()) == (n, total, cs, ws)
    table = out[32:32 + 8 * chunks].cpu().numpy().view("<u4").reshape(chunks, 2).astype(np.int64)
    f, d = table[:, 0], table[:, 1]
    sizes = np.where(f > 0, f + d, np.where(d & 0x80000000, d & 0x7FFFFFFF, 0))
    offs = np.concatenate([[0], np.cumsum(sizes)])
    assert 32 + 8 * chunks + offs[-1] == total
    sample = np.unique(np.concatenate([np.arange(8), rng.integers(0, chunks, size=300), [chunks - 1]]))
    base = 32 + 8 * chunks
    for c in sample:
        ef, ed, pay = oracle_mod.encode_chunk(data[c * cs: min((c + 1) * cs, n)], cs, ws, level)
        assert (int(f[c]), int(d[c])) == (ef, ed), c
        lo = base + int(offs[c])
        assert out[lo:lo + len(pay)].cpu().numpy().tobytes() == pay, c
    dec, db, st = g.decode(out[:total], out_capacity=n)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(db.item()) == n
    assert torch.equal(dec, x)
