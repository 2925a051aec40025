"""GPU checks of the timed entry points (gpulz_encode_timed,
gpulz_decode_timed), the ones the benchmark's kernel-time pass calls: the
same stream as gpulz_encode byte for byte (and so as the oracle's), the
same decode, and both events recorded around a launch (a positive elapsed
time).  Cases: the 1800 x 3600 Lorenzo field at chunk 2048 (both levels),
ragged inputs that take the one-wave decode, the workgroup decode and the
one-slot decode of 1024-element chunks, and an empty input."""
from __future__ import annotations

import ctypes

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


@pytest.fixture(scope="module")
def hip():
    h = ctypes.CDLL("libamdhip64.so.7")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    made = []

    def pair():
        evs = []
        for _ in range(2):
            e = ctypes.c_void_p()
            assert h.hipEventCreate(ctypes.byref(e)) == 0
            made.append(e)
            evs.append(e)
        return tuple(evs)

    def ms(p):
        f = ctypes.c_float()
        assert h.hipEventElapsedTime(ctypes.byref(f), p[0], p[1]) == 0
        return float(f.value)

    yield pair, ms
    torch.cuda.synchronize()
    for e in made:
        h.hipEventDestroy(e)


def run(g, hip, data: np.ndarray, cs, ws, level):
    pair, ms = hip
    n = data.size
    x = torch.from_numpy(data).to("cuda:0")
    cap = g.max_compressed_size(n, cs)
    ews = torch.empty(max(g.encode_workspace_size(n, cs), 1), dtype=torch.uint8, device="cuda:0")
    plain = torch.zeros(cap, dtype=torch.uint8, device="cuda:0")
    pnb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
    g.encode_into(x, cs, ws, level, plain, pnb, ews)
    timed = torch.full((cap,), 0xA5, dtype=torch.uint8, device="cuda:0")
    tnb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
    ke = pair()
    g.encode_into(x, cs, ws, level, timed, tnb, ews, events=ke)
    torch.cuda.synchronize()
    nb = int(pnb.item())
    assert int(tnb.item()) == nb
    assert torch.equal(timed[:nb], plain[:nb])
    assert ms(ke) > 0.0
    dws = torch.empty(max(g.decode_workspace_size(nb), 1), dtype=torch.uint8, device="cuda:0")
    y = torch.full((max(n, 1),), 0x5A, dtype=torch.uint8, device="cuda:0")
    yb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
    st = torch.full((1,), 77, dtype=torch.int32, device="cuda:0")
    kd = pair()
    g.decode_into(timed, nb, y, yb, st, dws, events=kd)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(yb.item()) == n
    assert y[:n].cpu().numpy().tobytes() == data.tobytes()
    assert ms(kd) > 0.0
    return timed[:nb].cpu().numpy().tobytes()


@pytest.mark.parametrize("level", [0, 1])
def test_timed_workload_1800x3600(g, hip, oracle_mod, level):
    import workloads as synth
    w = synth.workload(1)
    data = np.ascontiguousarray(w.data)
    got = run(g, hip, data, w.chunk_size, w.word_size, level)
    assert got == oracle_mod.encode(data, w.chunk_size, w.word_size, level).tobytes()


@pytest.mark.parametrize("cs,ws,chunks", [(2048, 4, 37), (4096, 1, 9), (4096, 4, 2050)])
def test_timed_ragged(g, hip, oracle_mod, cs, ws, chunks):
    rng = np.random.default_rng(cs + 10 * ws + chunks)
    n = (chunks - 1) * cs + int(rng.integers(1, cs))
    per = rng.integers(0, 1 << 16, size=int(rng.integers(2, 40))).astype(np.uint32)
    data = np.resize(per, n // 4 + 1).view(np.uint8)[:n].copy()
    data[rng.random(n) < 0.02] ^= 0x3C                           # sparse breaks in the pattern
    data[cs:2 * cs] = 0                                           # a zero chunk
    data[2 * cs:3 * cs] = rng.integers(0, 256, size=cs, dtype=np.uint8)  # a raw chunk
    got = run(g, hip, data, cs, ws, chunks % 2)
    assert got == oracle_mod.encode(data, cs, ws, chunks % 2).tobytes()


def test_timed_empty(g, hip, oracle_mod):
    data = np.zeros(0, np.uint8)
    got = run(g, hip, data, 2048, 4, 0)
    assert got == oracle_mod.encode(data, 2048, 4, 0).tobytes()
