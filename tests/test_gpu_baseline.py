"""GPU parity of the one-thread-per-chunk baseline decoder
(gpulz_decode_one_thread_per_chunk): bit-exact decodes of oracle streams and
the same status as the oracle on corrupted ones."""
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


def serial_decode(g, stream: bytes, cap: int):
    s = torch.from_numpy(np.frombuffer(stream, dtype=np.uint8).copy()).to("cuda:0")
    out = torch.zeros(max(cap, 1), dtype=torch.uint8, device="cuda:0")[:cap]
    nb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
    st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(max(g.decode_workspace_size(len(stream)), 1), dtype=torch.uint8, device="cuda:0")
    g.decode_one_thread_per_chunk_into(s, len(stream), out, nb, st, ws)
    torch.cuda.synchronize()
    return int(st.item()), int(nb.item()), out.cpu().numpy().tobytes()


def mixed(rng, n, ws):
    a = rng.integers(0, 4, size=n // ws + 1).astype(np.uint32)
    a = np.repeat(a, rng.integers(1, 30, size=a.size))[: n // ws + 1]
    noise = rng.random(a.size) < 0.2
    a[noise] = rng.integers(0, 1 << 30, size=int(noise.sum())).astype(np.uint32)
    return a.astype({1: np.uint8, 2: "<u2", 4: "<u4"}[ws]).view(np.uint8)[:n].copy()


@pytest.mark.parametrize("cs", [1024, 2048, 4096])
@pytest.mark.parametrize("ws", [1, 2, 4])
def test_serial_decode_matches(g, oracle_mod, cs, ws):
    rng = np.random.default_rng(cs + ws)
    for level in (0, 1):
        for n in [0, 1, cs + 3, 9 * cs + int(rng.integers(1, cs))]:
            data = mixed(rng, n, ws)
            if n > 3 * cs:
                data[cs:2 * cs] = 0
                data[2 * cs:3 * cs] = rng.integers(0, 256, size=cs, dtype=np.uint8)
            s = oracle_mod.encode(data, cs, ws, level).tobytes()
            st, nb, out = serial_decode(g, s, n)
            assert st == 0 and nb == n and out == data.tobytes()


def test_serial_decode_workload(g, oracle_mod):
    import workloads as synth
    w = synth.workload(1)
    s = oracle_mod.encode(w.data, w.chunk_size, w.word_size, 0).tobytes()
    st, nb, out = serial_decode(g, s, w.n)
    assert st == 0 and nb == w.n and out == w.data.tobytes()


def test_serial_decode_corrupted_matches_oracle(g, oracle_mod):
    rng = np.random.default_rng(3)
    data = mixed(rng, 12 * 2048 + 11, 4)
    s = bytearray(oracle_mod.encode(data, 2048, 4, 1).tobytes())
    for _ in range(80):
        t = bytearray(s)
        i = int(rng.integers(32, len(t)))
        t[i] ^= int(rng.integers(1, 256))
        r, want = oracle_mod.decode_status(bytes(t), cap=data.size)
        st, nb, out = serial_decode(g, bytes(t), data.size)
        if r >= 0:
            assert st == 0 and out == want.tobytes()
        else:
            assert st != 0 and nb == 0
