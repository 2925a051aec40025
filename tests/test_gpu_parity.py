"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Streams must be byte-identical to the oracle's and every decode bit-exact.
Covers the hand-worked streams, all (chunk_size, word_size, level) pairs on
ragged inputs, the five workloads (full size for the field workloads and the
byte mix; the 2 GiB stress stream whole, against the oracle run on chunk
ranges across the host's cores),
corrupted streams, capacity errors, unaligned buffers, poisoned workspace.
"""
from __future__ import annotations

import numpy as np
import pytest

import golden_cases

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunked_lzss_coder_amd as g
    g.lib()  # raises if the HIP library is not built
    return g


def to_dev(a: np.ndarray):
    return torch.from_numpy(np.array(a, copy=True)).to("cuda:0")  # a writable, contiguous copy


def gpu_encode(g, data: np.ndarray, cs: int, ws: int, level: int) -> np.ndarray:
    out, nb = g.encode(to_dev(data), cs, ws, level)
    torch.cuda.synchronize()
    n = int(nb.item())
    return out[:n].cpu().numpy()


def gpu_decode(g, stream: np.ndarray, cap: int):
    out, nb, st = g.decode(to_dev(stream), out_capacity=cap)
    torch.cuda.synchronize()
    return int(st.item()), int(nb.item()), out.cpu().numpy()


CASES = golden_cases.load()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_examples(g, case):
    data = np.frombuffer(case["input"], dtype=np.uint8)
    got = gpu_encode(g, data, case["cs"], case["ws"], case["level"])
    assert got.tobytes() == case["stream"]
    st, nb, out = gpu_decode(g, np.frombuffer(case["stream"], dtype=np.uint8), len(case["input"]))
    assert st == 0 and nb == len(case["input"])
    assert out.tobytes() == case["input"]


def structured_bytes(rng, n, ws):
    kind = rng.integers(0, 4)
    if kind == 0:
        a = rng.integers(0, 3, size=n // ws + 1).astype(np.uint32)
        a = np.repeat(a, rng.integers(1, 40, size=a.size))[: n // ws + 1]
    elif kind == 1:
        per = int(rng.integers(1, 300))
        a = np.resize(rng.integers(0, 1 << 30, size=per), n // ws + 1).astype(np.uint32)
    elif kind == 2:
        a = rng.integers(0, 1 << 32, size=n // ws + 1, dtype=np.uint64).astype(np.uint32)
    else:
        a = rng.integers(0, 6, size=n // ws + 1).astype(np.uint32)
    b = a.astype({1: np.uint8, 2: "<u2", 4: "<u4"}[ws]).view(np.uint8)
    return np.ascontiguousarray(b[:n])


@pytest.mark.parametrize("cs", [1024, 2048, 4096])
@pytest.mark.parametrize("ws", [1, 2, 4])
@pytest.mark.parametrize("level", [0, 1])
def test_random_ragged_inputs(g, oracle_mod, cs, ws, level):
    rng = np.random.default_rng(cs * 31 + ws * 7 + level)
    sizes = [0, 1, 5, cs - 1, cs, cs + 3, 7 * cs + int(rng.integers(1, cs)), 40 * cs]
    for n in sizes:
        data = structured_bytes(rng, n, ws)
        ref = oracle_mod.encode(data, cs, ws, level)
        got = gpu_encode(g, data, cs, ws, level)
        assert got.size == ref.size and np.array_equal(got, ref), (n, got.size, ref.size)
        st, nb, out = gpu_decode(g, got, n)
        assert st == 0 and nb == n and np.array_equal(out[:n], data)


@pytest.fixture(scope="module")
def workloads():
    import workloads as synth
    cache = {}

    def get(idx):
        if idx not in cache:
            cache.clear()
            cache[idx] = synth.workload(idx)
        return cache[idx]
    return get


@pytest.mark.parametrize("idx,level", [(0, 0), (1, 0), (1, 1), (2, 1), (3, 0), (3, 1)])
def test_workload_full_stream(g, oracle_mod, workloads, idx, level):
    w = workloads(idx)
    ref = oracle_mod.encode(w.data, w.chunk_size, w.word_size, level)
    got = gpu_encode(g, w.data, w.chunk_size, w.word_size, level)
    assert got.size == ref.size
    assert np.array_equal(got, ref)
    st, nb, out = gpu_decode(g, got, w.n)
    assert st == 0 and nb == w.n and np.array_equal(out, w.data)


@pytest.mark.parametrize("level", [1, 0])
def test_stress_2gib_whole_stream(g, oracle_mod, workloads, level):
    """2 GiB stress stream at its full size: the whole GPU stream (header,
    every size-table row, every payload byte) equals the oracle's, which is
    built from the single-threaded oracle run on contiguous whole-chunk ranges
    across the host's cores; the GPU decode reproduces all 2 GiB."""
    w = workloads(4)
    cs, ws = w.chunk_size, w.word_size
    print(f"stress 2 GiB level {level}: GPU encode", flush=True)
    x = to_dev(w.data)
    out, nb = g.encode(x, cs, ws, level)
    torch.cuda.synchronize()
    total = int(nb.item())
    assert total > 0
    got = out[:total].cpu().numpy()
    print(f"stress 2 GiB level {level}: oracle on host threads", flush=True)
    ref = oracle_mod.encode_parallel(w.data, cs, ws, level)
    assert got.size == ref.size
    assert np.array_equal(got, ref)
    del got, ref
    print(f"stress 2 GiB level {level}: GPU decode", flush=True)
    dec, db, st = g.decode(out[:total], out_capacity=w.n)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(db.item()) == w.n
    assert torch.equal(dec, x)


def test_decode_oracle_streams_all_levels(g, oracle_mod):
    import workloads as synth
    w = synth.workload(0)
    for level in (0, 1):
        s = oracle_mod.encode(w.data, w.chunk_size, w.word_size, level)
        st, nb, out = gpu_decode(g, s, w.n)
        assert st == 0 and np.array_equal(out, w.data)


def test_deterministic_with_poisoned_workspace(g):
    import workloads as synth
    w = synth.workload(0)
    x = to_dev(w.data)
    ref = None
    for trial in range(5):
        cap = g.max_compressed_size(w.n, 2048)
        out = torch.full((cap,), 0xA5, dtype=torch.uint8, device="cuda:0")
        nb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
        wsb = torch.full((g.encode_workspace_size(w.n, 2048),), 0xA5 ^ trial, dtype=torch.uint8, device="cuda:0")
        g.encode_into(x, 2048, 4, 1, out, nb, wsb)
        torch.cuda.synchronize()
        s = out[:int(nb.item())].cpu().numpy()
        if ref is None:
            ref = s
        assert np.array_equal(s, ref)
        assert (out[int(nb.item()):].cpu().numpy() == 0xA5).all()  # nothing written past the stream


def test_unaligned_buffers(g, oracle_mod):
    rng = np.random.default_rng(4)
    data = structured_bytes(rng, 3 * 2048 + 77, 4)
    ref = oracle_mod.encode(data, 2048, 4, 1)
    for shift_in in (1, 2, 3):
        for shift_out in (0, 1, 3):
            xin = torch.zeros(data.size + 16, dtype=torch.uint8, device="cuda:0")
            xin[shift_in:shift_in + data.size] = to_dev(data)
            cap = g.max_compressed_size(data.size, 2048)
            obuf = torch.zeros(cap + 16, dtype=torch.uint8, device="cuda:0")
            nb = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
            wsz = g.encode_workspace_size(data.size, 2048)
            wsb = torch.empty(wsz + 8, dtype=torch.uint8, device="cuda:0")[shift_in:shift_in + wsz]  # unaligned too
            g.encode_into(xin[shift_in:shift_in + data.size], 2048, 4, 1, obuf[shift_out:shift_out + cap], nb, wsb)
            torch.cuda.synchronize()
            n = int(nb.item())
            assert np.array_equal(obuf[shift_out:shift_out + n].cpu().numpy(), ref)
            # decode from an unaligned stream into an unaligned output
            sbuf = torch.zeros(n + 16, dtype=torch.uint8, device="cuda:0")
            sbuf[shift_in:shift_in + n] = obuf[shift_out:shift_out + n]
            dbuf = torch.zeros(data.size + 16, dtype=torch.uint8, device="cuda:0")
            db = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
            st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
            dsz = g.decode_workspace_size(n)
            dws = torch.empty(dsz + 8, dtype=torch.uint8, device="cuda:0")[shift_out + 1:shift_out + 1 + dsz]
            g.decode_into(sbuf[shift_in:shift_in + n], n, dbuf[shift_out:shift_out + data.size], db, st, dws)
            torch.cuda.synchronize()
            assert int(st.item()) == 0
            assert np.array_equal(dbuf[shift_out:shift_out + data.size].cpu().numpy(), data)


def test_capacity_error_writes_nothing(g, oracle_mod):
    data = np.tile(np.arange(7, dtype="<u4"), 1000).view(np.uint8)
    s = oracle_mod.encode(data, 2048, 4, 0)
    xs = to_dev(s)
    dbuf = torch.full((data.size + 64,), 0x5A, dtype=torch.uint8, device="cuda:0")
    db = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
    st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    dws = torch.empty(g.decode_workspace_size(s.size), dtype=torch.uint8, device="cuda:0")
    g.decode_into(xs, s.size, dbuf[:data.size - 1], db, st, dws)
    torch.cuda.synchronize()
    assert int(st.item()) == g.STATUS_CAPACITY and int(db.item()) == 0
    assert (dbuf.cpu().numpy() == 0x5A).all()


def test_corrupted_streams(g, oracle_mod):
    data = np.tile(np.array([1, 2, 3, 4, 1, 2, 3, 4, 9], dtype="<u4"), 2000).view(np.uint8)
    s = oracle_mod.encode(data, 2048, 4, 0)
    rng = np.random.default_rng(12)
    trials = []
    for _ in range(300):
        t = s.copy()
        i = int(rng.integers(0, t.size))
        t[i] ^= np.uint8(1 << int(rng.integers(0, 8)))
        trials.append(t)
    trials.append(s[:-1].copy())   # truncated
    trials.append(s[:40].copy())
    for t in trials:
        r, ref_out = oracle_mod.decode_status(t, data.size + 64)
        xs = to_dev(t)
        dbuf = torch.zeros(data.size + 64, dtype=torch.uint8, device="cuda:0")
        db = torch.zeros(1, dtype=torch.uint64, device="cuda:0")
        st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        dws = torch.empty(g.decode_workspace_size(t.size), dtype=torch.uint8, device="cuda:0")
        g.decode_into(xs, t.size, dbuf, db, st, dws)
        torch.cuda.synchronize()
        status = int(st.item())
        if r == oracle_mod.ECAP:  # a flipped size field asks for more than the buffer
            assert status == g.STATUS_CAPACITY and int(db.item()) == 0
        elif r < 0:
            assert status == g.STATUS_CORRUPT and int(db.item()) == 0
        else:  # the flip produced another valid stream: same result as the oracle
            assert status == 0 and int(db.item()) == r
            assert np.array_equal(dbuf[:r].cpu().numpy(), ref_out)


def test_many_one_wave_chunks(g, oracle_mod):
    """A stream of 33,000 chunks of 4096 bytes at word size 4 (enough that
    each chunk is decoded by one wave, its payload staged over its decoded
    bytes): the oracle's stream decodes to the input, and corrupting one
    coded chunk's match token gives the oracle's status."""
    import workloads as synth
    cs, ws = 4096, 4
    n = 33000 * cs - 1000  # ragged tail
    w = synth.workload(4, scale_bytes=n + 1000)
    data = w.data[:n].copy()
    stream = oracle_mod.encode(data, cs, ws, 0)
    st, nb, out = gpu_decode(g, stream, n)
    assert st == 0 and nb == n and np.array_equal(out, data)
    # first coded chunk with a match: zero its first match's offset byte
    chunks = -(-n // cs)
    table = stream[32:32 + 8 * chunks].view("<u4").reshape(chunks, 2).astype(np.int64)
    f, d = table[:, 0], table[:, 1]
    sizes = np.where(f > 0, f + d, np.where(d & 0x80000000, d & 0x7FFFFFFF, 0))
    offs = 32 + 8 * chunks + np.concatenate([[0], np.cumsum(sizes)])
    bad = stream.copy()
    hit = False
    for c in np.flatnonzero(f > 0)[5000:]:
        pay = bad[offs[c]: offs[c] + sizes[c]]
        F = int(f[c])
        k, pos = 0, F
        while pos < pay.size and k < 8 * F:
            if (pay[k >> 3] >> (k & 7)) & 1:
                pay[pos + 1] = 0  # offset 0 is never valid
                hit = True
                break
            pos += ws
            k += 1
        if hit:
            bad[offs[c]: offs[c] + sizes[c]] = pay
            break
    assert hit
    want, _ = oracle_mod.decode_status(bad, n)
    assert want == oracle_mod.ECORRUPT
    st, nb, _ = gpu_decode(g, bad, n)
    assert st == 3 and nb == 0
