"""GPU parity of split mode (literals / lengths / offsets / meta ports)
against the CPU oracle, through the C ABI: ports byte-identical to the
oracle's, decodes bit-exact, corrupted ports accepted or rejected exactly as
the oracle does (and decoded identically when accepted)."""
from __future__ import annotations

import struct

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
    g.lib()
    return g


def to_dev(a) -> "torch.Tensor":
    a = np.ascontiguousarray(np.frombuffer(a, dtype=np.uint8) if isinstance(a, (bytes, bytearray)) else a)
    return torch.from_numpy(a.view(np.uint8).reshape(-1).copy()).to("cuda:0")


def gpu_split(g, data, cs, ws, level):
    lit, lens, offs, meta, pb = g.encode_split(to_dev(data), cs, ws, level)
    torch.cuda.synchronize()
    v = [int(x) for x in pb.cpu().tolist()]
    assert v[1] == v[2]
    return (lit[:v[0]].cpu().numpy().tobytes(), lens[:v[1]].cpu().numpy().tobytes(),
            offs[:v[2]].cpu().numpy().tobytes(), meta[:v[3]].cpu().numpy().tobytes())


def gpu_split_decode(g, ports, cap):
    lit, lens, offs, meta = (to_dev(p) for p in ports)
    out, nb, st = g.decode_split(lit, lens, offs, meta, port_bytes=(len(ports[0]), len(ports[1]), len(ports[3])),
                                 out_capacity=cap)
    torch.cuda.synchronize()
    return int(st.item()), int(nb.item()), out.cpu().numpy().tobytes()


SPLIT_CASES = golden_cases.load_split()


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c["name"] for c in SPLIT_CASES])
def test_split_hand_examples(g, case):
    got = gpu_split(g, case["input"], case["cs"], case["ws"], case["level"])
    assert got == (case["lit"], case["lens"], case["offs"], case["meta"])
    st, nb, out = gpu_split_decode(g, got, len(case["input"]))
    assert st == 0 and nb == len(case["input"]) and out == case["input"]


def mixed_bytes(rng, n, ws):
    a = rng.integers(0, 4, size=n // ws + 1).astype(np.uint32)
    a = np.repeat(a, rng.integers(1, 30, size=a.size))[: n // ws + 1]
    noise = rng.random(a.size) < 0.15
    a[noise] = rng.integers(0, 1 << 30, size=int(noise.sum())).astype(np.uint32)
    b = a.astype({1: np.uint8, 2: "<u2", 4: "<u4"}[ws]).view(np.uint8)[:n].copy()
    if n > 3 * 4096:
        b[4096:8192] = 0                                              # zero chunks
        b[8192:12288] = rng.integers(0, 256, size=4096, dtype=np.uint8)  # raw chunks
    return b


@pytest.mark.parametrize("cs", [1024, 2048, 4096])
@pytest.mark.parametrize("ws", [1, 2, 4])
@pytest.mark.parametrize("level", [0, 1])
def test_split_random_ragged(g, oracle_mod, cs, ws, level):
    rng = np.random.default_rng(cs + 13 * ws + level)
    for n in [0, 1, cs - 1, cs + 3, 7 * cs + int(rng.integers(1, cs)), 40 * cs]:
        data = mixed_bytes(rng, n, ws)
        want = tuple(p.tobytes() for p in oracle_mod.encode_split(data, cs, ws, level))
        got = gpu_split(g, data, cs, ws, level)
        assert got == want, (n, [len(p) for p in got], [len(p) for p in want])
        st, nb, out = gpu_split_decode(g, got, n)
        assert st == 0 and nb == n and out == data.tobytes()


@pytest.mark.parametrize("idx,level", [(1, 0), (1, 1), (2, 1), (3, 0)])
def test_split_workloads(g, oracle_mod, idx, level):
    import workloads as synth
    w = synth.workload(idx)
    want = tuple(p.tobytes() for p in oracle_mod.encode_split(w.data, w.chunk_size, w.word_size, level))
    got = gpu_split(g, w.data, w.chunk_size, w.word_size, level)
    assert got == want
    st, nb, out = gpu_split_decode(g, got, w.n)
    assert st == 0 and nb == w.n and out == w.data.tobytes()


def test_split_corrupted_ports_match_oracle(g, oracle_mod):
    """Random byte changes in every port, header edits and short ports: the
    GPU rejects exactly what the oracle rejects and decodes the rest alike."""
    rng = np.random.default_rng(5)
    data = mixed_bytes(rng, 20 * 2048 + 77, 4)
    ports = [p.tobytes() for p in oracle_mod.encode_split(data, 2048, 4, 1)]
    n = data.size
    trials = []
    for _ in range(120):
        which = int(rng.integers(0, 4))
        if not ports[which]:
            continue
        mod = [bytearray(p) for p in ports]
        i = int(rng.integers(0, len(mod[which])))
        mod[which][i] ^= int(rng.integers(1, 256))
        if which == 1:  # keep lengths and offsets the same length
            pass
        trials.append([bytes(m) for m in mod])
    for cut in range(4):  # shorter ports
        mod = list(ports)
        if cut == 1 or cut == 2:
            mod[1], mod[2] = mod[1][:-1], mod[2][:-1]
        else:
            mod[cut] = mod[cut][:-1]
        trials.append(mod)
    for t in trials:
        r, want = oracle_mod.decode_split_status(*t, cap=n)
        st, nb, out = gpu_split_decode(g, t, n)
        if r >= 0:
            assert st == 0 and nb == n and out == want.tobytes()
        else:
            assert st != 0 and nb == 0


@pytest.mark.parametrize("level", [1, 0])
def test_split_stress_2gib_whole_ports(g, oracle_mod, level):
    """The 2 GiB stress stream in split mode: all four GPU ports equal the
    oracle's byte for byte (the oracle run on contiguous whole-chunk ranges
    across the host's cores), and the GPU decodes all of it."""
    import workloads as synth
    w = synth.workload(4)
    cs, ws = w.chunk_size, w.word_size
    print(f"split stress 2 GiB level {level}: GPU encode", flush=True)
    x = to_dev(w.data)
    lit, lens, offs, meta, pb = g.encode_split(x, cs, ws, level)
    torch.cuda.synchronize()
    nl, nt, no, nm = [int(v) for v in pb.cpu().tolist()]
    assert nm > 0 and nt == no
    print(f"split stress 2 GiB level {level}: oracle on host threads", flush=True)
    want = oracle_mod.encode_split_parallel(w.data, cs, ws, level)
    assert (nl, nt, nt, nm) == tuple(int(p.size) for p in want)
    for dev_port, n_, ref in zip((lit, lens, offs, meta), (nl, nt, nt, nm), want):
        assert np.array_equal(dev_port[:n_].cpu().numpy(), ref)
    del want
    print(f"split stress 2 GiB level {level}: GPU decode", flush=True)
    out, nb, st = g.decode_split(lit, lens, offs, meta, port_bytes=(nl, nt, nm), out_capacity=w.n)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(nb.item()) == w.n
    assert torch.equal(out, x)
