"""GPU tests of the boundary's stream contract, through the C ABI:

* both calls can be captured into a HIP graph (launch shapes depend only on
  host-visible sizes, the header is read on the device, nothing waits on the
  host) and every replay on fresh input gives the oracle's stream and an exact
  decode (GPULZStage page, CUDA-graph paragraph: the page's own inverse reads
  the header on the host and so cannot be captured);
* level-1 output is deterministic over 100 runs (hashed-table paragraph: the
  bucket keeps the largest position+1, whatever the insert order);
* two streams of the default priority running encodes and decodes side by
  side give the serial results byte for byte;
* the allocating wrappers on a stream other than the current one keep their
  workspaces and temporaries on that stream.
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


def field_bytes(idx):
    import workloads
    return workloads.workload(idx)


def to_dev(a):
    return torch.from_numpy(np.array(a, copy=True)).to("cuda:0")


@pytest.mark.parametrize("level", [0, 1])
def test_graph_capture_encode_decode(g, oracle_mod, level):
    """Capture encode_into + decode_into once, replay on three different inputs
    of the same size (copied into the captured input buffer between replays,
    with eager work and synchronizations in between), check every replay."""
    cs, ws = 2048, 4
    w = field_bytes(0)  # 1 MiB of Lorenzo codes
    n = 300 * cs + 1234  # ragged tail
    rng = np.random.default_rng(40 + level)
    inputs = [w.data[:n].copy(), np.roll(w.data, 777)[:n].copy(),
              np.resize(rng.integers(0, 9, size=5000, dtype=np.uint8), n)]
    dev = torch.device("cuda:0")
    x = torch.empty(n, dtype=torch.uint8, device=dev)
    cap = g.max_compressed_size(n, cs)
    out = torch.zeros(cap, dtype=torch.uint8, device=dev)
    nb = torch.zeros(1, dtype=torch.uint64, device=dev)
    ews = torch.empty(g.encode_workspace_size(n, cs), dtype=torch.uint8, device=dev)
    dout = torch.zeros(n, dtype=torch.uint8, device=dev)
    dnb = torch.zeros(1, dtype=torch.uint64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    dws = torch.empty(g.decode_workspace_size(cap), dtype=torch.uint8, device=dev)
    x.copy_(to_dev(inputs[0]))
    # warm up on a side stream, as torch's capture wants
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.encode_into(x, cs, ws, level, out, nb, ews)
        g.decode_into(out, cap, dout, dnb, st, dws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        # in_bytes = the buffer's capacity: the stream's own length is only
        # known on the device, where the decoder reads it from the header
        g.encode_into(x, cs, ws, level, out, nb, ews)
        g.decode_into(out, cap, dout, dnb, st, dws)
    for rep in range(2):
        for data in inputs:
            x.copy_(to_dev(data))
            dout.fill_(0xEE)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            k = int(nb.item())
            ref = oracle_mod.encode(data, cs, ws, level)
            assert k == ref.size, (rep, k, ref.size)
            assert np.array_equal(out[:k].cpu().numpy(), ref)
            assert int(st.item()) == 0 and int(dnb.item()) == n
            assert np.array_equal(dout.cpu().numpy(), data)
            # eager work between replays on the same buffers
            g.encode_into(x, cs, ws, 1 - level, out, nb, ews)
            torch.cuda.synchronize()


def test_level1_deterministic_100_runs(g, oracle_mod):
    """The 1800x3600 field at level 1, 100 encodes with the workspace refilled
    with a different byte before each: every stream equals the first, which
    equals the oracle's."""
    w = field_bytes(1)
    cs, ws = w.chunk_size, w.word_size
    x = to_dev(w.data)
    dev = x.device
    cap = g.max_compressed_size(w.n, cs)
    out = torch.empty(cap, dtype=torch.uint8, device=dev)
    nb = torch.zeros(1, dtype=torch.uint64, device=dev)
    ews = torch.empty(g.encode_workspace_size(w.n, cs), dtype=torch.uint8, device=dev)
    g.encode_into(x, cs, ws, 1, out, nb, ews)
    torch.cuda.synchronize()
    k = int(nb.item())
    first = out[:k].clone()
    ref = oracle_mod.encode(w.data, cs, ws, 1)
    assert k == ref.size and np.array_equal(first.cpu().numpy(), ref)
    same = 0
    for i in range(100):
        ews.fill_((i * 37) & 0xFF)
        out.fill_(i & 0xFF)
        g.encode_into(x, cs, ws, 1, out, nb, ews)
        same += int(bool(torch.equal(out[:k], first)) and int(nb.item()) == k)
    assert same == 100


def test_two_streams_side_by_side(g, oracle_mod):
    """Encodes and decodes of two inputs on two default-priority streams at
    once, several rounds, give the serial streams and exact decodes."""
    a = field_bytes(0).data
    b = np.roll(field_bytes(0).data, 4099)
    cs, ws = 2048, 4
    dev = torch.device("cuda:0")
    want = {}
    for name, data, level in (("a", a, 0), ("b", b, 1)):
        want[name] = oracle_mod.encode(data, cs, ws, level)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    bufs = {}
    for name, data, level, s in (("a", a, 0, s1), ("b", b, 1, s2)):
        n = data.size
        cap = g.max_compressed_size(n, cs)
        bufs[name] = dict(x=to_dev(data), level=level, s=s, n=n, cap=cap,
                          out=torch.empty(cap, dtype=torch.uint8, device=dev),
                          nb=torch.zeros(1, dtype=torch.uint64, device=dev),
                          ews=torch.empty(g.encode_workspace_size(n, cs), dtype=torch.uint8, device=dev),
                          dout=torch.empty(n, dtype=torch.uint8, device=dev),
                          dnb=torch.zeros(1, dtype=torch.uint64, device=dev),
                          st=torch.zeros(1, dtype=torch.int32, device=dev),
                          dws=torch.empty(g.decode_workspace_size(cap), dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    for rnd in range(5):
        for name in ("a", "b"):
            B = bufs[name]
            B["out"].fill_(rnd)
            B["dout"].fill_(rnd)
        torch.cuda.synchronize()
        for _ in range(3):  # interleave the enqueues of the two streams
            for name in ("a", "b"):
                B = bufs[name]
                g.encode_into(B["x"], cs, ws, B["level"], B["out"], B["nb"], B["ews"], stream=B["s"])
            for name in ("a", "b"):
                B = bufs[name]
                g.decode_into(B["out"], B["cap"], B["dout"], B["dnb"], B["st"], B["dws"], stream=B["s"])
        torch.cuda.synchronize()
        for name, data in (("a", a), ("b", b)):
            B = bufs[name]
            k = int(B["nb"].item())
            assert k == want[name].size
            assert np.array_equal(B["out"][:k].cpu().numpy(), want[name])
            assert int(B["st"].item()) == 0 and int(B["dnb"].item()) == B["n"]
            assert torch.equal(B["dout"], B["x"])


def test_allocating_wrappers_on_a_side_stream(g, oracle_mod):
    """encode / decode / encode_split / decode_split with stream= a non-current
    stream, a non-contiguous input, and allocation churn on the current stream
    right after each call returns: results equal the oracle's."""
    w = field_bytes(0)
    cs, ws = 2048, 4
    words = torch.from_numpy(w.data.view("<u4").astype(np.int64)).to("cuda:0")
    strided = words.view(-1, 2)[:, 0]  # every other word: a non-contiguous int64 view
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    want_in = strided.cpu().numpy().astype("<i8").view(np.uint8)
    want = oracle_mod.encode(want_in, cs, ws, 1)
    out, nb = g.encode(strided, cs, ws, 1, stream=side)
    junk = [torch.full((1 << 20,), i, dtype=torch.uint8, device="cuda:0") for i in range(32)]
    del junk
    side.synchronize()
    k = int(nb.item())
    assert k == want.size and np.array_equal(out[:k].cpu().numpy(), want)
    dec, dnb, st = g.decode(out, k, stream=side)
    junk = [torch.full((1 << 20,), i, dtype=torch.uint8, device="cuda:0") for i in range(32)]
    del junk
    side.synchronize()
    assert int(st.item()) == 0 and np.array_equal(dec.cpu().numpy(), want_in)
    lit, lens, offs, meta, pb = g.encode_split(strided, cs, ws, 0, stream=side)
    side.synchronize()
    ref = oracle_mod.encode_split(want_in, cs, ws, 0)
    sizes = [int(v) for v in pb.cpu().tolist()]
    for t, n_, r in zip((lit, lens, offs, meta), sizes, ref):
        assert np.array_equal(t[:n_].cpu().numpy(), r)
    dec, dnb, st = g.decode_split(lit, lens, offs, meta, port_bytes=pb, stream=side)
    side.synchronize()
    assert int(st.item()) == 0 and np.array_equal(dec.cpu().numpy(), want_in)
