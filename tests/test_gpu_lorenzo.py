"""GPU parity of the Lorenzo-quantizer front end (gpulz_lorenzo_quant):
bit-exact codes and the same clamped count as the oracle, on ragged 1-D,
2-D and 3-D fields, exact rounding ties, clamping fields and the full
1800 x 3600 and 256 x 256 x 100 shapes; and the quantizer feeding the coder
gives the oracle's stream byte for byte."""
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


def gpu_quant(g, f: np.ndarray, eb: float):
    d = torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32)).to("cuda:0")
    codes, clamped = g.lorenzo_quant(d, eb)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), int(clamped.item())


def check(g, oracle_mod, f, eb):
    want, wk = oracle_mod.lorenzo_quant(f, eb)
    got, gk = gpu_quant(g, f, eb)
    assert got.shape == want.shape
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{bad.size} codes differ, first at cell {bad[:5]}"
    assert gk == wk


@pytest.mark.parametrize("shape", [(1,), (2,), (7,), (4097,), (1, 1), (3, 5), (17, 33), (64, 130),
                                   (1, 1, 1), (2, 3, 5), (5, 6, 7), (9, 31, 66)])
def test_random_fields(g, oracle_mod, shape):
    rng = np.random.default_rng(sum(shape) + len(shape))
    for eb in (1e-4, 1e-2, 0.3):
        f = (rng.standard_normal(shape) * 2.0).astype(np.float32)
        check(g, oracle_mod, f, eb)


def test_rounding_ties(g, oracle_mod):
    # 2 eb = 1 and every value exactly halfway between two integers
    rng = np.random.default_rng(5)
    f = (rng.integers(-1000, 1000, size=(23, 41)) + 0.5).astype(np.float32)
    check(g, oracle_mod, f, 0.5)
    check(g, oracle_mod, f.reshape(-1), 0.5)
    check(g, oracle_mod, f[:20, :40].reshape(4, 5, 40), 0.5)


def test_clamping(g, oracle_mod):
    rng = np.random.default_rng(6)
    f = (rng.standard_normal((31, 45)) * 5e4).astype(np.float32)
    want, wk = oracle_mod.lorenzo_quant(f, 0.5)
    assert wk > 0
    check(g, oracle_mod, f, 0.5)


def test_constant_and_zero_patches(g, oracle_mod):
    f = np.zeros((40, 70), np.float32)
    f[10:30, 20:50] = 1.25
    check(g, oracle_mod, f, 1e-3)
    check(g, oracle_mod, np.zeros((3, 4, 5), np.float32), 1e-3)


@pytest.mark.parametrize("shape", [(1800, 3600), (100, 256, 256)])
def test_full_size_fields(g, oracle_mod, shape):
    import workloads as synth
    rng = np.random.default_rng(11)
    f = synth._sinusoid_field(rng, shape).astype(np.float32)
    f[synth._zero_patches(rng, shape, 0.3)] = 0.0
    eb = 1e-4 * float(f.max() - f.min())
    check(g, oracle_mod, f, eb)


def test_quantizer_feeds_the_coder(g, oracle_mod):
    # device codes -> device encode must equal oracle codes -> oracle encode
    import workloads as synth
    rng = np.random.default_rng(12)
    f = synth._sinusoid_field(rng, (300, 700)).astype(np.float32)
    eb = 1e-4 * float(f.max() - f.min())
    codes_o, _ = oracle_mod.lorenzo_quant(f, eb)
    d = torch.from_numpy(f).to("cuda:0")
    codes, _ = g.lorenzo_quant(d, eb)
    for level in (0, 1):
        out, nb = g.encode(codes, 2048, 4, level)
        torch.cuda.synchronize()
        got = out[: int(nb.item())].cpu().numpy().tobytes()
        want = oracle_mod.encode(codes_o.view(np.uint8).reshape(-1), 2048, 4, level).tobytes()
        assert got == want


def test_invalid_arguments(g):
    d = torch.zeros((4, 4), dtype=torch.float32, device="cuda:0")
    for eb in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(g.GpulzError):
            g.lorenzo_quant(d, eb)
