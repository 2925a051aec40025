"""Seeded synthetic workloads for the chunked LZSS coder.

This module only fabricates input bytes.  It holds none of the coder's
arithmetic, so both the HIP path's tests/benchmark and the CPU oracle's
tests may draw their inputs from it.

The pages measure on Lorenzo-quantized climate residuals (CESM CLDHGH) and on
SDRB fields that are not available here; the generators below stand in for
them with fields of the same shapes, value distributions and structure:

* ``lorenzo2d`` / ``lorenzo3d``: a smooth sum of random-phase sinusoids
  (optionally with additive noise and with ~30 % of the cells clamped to
  exactly 0.0 in contiguous patches), pre-quantized with an absolute error
  bound ``eb`` (q = rint(f / 2eb)), then the integer Lorenzo residual of q is
  taken and offset by the radius 32768, clamped to [0, 65535] and stored as
  little-endian uint32 words.
* ``byte_mix``: a byte stream mixing low-entropy Zipf bytes, repeats of short
  phrases at short distances and uniform random bytes.
* ``stress_u32``: segments cycling through constant runs, uniform random
  words, short-period patterns and Lorenzo residual codes.

Every generator is a pure function of its seed.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

RADIUS = 32768


def _sinusoid_field(rng: np.random.Generator, shape: tuple[int, ...], n_terms: int = 8) -> np.ndarray:
    """Sum of n_terms random-phase sinusoids over a grid (float64).

    Term k has amplitude 1/(k+1) and 0.5..8 cycles across each axis."""
    axes = [np.arange(s, dtype=np.float64) / s for s in shape]
    f = np.zeros(shape, dtype=np.float64)
    for k in range(n_terms):
        freqs = rng.uniform(0.5, 8.0, size=len(shape))
        phase = rng.uniform(0.0, 2.0 * np.pi)
        arg = phase
        for d, (a, fr) in enumerate(zip(axes, freqs)):
            sh = [1] * len(shape)
            sh[d] = shape[d]
            arg = arg + 2.0 * np.pi * fr * a.reshape(sh)
        f += np.sin(arg) / (k + 1)
    return f


def _zero_patches(rng: np.random.Generator, shape: tuple[int, ...], frac: float = 0.30) -> np.ndarray:
    """Boolean mask of contiguous patches covering ~frac of the grid: a smooth
    4-term low-frequency field thresholded at its frac-quantile."""
    axes = [np.arange(s, dtype=np.float64) / s for s in shape]
    g = np.zeros(shape, dtype=np.float64)
    for _ in range(4):
        freqs = rng.uniform(0.5, 3.0, size=len(shape))
        phase = rng.uniform(0.0, 2.0 * np.pi)
        arg = phase
        for d, (a, fr) in enumerate(zip(axes, freqs)):
            sh = [1] * len(shape)
            sh[d] = shape[d]
            arg = arg + 2.0 * np.pi * fr * a.reshape(sh)
        g += np.sin(arg)
    return g < np.quantile(g, frac)


def _lorenzo_codes(field32: np.ndarray, rel_eb: float) -> tuple[np.ndarray, int]:
    """Pre-quantize a float32 field and return uint32 Lorenzo residual codes
    (radius-offset, clamped) plus the number of clamped cells."""
    f = field32.astype(np.float64)
    eb = abs_error_bound(field32, rel_eb)
    q = np.rint(f / (2.0 * eb)).astype(np.int64)
    # integer Lorenzo predictor: inclusion-exclusion over the lower corner
    # neighbours, cells outside the grid read as 0
    p = np.pad(q, [(1, 0)] * q.ndim)
    d = np.zeros_like(q)
    nd = q.ndim
    for mask in range(1 << nd):
        sl = tuple(slice(0, -1) if (mask >> ax) & 1 else slice(1, None) for ax in range(nd))
        sign = -1 if bin(mask).count("1") % 2 else 1
        d += sign * p[sl]
    code = d + RADIUS
    clamped = int(np.count_nonzero((code < 0) | (code > 65535)))
    return np.clip(code, 0, 65535).astype(np.uint32).reshape(-1), clamped


def field2d(seed: int, rows: int, cols: int, noise: float = 0.0, zero_frac: float = 0.0) -> np.ndarray:
    """The float32 field behind the 2-D Lorenzo workloads."""
    rng = np.random.default_rng(seed)
    f = _sinusoid_field(rng, (rows, cols))
    if noise > 0:
        f = f + rng.normal(0.0, noise, size=f.shape)
    if zero_frac > 0:
        f[_zero_patches(rng, (rows, cols), zero_frac)] = 0.0
    return f.astype(np.float32)


def field3d(seed: int, nz: int, ny: int, nx: int, zero_frac: float = 0.0) -> np.ndarray:
    """The float32 field behind the 3-D Lorenzo workload."""
    rng = np.random.default_rng(seed)
    f = _sinusoid_field(rng, (nz, ny, nx))
    if zero_frac > 0:
        f[_zero_patches(rng, (nz, ny, nx), zero_frac)] = 0.0
    return f.astype(np.float32)


def abs_error_bound(field32: np.ndarray, rel_eb: float) -> float:
    """Absolute error bound of a relative one: rel_eb times the value range."""
    f = field32.astype(np.float64)
    rng_ = float(f.max() - f.min())
    return rel_eb * (rng_ if rng_ > 0 else 1.0)


def lorenzo2d(seed: int, rows: int, cols: int, rel_eb: float, noise: float = 0.0,
              zero_frac: float = 0.0) -> tuple[np.ndarray, int]:
    return _lorenzo_codes(field2d(seed, rows, cols, noise, zero_frac), rel_eb)


def lorenzo3d(seed: int, nz: int, ny: int, nx: int, rel_eb: float, zero_frac: float = 0.0):
    return _lorenzo_codes(field3d(seed, nz, ny, nx, zero_frac), rel_eb)


def byte_mix(seed: int, n: int, fractions=(0.60, 0.25, 0.15)) -> tuple[np.ndarray, dict]:
    """Bytes from segments: Zipf(s=1.2) over 16 fixed symbols (length 32..512),
    repeats of an earlier 4..64-byte phrase at distance 1..300 (overlap allowed),
    uniform random bytes (length 16..256).  Segment kinds are drawn so that the
    expected byte fractions match ``fractions``."""
    rng = np.random.default_rng(seed)
    out = np.empty(n, dtype=np.uint8)
    symbols = rng.choice(256, size=16, replace=False).astype(np.uint8)
    pz = (np.arange(1, 17, dtype=np.float64)) ** -1.2
    pz /= pz.sum()
    mean_len = np.array([(32 + 512) / 2, (4 + 64) / 2, (16 + 256) / 2])
    pk = np.asarray(fractions) / mean_len
    pk /= pk.sum()
    # pre-draw enough segment descriptors in bulk
    est = int(n / float((pk * mean_len).sum()) * 1.2) + 64
    kinds = rng.choice(3, size=est, p=pk)
    zl = rng.integers(32, 513, size=est)
    pl = rng.integers(4, 65, size=est)
    pd = rng.integers(1, 301, size=est)
    rl = rng.integers(16, 257, size=est)
    zipf_pool = symbols[rng.choice(16, size=min(n, 1 << 22), p=pz)]
    rand_pool = rng.integers(0, 256, size=min(n, 1 << 22), dtype=np.uint8)
    counts = [0, 0, 0]
    pos, i, zp, rp = 0, 0, 0, 0
    while pos < n:
        if i >= est:  # extremely unlikely; extend with fresh draws
            kinds = np.append(kinds, rng.choice(3, size=est, p=pk))
            zl = np.append(zl, rng.integers(32, 513, size=est))
            pl = np.append(pl, rng.integers(4, 65, size=est))
            pd = np.append(pd, rng.integers(1, 301, size=est))
            rl = np.append(rl, rng.integers(16, 257, size=est))
            est = kinds.size
        k = int(kinds[i])
        if k == 1 and pos == 0:
            k = 2
        if k == 0:
            ln = min(int(zl[i]), n - pos)
            if zp + ln > zipf_pool.size:
                zp = 0
            out[pos:pos + ln] = zipf_pool[zp:zp + ln]
            zp += ln
        elif k == 1:
            ln = min(int(pl[i]), n - pos)
            d = min(int(pd[i]), pos)
            src = out[pos - d:pos]
            out[pos:pos + ln] = np.resize(src, ln)  # overlapping copy = period-d repeat
        else:
            ln = min(int(rl[i]), n - pos)
            if rp + ln > rand_pool.size:
                rp = 0
                rand_pool = rng.integers(0, 256, size=rand_pool.size, dtype=np.uint8)
            out[pos:pos + ln] = rand_pool[rp:rp + ln]
            rp += ln
        counts[k] += ln
        pos += ln
        i += 1
    return out, {"zipf": counts[0] / n, "phrase": counts[1] / n, "random": counts[2] / n}


def stress_u32(seed: int, n_bytes: int) -> tuple[np.ndarray, dict]:
    """uint32 stream of 1..64 KiB segments cycling: constant run (value 0 with
    probability 1/2, else random), uniform random words, a random pattern of
    period 1..300 repeated, Lorenzo residual codes (2D recipe, slices of a pool
    of 512x512 tiles with their own sub-seeds)."""
    assert n_bytes % 4 == 0
    rng = np.random.default_rng(seed)
    nw = n_bytes // 4
    out = np.empty(nw, dtype=np.uint32)
    pool = [lorenzo2d(seed * 1000 + 100 + t, 512, 512, 1e-3, noise=0.01)[0] for t in range(8)]
    kinds_bytes = [0, 0, 0, 0]
    pos, kind = 0, 0
    while pos < nw:
        ln = min(int(rng.integers(256, 16385)), nw - pos)
        if kind == 0:
            v = 0 if rng.random() < 0.5 else int(rng.integers(1, 1 << 32))
            out[pos:pos + ln] = v
        elif kind == 1:
            out[pos:pos + ln] = rng.integers(0, 1 << 32, size=ln, dtype=np.uint64).astype(np.uint32)
        elif kind == 2:
            period = int(rng.integers(1, 301))
            pat = rng.integers(0, 1 << 32, size=period, dtype=np.uint64).astype(np.uint32)
            out[pos:pos + ln] = np.resize(pat, ln)
        else:
            tile = pool[int(rng.integers(0, len(pool)))]
            st = int(rng.integers(0, tile.size))
            idx = (st + np.arange(ln)) % tile.size
            out[pos:pos + ln] = tile[idx]
        kinds_bytes[kind] += 4 * ln
        pos += ln
        kind = (kind + 1) % 4
    tot = float(n_bytes)
    return out, {"const": kinds_bytes[0] / tot, "random": kinds_bytes[1] / tot,
                 "periodic": kinds_bytes[2] / tot, "lorenzo": kinds_bytes[3] / tot}


@dataclass
class Workload:
    """One synthetic workload: the bytes plus the coder parameters."""
    name: str
    data: np.ndarray  # uint8, 1-D
    chunk_size: int
    word_size: int
    levels: tuple[int, ...]
    info: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.data.size)

    def sha256(self) -> str:
        return hashlib.sha256(self.data.tobytes()).hexdigest()


def _as_bytes(words: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(words.astype("<u4")).view(np.uint8).reshape(-1)


# The five workload shapes.  Index = seed.
WORKLOAD_NAMES = (
    "lorenzo2d_512x512_u32_cs2048",       # 1 MiB, level 0
    "lorenzo2d_1800x3600_u32_cs2048",     # ~26 MB, levels 0 and 1
    "lorenzo3d_256x256x100_u32_cs4096",   # ~26 MB, level 1
    "bytemix_64MiB_u8_cs4096",            # 64 MiB, ws 1, levels 0 and 1
    "stress_2GiB_u32_cs4096",             # 2 GiB, level 1 (+ level 0 row)
)


def field_of(idx: int) -> tuple[np.ndarray, float] | None:
    """(float32 field, relative error bound) behind workload idx, for the
    Lorenzo-field workloads (0, 1, 2); None for the others."""
    if idx == 0:
        return field2d(0, 512, 512, noise=0.01), 1e-3
    if idx == 1:
        return field2d(1, 1800, 3600, zero_frac=0.30), 1e-4
    if idx == 2:
        return field3d(2, 100, 256, 256, zero_frac=0.30), 1e-4
    return None


def workload(idx: int, scale_bytes: int | None = None) -> Workload:
    """Build workload idx (0..4).  scale_bytes shrinks the byte-stream and
    stress workloads (3, 4) for quick tests; the field workloads have fixed
    grids."""
    seed = idx
    if idx == 0:
        w, cl = lorenzo2d(seed, 512, 512, 1e-3, noise=0.01)
        return Workload(WORKLOAD_NAMES[0], _as_bytes(w), 2048, 4, (0,), {"clamped": cl})
    if idx == 1:
        w, cl = lorenzo2d(seed, 1800, 3600, 1e-4, zero_frac=0.30)
        return Workload(WORKLOAD_NAMES[1], _as_bytes(w), 2048, 4, (0, 1), {"clamped": cl})
    if idx == 2:
        w, cl = lorenzo3d(seed, 100, 256, 256, 1e-4, zero_frac=0.30)
        return Workload(WORKLOAD_NAMES[2], _as_bytes(w), 4096, 4, (1,), {"clamped": cl})
    if idx == 3:
        n = scale_bytes if scale_bytes is not None else 64 << 20
        b, fr = byte_mix(seed, n)
        return Workload(WORKLOAD_NAMES[3], b, 4096, 1, (0, 1), fr)
    if idx == 4:
        n = scale_bytes if scale_bytes is not None else 2 << 30
        n -= n % 4
        w, fr = stress_u32(seed, n)
        return Workload(WORKLOAD_NAMES[4], _as_bytes(w), 4096, 4, (1, 0), fr)
    raise ValueError(idx)
