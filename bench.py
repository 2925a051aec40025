#!/usr/bin/env python3
"""Benchmark of the gfx950 chunked LZSS coder on one MI355X.

A step is one pass of the whole hot path over the workload: for every match
level, gpulz_encode (chunk encode + size scan + stream assembly) followed by
gpulz_decode of the stream it produced, inputs resident in HBM.

Prints ONE JSON line.  ``value`` is the level-0 encode throughput in decimal
GB/s of uncompressed input (whole gpulz_encode call); decode GB/s and the
compression ratio of every level sit beside it.  ``roofline`` reports the
dominant kernel (the chunk encode kernel) against the HBM peak, with its
duration taken from HIP events recorded around that kernel alone, and
``cpu_baseline`` the CPU oracle (one pinned core, and all cores) on the
same bytes.

Default workload: 2D Lorenzo residual codes of a 1800x3600 field
(25,920,000 bytes of uint32 words), chunk_size 2048, word_size 4, levels 0
and 1.  ``stress_level0`` adds the largest level-0 run beside it: the 2 GiB
stress stream (chunk 4096, word 4) with per-call and per-kernel encode and
decode times and their fractions of the HBM peak (``--no-stress-row`` skips
it).  ``--workload 4 --levels 0`` makes the stress stream the main workload.
Every stream is compared whole with the oracle's in the CPU-baseline leg.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

_ROOT = os.path.dirname(os.path.abspath(__file__))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (torch.cuda.Event only sees torch's stream;
    these are handed to the library, which records them on its stream)."""

    def __init__(self):
        import torch  # noqa: F401  (binds the HIP runtime torch uses)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def pair(self):
        evs = []
        for _ in range(2):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events.append(e)
            evs.append(e)
        return tuple(evs)

    def ms(self, pair) -> float:
        f = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(f), pair[0], pair[1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(f.value)

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def kernel_source_hash() -> str:
    """sha256 over the encode kernel's sources: a counter record taken from
    other sources no longer describes the kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in ("encode.hip", "common.h"):
        with open(os.path.join(_ROOT, "chunked_lzss_coder_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(cs: int, ws: int, level: int, workload: str):
    """HBM bytes per launch of the chunk encode kernel from the committed
    rocprofv3 counter record (FETCH_SIZE and WRITE_SIZE, each scaled by the
    same counter's reading for a plain copy of known size), or None when no
    record matches this workload and these kernel sources."""
    path = os.path.join(_ROOT, "profiles", "encode_traffic.json")
    try:
        with open(path) as fh:
            recs = json.load(fh)
    except (OSError, ValueError):
        return None
    src = kernel_source_hash()
    for r in recs.get("records", []):
        if (r.get("source_sha256") == src and r.get("workload") == workload and r.get("chunk_size") == cs
                and r.get("word_size") == ws and r.get("level") == level):
            return r.get("traffic_bytes")
    return None


def host_cpu() -> dict:
    """The host's CPU model and counts, as the CPU-baseline leg reports them."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(w, levels):
    """Oracle leg: the plain single-threaded C oracle on the workload's bytes,
    timed on one pinned host core (whole encodes repeated for a few seconds
    per level), and the same oracle calls over contiguous whole-chunk ranges on
    all usable cores (at most 16, the host share of one GPU)."""
    import numpy as np

    import oracle
    oracle.build()
    n, cs, ws = w.n, w.chunk_size, w.word_size
    # bounded sample: the whole workload if it is small, else a prefix of
    # whole chunks worth about 64 MiB (chunks are coded independently)
    limit = 64 << 20
    take = n if n <= limit else (limit // cs) * cs
    sample = w.data[:take]
    cpu = host_cpu()
    try:
        allowed = sorted(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = []
    threads = max(1, min(16, cpu["usable_cpus"]))
    per_level = {}
    for level in levels:
        # single thread, pinned to one core for the timed passes
        pinned = None
        if allowed:
            pinned = allowed[-1]
            os.sched_setaffinity(0, {pinned})
        try:
            times = []
            while len(times) < 3 or (sum(times) < 6.0 and len(times) < 200):
                t0 = time.perf_counter()
                ref = oracle.encode(sample, cs, ws, level)
                times.append(time.perf_counter() - t0)
            t0 = time.perf_counter()
            back = oracle.decode(ref)
            t_dec = time.perf_counter() - t0
        finally:
            if allowed:
                os.sched_setaffinity(0, set(allowed))
        ok_rt = bool(np.array_equal(back, sample))
        # all cores: the same oracle calls over contiguous whole-chunk ranges
        mt = []
        while len(mt) < 3 or (sum(mt) < 3.0 and len(mt) < 200):
            t0 = time.perf_counter()
            oracle.encode_parallel(sample, cs, ws, level, threads=threads)
            mt.append(time.perf_counter() - t0)
        med, mmed = float(np.median(times)), float(np.median(mt))
        per_level[level] = {
            "encode_gbps": round(take / med / 1e9, 6),
            "encode_gbps_mean": round(take * len(times) / sum(times) / 1e9, 6),
            "decode_gbps": round(take / t_dec / 1e9, 6),
            "passes": len(times), "encode_s": round(sum(times), 3), "pinned_cpu": pinned,
            "round_trip": ok_rt,
            "all_cores": {"encode_gbps": round(take / mmed / 1e9, 6), "threads": threads, "passes": len(mt)},
        }
    l0 = per_level[levels[0]]
    return {
        "value": l0["encode_gbps"],
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"level-{levels[0]} encode of {'the whole workload' if take == n else 'the first %d bytes' % take}"
                   f" ({take} bytes), median of {l0['passes']} whole passes, single-threaded C oracle pinned to"
                   f" one core; all_cores: the same calls over contiguous whole-chunk ranges on {threads} threads"),
        "host_cpu": cpu,
        "all_cores": {"value": l0["all_cores"]["encode_gbps"], "unit": "GB/s", "cores": threads},
        "levels": {str(k): v for k, v in per_level.items()},
    }


def oracle_identical(w, level, gpu_stream):
    """Oracle leg: is the whole GPU stream (a host uint8 array) the oracle's,
    byte for byte?  The oracle's stream is built by the single-threaded oracle
    run on contiguous whole-chunk ranges across the host's cores (chunks are
    coded independently).  Returns (flag, scope)."""
    import numpy as np

    import oracle
    oracle.build()
    ref = oracle.encode_parallel(w.data, w.chunk_size, w.word_size, level)
    return bool(ref.size == gpu_stream.size and np.array_equal(ref, gpu_stream)), "whole stream"


def stress_level0_row(g, ev, dev, steps: int, warmup: int):
    """The 2 GiB stress stream (chunk 4096, word 4) at level 0, the largest
    level-0 run: per-call and per-kernel encode and decode times, their
    fractions of the HBM peak, the ratio and the round trip.  Returns the row,
    the workload and a host copy of the GPU stream (for the oracle check)."""
    import numpy as np
    import torch

    import workloads
    t0 = time.perf_counter()
    w = workloads.workload(4)
    log(f"stress row: {w.name}, {w.n} bytes, generated in {time.perf_counter() - t0:.1f}s")
    cs, ws, n = w.chunk_size, w.word_size, w.n
    x = torch.from_numpy(w.data).to(dev)
    cap = g.max_compressed_size(n, cs)
    out = torch.empty(cap, dtype=torch.uint8, device=dev)
    nb = torch.zeros(1, dtype=torch.uint64, device=dev)
    ews = torch.empty(g.encode_workspace_size(n, cs), dtype=torch.uint8, device=dev)
    dout = torch.empty(n, dtype=torch.uint8, device=dev)
    dnb = torch.zeros(1, dtype=torch.uint64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    dws = torch.empty(g.decode_workspace_size(cap), dtype=torch.uint8, device=dev)
    g.encode_into(x, cs, ws, 0, out, nb, ews)
    torch.cuda.synchronize()
    sb = int(nb.item())
    g.decode_into(out, sb, dout, dnb, st, dws)
    torch.cuda.synchronize()
    if sb < 32 or int(st.item()) != 0 or int(dnb.item()) != n or not torch.equal(dout, x):
        raise RuntimeError("stress row: level-0 round trip failed")
    hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = []
    for i in range(warmup + steps):
        ce, cd = ev.pair(), ev.pair()
        ev.hip.hipEventRecord(ce[0], hs)
        g.encode_into(x, cs, ws, 0, out, nb, ews)
        ev.hip.hipEventRecord(ce[1], hs)
        ev.hip.hipEventRecord(cd[0], hs)
        g.decode_into(out, sb, dout, dnb, st, dws)
        ev.hip.hipEventRecord(cd[1], hs)
        if i >= warmup:
            calls.append((ce, cd))
    kern = []
    for _ in range(steps):
        ke, kd = ev.pair(), ev.pair()
        g.encode_into(x, cs, ws, 0, out, nb, ews, events=ke)
        g.decode_into(out, sb, dout, dnb, st, dws, events=kd)
        kern.append((ke, kd))
    torch.cuda.synchronize()
    if int(nb.item()) != sb or int(st.item()) != 0 or not torch.equal(dout, x):
        raise RuntimeError("stress row: repeated calls differ")
    me = float(np.mean([ev.ms(c[0]) for c in calls]))
    md = float(np.mean([ev.ms(c[1]) for c in calls]))
    mke = float(np.mean([ev.ms(k[0]) for k in kern]))
    mkd = float(np.mean([ev.ms(k[1]) for k in kern]))
    algo = n + (sb - 32)  # input + size-table rows + payloads (decode: the same, read and write swapped)

    def frac(ms):
        return round(algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 5)
    row = {
        "workload": w.name, "bytes": n, "chunk_size": cs, "word_size": ws, "level": 0,
        "ratio": round(n / sb, 4), "stream_bytes": sb, "algorithmic_bytes": algo,
        "encode_ms": round(me, 4), "encode_gbps": round(n / (me * 1e-3) / 1e9, 3),
        "encode_kernel_ms": round(mke, 4), "encode_assembly_ms": round(me - mke, 4),
        "decode_ms": round(md, 4), "decode_gbps": round(n / (md * 1e-3) / 1e9, 3),
        "decode_kernel_ms": round(mkd, 4),
        "encode_frac_per_call": frac(me), "encode_frac_kernel": frac(mke),
        "decode_frac_per_call": frac(md), "decode_frac_kernel": frac(mkd),
        "encode_kernel_traffic": measured_traffic(cs, ws, 0, w.name),
        "round_trip": True, "steps": steps, "warmup": warmup,
    }
    host_stream = out[:sb].cpu().numpy()
    del x, out, nb, ews, dout, dnb, st, dws
    torch.cuda.empty_cache()
    return row, w, host_stream


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, help="workload index 0..4 (default 1)")
    ap.add_argument("--levels", type=str, default=None, help="comma-separated match levels (default: workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (the HBM-counter reference)")
    ap.add_argument("--no-split", action="store_true", help="skip the split-mode (four ports) measurement")
    ap.add_argument("--no-stress-row", action="store_true",
                    help="skip the level-0 row of the 2 GiB stress stream beside the headline workload")
    ap.add_argument("--flush-reps", type=int, default=11,
                    help="repetitions of the flushed-cache and host-latency measurements (0: skip)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this coder runs on one GPU; --gpus {args.gpus} is not supported "
              f"(chunks shard across GPUs with one scan of per-shard sizes, not built here)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import chunked_lzss_coder_amd as g
    import workloads as synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    g.lib()
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    w = synth.workload(args.workload)
    log(f"workload {w.name}: {w.n} bytes, cs {w.chunk_size}, ws {w.word_size}, sha256 {w.sha256()[:16]}, "
        f"generated in {time.perf_counter() - t0:.1f}s")
    levels = tuple(int(x) for x in args.levels.split(",")) if args.levels else tuple(sorted(w.levels))
    cs, ws = w.chunk_size, w.word_size
    n = w.n
    x = torch.from_numpy(w.data.copy()).to(dev)
    cap = g.max_compressed_size(n, cs)
    ev = HipEvents()

    bufs = {}
    for lv in levels:
        out = torch.empty(cap, dtype=torch.uint8, device=dev)
        nb = torch.zeros(1, dtype=torch.uint64, device=dev)
        ews = torch.empty(g.encode_workspace_size(n, cs), dtype=torch.uint8, device=dev)
        dout = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        dnb = torch.zeros(1, dtype=torch.uint64, device=dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        dws = torch.empty(g.decode_workspace_size(cap), dtype=torch.uint8, device=dev)
        bufs[lv] = (out, nb, ews, dout, dnb, st, dws)

    # first pass: sizes, round trip (outside any timed region)
    stream_bytes = {}
    for lv in levels:
        out, nb, ews, dout, dnb, st, dws = bufs[lv]
        g.encode_into(x, cs, ws, lv, out, nb, ews)
        torch.cuda.synchronize()
        stream_bytes[lv] = int(nb.item())
        g.decode_into(out, stream_bytes[lv], dout, dnb, st, dws)
        torch.cuda.synchronize()
        if int(st.item()) != 0 or int(dnb.item()) != n or not torch.equal(dout[:n], x):
            print(f"bench.py: level {lv} round trip failed (status {int(st.item())})", file=sys.stderr)
            return 1

    def step(record):
        # one step: every level's encode and decode call, each between its own
        # pair of events, nothing recorded inside the calls
        for lv in levels:
            out, nb, ews, dout, dnb, st, dws = bufs[lv]
            ce = ev.pair() if record is not None else None
            cd = ev.pair() if record is not None else None
            s = torch.cuda.current_stream()
            if ce:
                ev.hip.hipEventRecord(ce[0], ctypes.c_void_p(s.cuda_stream))
            g.encode_into(x, cs, ws, lv, out, nb, ews)
            if ce:
                ev.hip.hipEventRecord(ce[1], ctypes.c_void_p(s.cuda_stream))
                ev.hip.hipEventRecord(cd[0], ctypes.c_void_p(s.cuda_stream))
            g.decode_into(out, stream_bytes[lv], dout, dnb, st, dws)
            if cd:
                ev.hip.hipEventRecord(cd[1], ctypes.c_void_p(s.cuda_stream))
            if record is not None:
                record.append((lv, ce, cd))

    ev.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done; timing {args.steps} steps")
    rec = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    # Kernel times, after the timed steps: the same calls through the timed
    # entry points (events around each chunk kernel only), K of each per level.
    krec = []
    for _ in range(args.steps):
        for lv in levels:
            out, nb, ews, dout, dnb, st, dws = bufs[lv]
            ke, kd = ev.pair(), ev.pair()
            g.encode_into(x, cs, ws, lv, out, nb, ews, events=ke)
            g.decode_into(out, stream_bytes[lv], dout, dnb, st, dws, events=kd)
            krec.append((lv, ke, kd))
    torch.cuda.synchronize()

    # Back to back: the same calls with no events inside them, K encodes then
    # K decodes between one pair of events per level (the GPU never waits for
    # the host: a call enqueues in far less time than it runs).
    b2b = {}
    s_ = torch.cuda.current_stream()
    for lv in levels:
        out, nb, ews, dout, dnb, st, dws = bufs[lv]
        e_enc, e_dec = ev.pair(), ev.pair()
        torch.cuda.synchronize()
        ev.hip.hipEventRecord(e_enc[0], ctypes.c_void_p(s_.cuda_stream))
        for _ in range(args.steps):
            g.encode_into(x, cs, ws, lv, out, nb, ews)
        ev.hip.hipEventRecord(e_enc[1], ctypes.c_void_p(s_.cuda_stream))
        ev.hip.hipEventRecord(e_dec[0], ctypes.c_void_p(s_.cuda_stream))
        for _ in range(args.steps):
            g.decode_into(out, stream_bytes[lv], dout, dnb, st, dws)
        ev.hip.hipEventRecord(e_dec[1], ctypes.c_void_p(s_.cuda_stream))
        torch.cuda.synchronize()
        if int(st.item()) != 0 or int(nb.item()) != stream_bytes[lv] or not torch.equal(dout[:n], x):
            print(f"bench.py: level {lv} back-to-back run differs", file=sys.stderr)
            return 1
        b2b[lv] = (ev.ms(e_enc) / max(args.steps, 1), ev.ms(e_dec) / max(args.steps, 1))

    res = {}
    for lv in levels:
        rows = [r for r in rec if r[0] == lv]
        krows = [r for r in krec if r[0] == lv]
        enc_ms = [ev.ms(r[1]) for r in rows]
        dec_ms = [ev.ms(r[2]) for r in rows]
        kenc_ms = [ev.ms(r[1]) for r in krows]
        kdec_ms = [ev.ms(r[2]) for r in krows]
        me, mke, md, mkd = (float(np.mean(v)) for v in (enc_ms, kenc_ms, dec_ms, kdec_ms))
        sb = stream_bytes[lv]
        chunks = -(-n // cs)
        algo = n + 8 * chunks + (sb - 32 - 8 * chunks)  # read input, write table rows + payloads
        res[lv] = {
            "encode_gbps": round(n / (me * 1e-3) / 1e9, 3),
            "decode_gbps": round(n / (md * 1e-3) / 1e9, 3),
            "ratio": round(n / sb, 4),
            "stream_bytes": sb,
            "encode_ms": round(me, 4),
            "decode_ms": round(md, 4),
            "encode_ms_median": round(float(np.median(enc_ms)), 4),
            "decode_ms_median": round(float(np.median(dec_ms)), 4),
            "encode_kernel_ms": round(mke, 4),
            "decode_kernel_ms": round(mkd, 4),
            "encode_ms_back_to_back": round(b2b[lv][0], 4),
            "decode_ms_back_to_back": round(b2b[lv][1], 4),
            "encode_gbps_back_to_back": round(n / (b2b[lv][0] * 1e-3) / 1e9, 3),
            "decode_gbps_back_to_back": round(n / (b2b[lv][1] * 1e-3) / 1e9, 3),
            "encode_kernel_hbm_gbps": round(algo / (mke * 1e-3) / 1e9, 2),
            "decode_kernel_hbm_gbps": round(algo / (mkd * 1e-3) / 1e9, 2),
            "algorithmic_bytes": algo,
            "round_trip": True,
        }
    # Flushed runs: a 512 MiB write between repetitions evicts the input and
    # the stream from the caches (the 256 MB last-level cache included); and
    # host-observed latency: the call plus the read-back of *d_out_bytes.
    if args.flush_reps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        s_ = torch.cuda.current_stream()
        for lv in levels:
            out, nb, ews, dout, dnb, st, dws = bufs[lv]
            fe, fd, he, hd = [], [], [], []
            for i in range(args.flush_reps):
                flush.fill_(i & 0xFF)
                ce = ev.pair()
                ev.hip.hipEventRecord(ce[0], ctypes.c_void_p(s_.cuda_stream))
                g.encode_into(x, cs, ws, lv, out, nb, ews)
                ev.hip.hipEventRecord(ce[1], ctypes.c_void_p(s_.cuda_stream))
                flush.fill_((i + 1) & 0xFF)
                cd = ev.pair()
                ev.hip.hipEventRecord(cd[0], ctypes.c_void_p(s_.cuda_stream))
                g.decode_into(out, stream_bytes[lv], dout, dnb, st, dws)
                ev.hip.hipEventRecord(cd[1], ctypes.c_void_p(s_.cuda_stream))
                torch.cuda.synchronize()
                fe.append(ev.ms(ce))
                fd.append(ev.ms(cd))
                th = time.perf_counter()
                g.encode_into(x, cs, ws, lv, out, nb, ews)
                _ = int(nb.item())
                he.append((time.perf_counter() - th) * 1e3)
                th = time.perf_counter()
                g.decode_into(out, stream_bytes[lv], dout, dnb, st, dws)
                _ = int(dnb.item())
                hd.append((time.perf_counter() - th) * 1e3)
            res[lv]["flushed"] = {
                "reps": args.flush_reps,
                "encode_ms_median": round(float(np.median(fe)), 4),
                "decode_ms_median": round(float(np.median(fd)), 4),
                "encode_gbps": round(n / (float(np.median(fe)) * 1e-3) / 1e9, 3),
                "decode_gbps": round(n / (float(np.median(fd)) * 1e-3) / 1e9, 3),
            }
            res[lv]["host_latency_ms_median"] = {"encode": round(float(np.median(he)), 4),
                                                 "decode": round(float(np.median(hd)), 4)}
        del flush
    # Split mode (four ports) at the first level: whole-call encode and decode
    # times with the same inputs, and the port sizes.
    split = None
    if not args.no_split:
        lv = levels[0]
        bl, bt, bm = g.split_bounds(n, cs, ws)
        p_lit = torch.empty(max(bl, 1), dtype=torch.uint8, device=dev)
        p_len = torch.empty(max(bt, 1), dtype=torch.uint8, device=dev)
        p_off = torch.empty(max(bt, 1), dtype=torch.uint8, device=dev)
        p_meta = torch.empty(max(bm, 1), dtype=torch.uint8, device=dev)
        p_bytes = torch.zeros(4, dtype=torch.uint64, device=dev)
        s_ews = torch.empty(g.encode_split_workspace_size(n, cs), dtype=torch.uint8, device=dev)
        g.encode_split_into(x, cs, ws, lv, p_lit, p_len, p_off, p_meta, p_bytes, s_ews)
        torch.cuda.synchronize()
        pbv = [int(v) for v in p_bytes.cpu().tolist()]
        s_dws = torch.empty(g.decode_split_workspace_size(pbv[3]), dtype=torch.uint8, device=dev)
        dout, dnb, st = bufs[lv][3], bufs[lv][4], bufs[lv][5]
        g.decode_split_into(p_lit, pbv[0], p_len, p_off, pbv[1], p_meta, pbv[3], dout, dnb, st, s_dws)
        torch.cuda.synchronize()
        if int(st.item()) != 0 or not torch.equal(dout[:n], x):
            print("bench.py: split-mode round trip failed", file=sys.stderr)
            return 1
        s_ = torch.cuda.current_stream()
        se, sd = [], []
        for i in range(args.warmup + args.steps):
            ce, cd = ev.pair(), ev.pair()
            ev.hip.hipEventRecord(ce[0], ctypes.c_void_p(s_.cuda_stream))
            g.encode_split_into(x, cs, ws, lv, p_lit, p_len, p_off, p_meta, p_bytes, s_ews)
            ev.hip.hipEventRecord(ce[1], ctypes.c_void_p(s_.cuda_stream))
            ev.hip.hipEventRecord(cd[0], ctypes.c_void_p(s_.cuda_stream))
            g.decode_split_into(p_lit, pbv[0], p_len, p_off, pbv[1], p_meta, pbv[3], dout, dnb, st, s_dws)
            ev.hip.hipEventRecord(cd[1], ctypes.c_void_p(s_.cuda_stream))
            if i >= args.warmup:
                se.append(ce)
                sd.append(cd)
        torch.cuda.synchronize()
        me = float(np.mean([ev.ms(p) for p in se]))
        md = float(np.mean([ev.ms(p) for p in sd]))
        split = {"level": lv, "encode_gbps": round(n / (me * 1e-3) / 1e9, 3),
                 "decode_gbps": round(n / (md * 1e-3) / 1e9, 3), "encode_ms": round(me, 4),
                 "decode_ms": round(md, 4),
                 "port_bytes": {"literals": pbv[0], "lengths": pbv[1], "offsets": pbv[2], "meta": pbv[3]},
                 "ratio_before_entropy_coding": round(n / max(1, sum(pbv)), 4)}
        del p_lit, p_len, p_off, p_meta, s_ews, s_dws
    # Baseline: the one-thread-per-chunk decode of the same stream (the shape
    # the pages attribute to upstream), kernel time against the block decoder.
    baseline = None
    if not args.no_split:
        lv = levels[0]
        out, nb, ews, dout, dnb, st, dws = bufs[lv]
        s_ = torch.cuda.current_stream()
        kb, ks = [], []
        for i in range(args.warmup + args.steps):
            k1, k2 = ev.pair(), ev.pair()
            g.decode_into(out, stream_bytes[lv], dout, dnb, st, dws, events=k1)
            g.decode_one_thread_per_chunk_into(out, stream_bytes[lv], dout, dnb, st, dws, events=k2)
            if i >= args.warmup:
                kb.append(k1)
                ks.append(k2)
        torch.cuda.synchronize()
        if int(st.item()) != 0 or not torch.equal(dout[:n], x):
            print("bench.py: one-thread-per-chunk decode mismatch", file=sys.stderr)
            return 1
        mb_, ms_ = float(np.mean([ev.ms(p) for p in kb])), float(np.mean([ev.ms(p) for p in ks]))
        baseline = {"level": lv, "block_decode_kernel_ms": round(mb_, 4),
                    "one_thread_per_chunk_decode_kernel_ms": round(ms_, 4), "speedup": round(ms_ / mb_, 2)}
    # Baseline: the upstream-style advancing-window search (level 0), its
    # stream's ratio and its chunk kernel time beside the exact search's.
    search_base = None
    if not args.no_split and 0 in levels:
        a_out = torch.empty(g.max_compressed_size(n, cs), dtype=torch.uint8, device=dev)
        a_nb = torch.zeros(1, dtype=torch.uint64, device=dev)
        ews = bufs[0][2]
        ka = []
        for i in range(args.warmup + args.steps):
            k = ev.pair()
            g.encode_advancing_into(x, cs, ws, a_out, a_nb, ews, events=k)
            if i >= args.warmup:
                ka.append(k)
        torch.cuda.synchronize()
        a_bytes = int(a_nb.item())
        _, _, _, dout, dnb, st, dws = bufs[0]
        g.decode_into(a_out, a_bytes, dout, dnb, st, dws)
        torch.cuda.synchronize()
        if int(st.item()) != 0 or not torch.equal(dout[:n], x):
            print("bench.py: advancing-search stream does not round-trip", file=sys.stderr)
            return 1
        ma_ = float(np.mean([ev.ms(p) for p in ka]))
        search_base = {"level": 0, "exact_search_ratio": res[0]["ratio"],
                       "advancing_search_ratio": round(n / a_bytes, 4),
                       "exact_search_kernel_ms": res[0]["encode_kernel_ms"],
                       "advancing_search_kernel_ms": round(ma_, 4),
                       "exact_kernel_speedup": round(ma_ / res[0]["encode_kernel_ms"], 2)}
        del a_out, a_nb
    # The Lorenzo-quantizer front end on the device: the workload's float
    # field -> its u32 codes, kernel time and the front end's roofline (4 bytes
    # read + 4 written per cell).  Its codes are checked against the oracle's
    # by the GPU tests, not here.
    front = None
    fld = synth.field_of(args.workload)
    if fld is not None and not args.no_split:
        f32, rel = fld
        eb = synth.abs_error_bound(f32, rel)
        d_f = torch.from_numpy(f32).to(dev)
        codes = torch.empty(f32.shape, dtype=torch.uint32, device=dev)
        clamped = torch.zeros(1, dtype=torch.int64, device=dev)
        s_ = torch.cuda.current_stream()
        ts_ = []
        for i in range(args.warmup + args.steps):
            e_ = ev.pair()
            ev.hip.hipEventRecord(e_[0], ctypes.c_void_p(s_.cuda_stream))
            g.lorenzo_quant_into(d_f, eb, codes, clamped)
            ev.hip.hipEventRecord(e_[1], ctypes.c_void_p(s_.cuda_stream))
            if i >= args.warmup:
                ts_.append(e_)
        torch.cuda.synchronize()
        mq = float(np.mean([ev.ms(p_) for p_ in ts_]))
        cells = f32.size
        hbm = 8.0 * cells / (mq * 1e-3) / 1e9
        front = {"field": "x".join(str(d_) for d_ in f32.shape) + " float32", "abs_error_bound": eb,
                 "ms": round(mq, 4), "field_gbps": round(4.0 * cells / (mq * 1e-3) / 1e9, 3),
                 "clamped": int(clamped.item()),
                 "roofline": {"bound": "hbm", "achieved": round(hbm, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(hbm / HBM_PEAK_GBPS, 5)}}
        del d_f, codes, clamped
    # Near-window and chunk-size sweep (the pages' ratio trade): ratio and
    # encode kernel time for windows 32 / 48 / 64, both levels, chunk sizes
    # 2048 and 4096, on the same input.
    sweep = None
    if not args.no_split and ws == 4 and n <= (64 << 20):
        sweep = []
        s_ = torch.cuda.current_stream()
        for cs_ in (2048, 4096):
            cap_ = g.max_compressed_size(n, cs_)
            o_ = torch.empty(cap_, dtype=torch.uint8, device=dev)
            nb_ = torch.zeros(1, dtype=torch.uint64, device=dev)
            w_ = torch.empty(g.encode_workspace_size(n, cs_), dtype=torch.uint8, device=dev)
            for lv in (0, 1):
                for win in (32, 48, 64):
                    g.encode_window_into(x, cs_, ws, lv, win, o_, nb_, w_)
                    ts_ = []
                    for i in range(3 + 5):
                        e_ = ev.pair()
                        ev.hip.hipEventRecord(e_[0], ctypes.c_void_p(s_.cuda_stream))
                        g.encode_window_into(x, cs_, ws, lv, win, o_, nb_, w_)
                        ev.hip.hipEventRecord(e_[1], ctypes.c_void_p(s_.cuda_stream))
                        if i >= 3:
                            ts_.append(e_)
                    torch.cuda.synchronize()
                    sb_ = int(nb_.item())
                    me_ = float(np.median([ev.ms(p_) for p_ in ts_]))
                    sweep.append({"chunk_size": cs_, "level": lv, "window": win, "ratio": round(n / sb_, 4),
                                  "encode_ms": round(me_, 4), "encode_gbps": round(n / (me_ * 1e-3) / 1e9, 3)})
            del o_, nb_, w_
    if args.calibration_copy_mib > 0:
        a_ = torch.empty(args.calibration_copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        b_ = torch.empty_like(a_)
        torch.cuda.synchronize()
        b_.copy_(a_)
        torch.cuda.synchronize()
        del a_, b_
    # measured device-to-device copy rate (bytes read + written per second),
    # reported beside the published HBM peak
    copy_gbps = None
    if args.flush_reps > 0:
        a_ = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
        b_ = torch.empty_like(a_)
        b_.copy_(a_)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(5):
            e0.record()
            b_.copy_(a_)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        copy_gbps = round(2 * a_.numel() / (float(np.median(ts)) * 1e-3) / 1e9, 1)
        del a_, b_

    lv0 = levels[0]
    r0 = res[lv0]
    E = cs // ws
    roof = {
        "bound": "hbm",
        # the template instance as the kernel trace names it (word, elements, level,
        # window, waves per chunk, chunks per workgroup)
        "kernel": "encode_kernel<%d, %d, %d, 32, %d, %d>" % (ws, E, lv0, 1 if E <= 512 else E // 512,
                                                           2 if E <= 512 else 1),
        "decode_kernel": "chunks_kernel",
        "achieved": r0["encode_kernel_hbm_gbps"],
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(r0["encode_kernel_hbm_gbps"] / HBM_PEAK_GBPS, 5),
        "traffic": measured_traffic(cs, ws, lv0, w.name),
        "measured_copy_gbps": copy_gbps,
        "kernel_ms": r0["encode_kernel_ms"],
        "algorithmic_bytes_per_launch": r0["algorithmic_bytes"],
        # the stricter reading: input bytes only over the same kernel time
        "frac_input_only": round(w.n / (r0["encode_kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 5),
        # the decode kernel of the same level against the same peak
        "decode_frac": round(r0["decode_kernel_hbm_gbps"] / HBM_PEAK_GBPS, 5),
        "decode_frac_input_only": round(w.n / (r0["decode_kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 5),
    }

    # The largest level-0 run beside the headline workload: the 2 GiB stress
    # stream (its inputs do not fit the 256 MB last-level cache).
    stress = None
    stress_w = stress_stream = None
    if not args.no_stress_row and args.workload != 4:
        stress, stress_w, stress_stream = stress_level0_row(g, ev, dev, max(3, min(args.steps, 10)),
                                                            max(1, min(args.warmup, 3)))
        log(f"stress row: encode {stress['encode_ms']} ms/call ({stress['encode_kernel_ms']} kernel), "
            f"decode {stress['decode_ms']} ms/call ({stress['decode_kernel_ms']} kernel)")
    ev.close()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, levels)
        log(f"cpu oracle: {cpu['value']} GB/s encode, single pinned core ({cpu['host_cpu']})")
        for lv in levels:
            out = bufs[lv][0]
            flag, scope = oracle_identical(w, lv, out[:stream_bytes[lv]].cpu().numpy())
            res[lv]["byte_identical"] = bool(flag)
            res[lv]["byte_identical_scope"] = scope
            log(f"level {lv}: byte_identical={flag} ({scope})")
        if stress is not None:
            flag, scope = oracle_identical(stress_w, 0, stress_stream)
            stress["byte_identical"] = flag
            stress["byte_identical_scope"] = scope
            log(f"stress row: byte_identical={flag} ({scope})")
    del stress_w, stress_stream

    ms_per_step = wall * 1e3 / max(args.steps, 1)
    line = {
        "metric": "encode/decode GB/s (uncompressed) + compression ratio, word4 chunk2048, 1 GPU",
        "value": r0["encode_gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32" if ws == 4 else ("u16" if ws == 2 else "u8"),
        "data": "synthetic",
        "config": {"workload": w.name, "bytes": n, "chunk_size": cs, "word_size": ws, "levels": list(levels),
                   "sha256": w.sha256()},
        "encode_gbps": r0["encode_gbps"],
        "decode_gbps": r0["decode_gbps"],
        "ratio": r0["ratio"],
        "levels": {str(k): v for k, v in res.items()},
        "split": split,
        "decode_baseline": baseline,
        "search_baseline": search_base,
        "lorenzo_front_end": front,
        "window_sweep": sweep,
        "roofline": roof,
        "stress_level0": stress,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
