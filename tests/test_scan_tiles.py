"""Decode scan geometry (csrc/scan_tiles.h), checked on the host: for every
chunk count a stream can declare under the host's bound, the scan launch has
a workgroup for each of its tiles and the workspace a slot for each tile's
total.  The header is compiled with g++ into a small checker."""
from __future__ import annotations

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_scan_tiles_cover_every_stream_under_the_bound(tmp_path):
    exe = tmp_path / "scan_tiles_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "chunked_lzss_coder_amd", "csrc"),
                    os.path.join(ROOT, "tests", "native", "scan_tiles_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
