"""Host sanitizers (CPU only): the oracle and the C ABI's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer, and their CPU tests run
against those builds in a child process.

* The oracle (plain C) is built with gcc ``-fsanitize=address,undefined`` and
  the oracle pin suites run on it.
* The library is built with hipcc, the sanitizers on its host code only
  (``-Xarch_host`` before each ``-fsanitize=``; device code is built as
  usual), and the host-side ABI tests run on it: argument checks, sizes,
  header reads.  No GPU is touched.
Any sanitizer report aborts the child, which fails the test.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run_pytest(env_extra: dict, preload: str, files: list[str]):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *files], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-shared", "-fPIC", os.path.join(ROOT, "oracle", "gpulz_oracle.c"),
                    "-o", str(lib), "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    files = [os.path.join("tests", f) for f in ("test_oracle_pins.py", "test_oracle_split.py",
                                                 "test_oracle_advancing.py", "test_oracle_lorenzo.py",
                                                 "test_oracle_parallel.py")]
    _run_pytest({"GPULZ_ORACLE_LIB": str(lib)}, asan, files)


def _clang_asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    for v in sorted(os.listdir(base)) if os.path.isdir(base) else []:
        p = os.path.join(base, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def test_abi_host_code_under_asan_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("no hipcc / clang ASan runtime")
    csrc = os.path.join(ROOT, "chunked_lzss_coder_amd", "csrc")
    flags = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", csrc]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs, procs = [], []
    for f in sorted(os.listdir(csrc)):
        if not f.endswith(".hip"):
            continue
        o = tmp_path / (f + ".o")
        objs.append(str(o))
        # the sanitizers go on the host code of the ABI entry points; the
        # kernel files keep their usual build
        extra = san if f == "abi.hip" else []
        procs.append(subprocess.Popen([HIPCC, *flags, *extra, "-c", os.path.join(csrc, f), "-o", str(o)],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out = p.communicate(timeout=900)[0].decode(errors="replace")
        assert p.returncode == 0, out[-3000:]
    lib = tmp_path / "libgpulz_san.so"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, *objs, "-o", str(lib)], check=True,
                   capture_output=True)
    _run_pytest({"GPULZ_LIB": str(lib)}, rt, [os.path.join("tests", "test_abi_host.py")])
