"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU):

- the oracle (plain C), built with gcc's sanitizers together with a driver
  that calls every entry point on small ragged problems;
- the C ABI's host code (argument validation, plan choice, workspace sizing),
  compiled with clang's sanitizers on the host side only (device code is
  built as usual) and linked with the library's other objects, driven
  through every error path by a C program. No call there reaches a HIP API.

Any sanitizer report aborts the driver with a non-zero status."""
from __future__ import annotations

import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "oracle"), "-o", exe, os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "gspn_oracle.c"), "-lm", "-lpthread"])
    res = _run([exe], env=ENV)
    assert "all calls clean" in res.stdout


def _clang_rt_dir():
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return os.path.dirname(sorted(hits)[-1]) if hits else None


def test_abi_host_code_under_asan_ubsan():
    from linear_spatial_propagation_line_amd import build as b
    rt = _clang_rt_dir()
    if rt is None or not os.path.exists(b._hipcc()):
        pytest.skip("clang's sanitizer runtime or hipcc is not installed")
    others = [os.path.join(b.BUILD, os.path.splitext(s)[0] + ".o")
              for s in b.SOURCES if s != "gspn_api.cpp"]
    if not all(os.path.exists(o) for o in others):
        b.build()
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "gspn_api_asan.o")
    lib = os.path.join(OUT, "libgspn_asan.so")
    exe = os.path.join(OUT, "abi_driver")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in b.FLAGS if f != "-O3"]
    _run([b._hipcc(), *flags, "-O1", "-g", *host_san, "-c",
          os.path.join(b.CSRC, "gspn_api.cpp"), "-o", api_o])
    _run([b._hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-Xarch_host",
          "-shared-libasan", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-o", lib, api_o, *others])
    _run(["/opt/rocm/lib/llvm/bin/clang", "-std=c11", "-g", "-shared-libasan",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
          "-D__HIP_PLATFORM_AMD__", "-o", exe, os.path.join(HERE, "abi_driver.c"),
          "-L", OUT, "-lgspn_asan", f"-Wl,-rpath,{OUT}", f"-Wl,-rpath,{rt}"])
    res = _run([exe], env=ENV)
    assert "all calls clean" in res.stdout
