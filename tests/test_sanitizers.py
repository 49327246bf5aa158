"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer: the oracle
(every shape of row the checks use, against the rank definition) and the
library's host-side argument checks (host code only, no GPU)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, "%s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr[-4000:])
    return res.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "ets_oracle.c"), os.path.join(NATIVE, "oracle_sanitize.c"),
          "-lpthread", "-o", exe])
    out = _run([exe], env=SAN_ENV, timeout=300)
    assert "all rows match" in out


def test_library_host_checks_under_sanitizers(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hipcc = os.path.join(rocm, "bin", "hipcc")
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("hipcc or ROCm clang not available")
    lib = str(tmp_path / "libets_host_san.so")
    empty = tmp_path / "empty.gpubin"
    empty.write_bytes(b"")
    # Host code only, sanitizers on the host compilation alone; an empty GPU
    # binary stands in for the device code, which these calls never reach.
    _run([hipcc, "--offload-host-only", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
          "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
          "-Xclang", "-fcuda-include-gpubinary", "-Xclang", str(empty),
          "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "exact_top_selection_amd", "csrc", "ets_topk.hip"), "-o", lib])
    # the driver is built with the same compiler family, so that both share
    # one sanitizer runtime
    exe = str(tmp_path / "abi_san")
    _run([clang, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), os.path.join(NATIVE, "abi_sanitize.c"),
          lib, "-Wl,-rpath," + str(tmp_path), "-o", exe])
    out = _run([exe], env=SAN_ENV, timeout=300)
    assert "rejected as documented" in out
