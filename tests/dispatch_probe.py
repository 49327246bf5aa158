"""Build and load the test-only dispatch probe (tests/native/dispatch_probe.hip)."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "dispatch_probe.hip")
LIB = os.path.join(HERE, "native", "libets_dispatch_probe.so")


def build() -> str:
    """Compile the probe for gfx950 with the library's hipcc flags (always)."""
    from exact_top_selection_amd import _build
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_build.hipcc(), *_build.HIPCC_FLAGS, SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


def load():
    lib = ctypes.CDLL(LIB)
    lib.ets_test_dispatch_probe.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32,
                                            ctypes.c_uint32, ctypes.c_void_p]
    lib.ets_test_dispatch_probe.restype = ctypes.c_int
    return lib
