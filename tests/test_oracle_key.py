"""Pins of the oracle's order-preserving key (sglang PR #37591 digest, the
``order_key32`` excerpt: unsigned comparison of keys must equal float order).

The exhaustive walk compares against libm's ``nextafterf``; the hand values
below follow from the IEEE-754 binary32 layout, not from the key formula.
"""
import os
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _f2b(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def test_key_exhaustive_walk(oracle_mod, tmp_path):
    exe = str(tmp_path / "key_walk")
    odir = os.path.join(ROOT, "oracle")
    subprocess.run(["gcc", "-O2", os.path.join(ROOT, "tests", "native", "key_walk.c"),
                    "-L" + odir, "-lets_oracle", "-Wl,-rpath," + odir, "-lm", "-o", exe],
                   check=True)
    nsh = 8
    procs = [subprocess.Popen([exe, str(i), str(nsh)], stdout=subprocess.PIPE, text=True)
             for i in range(nsh)]
    total = 0
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out
        assert out.startswith("OK"), out
        total += int(out.split()[1])
    # every non-NaN pattern except +inf has a successor: 2^32 - 2 * (2^23 - 1) - 1
    assert total == 2 ** 32 - 2 * (2 ** 23 - 1) - 1


@pytest.mark.parametrize("lo,hi", [
    (float("-inf"), -3.0e38), (-1.0, -0.5), (-1.17549435e-38, -1.4e-45),
    (-1.4e-45, -0.0), (-0.0, 0.0), (0.0, 1.4e-45), (1.4e-45, 1.17549435e-38),
    (0.5, 1.0), (1.0, 1.0000001), (3.0e38, float("inf")),
])
def test_key_hand_order(oracle_mod, lo, hi):
    assert oracle_mod.order_key(_f2b(lo)) < oracle_mod.order_key(_f2b(hi))


def test_key_fixed_points(oracle_mod):
    # the key keeps the binary32 layout's monotone part and only moves signs:
    # +0.0 -> 0x80000000 (just above every negative value), -0.0 just below it
    assert oracle_mod.order_key(0x00000000) == 0x80000000
    assert oracle_mod.order_key(0x80000000) == 0x7FFFFFFF
    # -inf is the smallest non-NaN key, +inf the largest
    assert oracle_mod.order_key(_f2b(float("-inf"))) == 0x007FFFFF
    assert oracle_mod.order_key(_f2b(float("inf"))) == 0xFF800000
