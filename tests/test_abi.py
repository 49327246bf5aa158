"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ets_topk.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:ets_status|int32_t|const char\*)\s+(ets_\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    import exact_top_selection_amd as ets
    if not os.path.exists(ets.library_path()):
        from exact_top_selection_amd import _build
        _build.build()
    return ets._load()


def test_header_declares_the_api():
    assert {"ets_topk_raw", "ets_topk_paged", "ets_topk_ragged", "ets_workspace_size",
            "ets_workspace_init", "ets_workspace_error", "ets_device_limits", "ets_group_cap",
            "ets_row_split", "ets_status_string"} <= set(_declared())


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ets_\w+)$", out, re.M))
    assert set(_declared()) <= exported


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "ets_topk.h"\nint main(void){ return ETS_OK; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                    str(src), "-o", str(tmp_path / "use")], check=True)


def test_status_strings(lib):
    for s in range(0, 6):
        assert lib.ets_status_string(s)
    assert b"unknown" in lib.ets_status_string(99)


def test_host_validation_rejects_before_device_work(lib):
    vp = ctypes.c_void_p
    fake = vp(0x1000)  # never dereferenced: validation fails first
    # k out of range
    assert lib.ets_topk_raw(fake, 64, 1, 64, None, 0, fake, 64, None, 0, None) == 2
    assert lib.ets_topk_raw(fake, 64, 1, 64, None, 2049, fake, 4096, None, 0, None) == 2
    # negative sizes, bad strides
    assert lib.ets_topk_raw(fake, 64, -1, 64, None, 8, fake, 8, None, 0, None) == 1
    assert lib.ets_topk_raw(fake, 32, 1, 64, None, 8, fake, 8, None, 0, None) == 1
    assert lib.ets_topk_raw(fake, 64, 1, 64, None, 8, fake, 4, None, 0, None) == 1
    # null output / scores
    assert lib.ets_topk_raw(fake, 64, 1, 64, None, 8, None, 8, None, 0, None) == 1
    assert lib.ets_topk_raw(None, 64, 1, 64, None, 8, fake, 8, None, 0, None) == 1
    # paged: bad page size, missing seq_lens / page table
    assert lib.ets_topk_paged(fake, 64, 1, 64, fake, fake, 1, 0, 8, fake, 8, None, 0, None) == 1
    assert lib.ets_topk_paged(fake, 64, 1, 64, None, fake, 1, 64, 8, fake, 8, None, 0, None) == 1
    assert lib.ets_topk_paged(fake, 64, 1, 64, fake, None, 1, 64, 8, fake, 8, None, 0, None) == 1
    # ragged: missing arrays, negative hint
    assert lib.ets_topk_ragged(fake, None, fake, 1, 10, 8, fake, 8, None, 0, None) == 1
    assert lib.ets_topk_ragged(fake, fake, fake, 1, -1, 8, fake, 8, None, 0, None) == 1
    # an empty batch is a no-op that needs no device
    assert lib.ets_topk_raw(None, 0, 0, 0, None, 8, None, 8, None, 0, None) == 0


def test_floor_validation(lib):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # dense: negative batch or length, stride below L, missing sink or scores
    assert lib.ets_floor_read(fake, 64, -1, 64, None, None, 0, fake, 64, None) == 1
    assert lib.ets_floor_read(fake, 32, 1, 64, None, None, 0, fake, 64, None) == 1
    assert lib.ets_floor_read(fake, 64, 1, 64, None, None, 0, None, 64, None) == 1
    assert lib.ets_floor_read(None, 64, 1, 64, None, None, 0, fake, 64, None) == 1
    # ragged: lengths required, hint >= 0
    assert lib.ets_floor_read(fake, 0, 1, 0, None, fake, 10, fake, 64, None) == 1
    assert lib.ets_floor_read(fake, 0, 1, 0, fake, fake, -1, fake, 64, None) == 1
    # empty batches need no device
    assert lib.ets_floor_read(None, 0, 0, 0, None, None, 0, None, 0, None) == 0
    assert lib.ets_floor_launch(0, 100, None) == 0
    assert lib.ets_floor_launch(-1, 100, None) == 1
    assert lib.ets_floor_launch(1, -1, None) == 1


def test_workspace_query_validation(lib):
    n = ctypes.c_size_t(123)
    assert lib.ets_workspace_size(4, 1000, 0, -1, ctypes.byref(n)) == 2
    assert lib.ets_workspace_size(-1, 1000, 8, -1, ctypes.byref(n)) == 1
    assert lib.ets_workspace_size(4, 1000, 8, -1, None) == 1


def test_workspace_init_validation(lib):
    # zero bytes is a no-op; a null or misaligned pointer is rejected on the host
    assert lib.ets_workspace_init(None, 0, None) == 0
    assert lib.ets_workspace_init(None, 256, None) == 1
    assert lib.ets_workspace_init(ctypes.c_void_p(0x1004), 256, None) == 1


def test_workspace_error_validation(lib):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # a flag buffer is required; a workspace must be aligned and hold the header
    assert lib.ets_workspace_error(fake, 4096, None, None) == 1
    assert lib.ets_workspace_error(None, 4096, fake, None) == 1
    assert lib.ets_workspace_error(ctypes.c_void_p(0x1004), 4096, fake, None) == 1
    assert lib.ets_workspace_error(fake, 128, fake, None) == 1


def test_device_limits_validation(lib):
    x = ctypes.c_int32(0)
    assert lib.ets_device_limits(-1, None, ctypes.byref(x), ctypes.byref(x)) == 1
    assert lib.ets_device_limits(-1, ctypes.byref(x), None, ctypes.byref(x)) == 1


def test_group_cap():
    """One XCD's compute units times the row-group workgroups each holds, at
    most the 64 member slots of a row's workspace record."""
    import exact_top_selection_amd as ets
    assert ets.group_cap(256, 8, 1) == 32   # MI355X: 32 CUs per XCD, one 1024-lane workgroup each
    assert ets.group_cap(256, 8, 2) == 64
    assert ets.group_cap(304, 8, 1) == 38
    assert ets.group_cap(304, 8, 3) == 64
    assert ets.group_cap(80, 1, 1) == 64
    assert ets.group_cap(0, 8, 1) == 0 and ets.group_cap(256, 0, 1) == 0 and ets.group_cap(256, 8, 0) == 0


def test_ticket_cap():
    """One shader engine's row-group slots: an XCD's compute units over its 4
    engines, times the row-group workgroups each holds, at least 1 and at
    most 64."""
    import exact_top_selection_amd as ets
    assert ets.ticket_cap(256, 8, 1) == 8   # MI355X: 8 CUs per engine, one 1024-lane workgroup each
    assert ets.ticket_cap(256, 8, 2) == 16
    assert ets.ticket_cap(32, 1, 1) == 8    # one XCD as its own device
    assert ets.ticket_cap(256, 8, 16) == 64
    assert ets.ticket_cap(8, 8, 1) == 1
    assert ets.ticket_cap(0, 8, 1) == 0 and ets.ticket_cap(256, 0, 1) == 0 and ets.ticket_cap(256, 8, 0) == 0
    for cu, x, occ in ((256, 8, 1), (304, 8, 1), (256, 8, 2), (80, 1, 1)):
        assert ets.ticket_cap(cu, x, occ) <= ets.group_cap(cu, x, occ)


def test_row_split_env_override(tmp_path):
    code = ("import exact_top_selection_amd as e; "
            "print(e.row_split(4, 262144, 256, 8, 1), e.row_split(64, 32768, 256, 8, 1), "
            "e.row_split(4, 262144, 256, 8, 2))")

    def run(v):
        env = dict(os.environ, ETS_ROW_SPLIT=v, PYTHONPATH=ROOT)
        return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                              text=True, check=True).stdout.split()

    assert run("7") == ["7", "7", "7"]
    assert run("0") == ["0", "0", "0"]
    assert run("1") == ["0", "0", "0"]
    assert run("32") == ["32", "32", "32"]
    # above the device's cap (or the record's 64 slots): rejected, never clamped
    assert run("64") == ["-1", "-1", "64"]
    assert run("1000") == ["-1", "-1", "-1"]


def test_row_split_heuristic():
    import exact_top_selection_amd as ets
    env = os.environ.pop("ETS_ROW_SPLIT", None)
    try:
        # rows that fit one 32768-score workgroup tile stay whole, whatever the batch
        for B, L in ((64, 32768), (128, 32768), (48, 8192), (1, 2048), (4, 4096), (1024, 8192)):
            assert ets.row_split(B, L, 256, 8, 1) == 0, (B, L)
        assert ets.row_split(0, 262144, 256, 8, 1) == 0
        # longer rows: chunks of about 16384 scores while one index grid (8 XCDs
        # x G x rows per XCD, at most 256 at one workgroup per CU) holds them
        assert ets.row_split(4, 32769, 256, 8, 1) == 3
        assert ets.row_split(4, 65536, 256, 8, 1) == 4
        assert ets.row_split(2, 100000, 256, 8, 1) == 7
        assert ets.row_split(1, 262144, 256, 8, 1) == 16
        assert ets.row_split(4, 262144, 256, 8, 1) == 16
        assert ets.row_split(16, 262144, 256, 8, 1) == 16  # 8 x 16 x 2 = 256
        assert ets.row_split(64, 65536, 256, 8, 1) == 4    # 8 x 4 x 8 = 256
        assert ets.row_split(4, 229000, 256, 8, 1) == 14
        assert ets.row_split(1, 10 ** 7, 256, 8, 1) == 32  # one XCD's slots
        # fewer members where that keeps the index grid within the device and
        # the chunks within one tile
        assert ets.row_split(20, 262144, 256, 8, 1) == 10  # 8 x 10 x 3 = 240
        assert ets.row_split(48, 131072, 256, 8, 1) == 5   # 8 x 5 x 6 = 240
        assert ets.row_split(64, 131072, 256, 8, 1) == 4   # 8 x 4 x 8 = 256
        assert ets.row_split(128, 65536, 256, 8, 1) == 2   # 8 x 2 x 16 = 256
        assert ets.row_split(40, 100000, 256, 8, 1) == 6
        # otherwise the fewest members whose chunks fit one tile, whatever the
        # batch: a ticketed grid, or several index grids above 8 members
        assert ets.row_split(32, 262144, 256, 8, 1) == 8
        assert ets.row_split(64, 262144, 256, 8, 1) == 8
        assert ets.row_split(128, 262144, 256, 8, 1) == 8
        assert ets.row_split(96, 65536, 256, 8, 1) == 2
        assert ets.row_split(192, 65536, 256, 8, 1) == 2
        assert ets.row_split(192, 131072, 256, 8, 1) == 4
        assert ets.row_split(256, 65536, 256, 8, 1) == 2
        assert ets.row_split(256, 262144, 256, 8, 1) == 8
        assert ets.row_split(4096, 262144, 256, 8, 1) == 8
        assert ets.row_split(16, 600000, 256, 8, 1) == 19
        # rows longer than 32 tiles: one XCD's slots, chunks streamed
        assert ets.row_split(64, 10 ** 7, 256, 8, 1) == 32
        # two row-group workgroups per CU: 512 slots
        assert ets.row_split(20, 262144, 256, 8, 2) == 16  # 8 x 16 x 3 = 384
        # the device's group cap bounds G (one XCD's slots: 20 for 160 CUs in 8 XCDs)
        assert ets.row_split(1, 10 ** 7, 160, 8, 1) == 20
        # unknown device facts: chunks of about 16384, within the 64 record slots
        assert ets.row_split(4, 262144, 0, 8, 1) == 16
        assert ets.row_split(4096, 262144, 0, 8, 1) == 16
        assert ets.row_split(1, 10 ** 7, 256, 0, 1) == 64
        assert ets.row_split(1, 10 ** 7, 256, 8, 0) == 64
        assert ets.row_split(1, 10 ** 7, 256, 8, 4) == 64
    finally:
        if env is not None:
            os.environ["ETS_ROW_SPLIT"] = env


def test_row_split_bounds_hold_everywhere():
    """Over a grid of shapes and devices: at most one XCD's row-group slots per
    row; a row that fits one 32768-score tile is never split and a longer one
    always is; chunks of at most 16384 scores are never cut further; chunks
    stay within one tile where the cap allows; and a G above the fewest
    members with resident chunks only where its index grid fits the device."""
    import exact_top_selection_amd as ets
    env = os.environ.pop("ETS_ROW_SPLIT", None)
    try:
        for cu, nx in ((80, 1), (256, 8), (304, 8)):
            cap = ets.group_cap(cu, nx, 1)
            for B in (1, 2, 3, 5, 8, 17, 64, 100, 128, 129, 256, 1000):
                for L in (1, 32768, 32769, 65536, 100000, 262144, 10 ** 6, 2 ** 31 - 1):
                    g = ets.row_split(B, L, cu, nx, 1)
                    assert 0 <= g <= cap, (cu, B, L, g)
                    assert (g == 0) == (L <= 32768), (cu, B, L, g)
                    if g:
                        tiles = -(-L // 32768)
                        g16 = min(-(-L // 16384), cap)
                        assert min(tiles, cap) <= g <= g16, (cu, B, L, g)
                        if g > min(tiles, cap):
                            assert nx * g * -(-B // nx) <= cu, (cu, B, L, g)
    finally:
        if env is not None:
            os.environ["ETS_ROW_SPLIT"] = env


def test_binding_constants_match_the_header():
    """The binding's copies of the header's limits."""
    import exact_top_selection_amd as ets
    text = open(HEADER).read()
    max_k = int(re.search(r"#define ETS_MAX_K (\d+)", text).group(1))
    scratch = re.search(r"#define ETS_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert ets.MAX_K == max_k
    assert ets.NOALLOC_SCRATCH_BYTES == int(scratch.group(1)) << int(scratch.group(2))


def test_error_bits_match_the_header_and_the_kernels():
    """The error word's bits: the binding's table, the header's description
    and the kernel source's enum name the same values."""
    import exact_top_selection_amd as ets
    text = " ".join(open(HEADER).read().replace("\n *", "\n").split())
    assert "2 marks a stale ticket" in text
    for bit, words in ((1, "the exchange of the row's bounds"), (4, "the poll of the row's coarse histogram"),
                       (8, "a barrier between radix rounds"), (16, "the wait for the row's tie-list entries")):
        assert "%d %s" % (bit, words) in text, bit
    src = open(os.path.join(ROOT, "exact_top_selection_amd", "csrc", "ets_topk.hip")).read()
    enum = re.search(r"enum ErrBit : uint32_t \{([^}]*)\}", src).group(1)
    vals = {name.strip(): int(v.strip().rstrip("u"), 0) for name, v in
            (item.split("=") for item in enum.split(","))}
    assert vals == {"kErrBounds": 1, "kErrStale": 2, "kErrCoarse": 4, "kErrBarrier": 8, "kErrTies": 16}
    assert sorted(ets.ERROR_BITS) == [1, 2, 4, 8, 16]
    assert ets.ERROR_BITS[2] == "stale ticket"
