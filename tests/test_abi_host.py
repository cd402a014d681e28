"""Host-side checks of the C ABI: no GPU needed, nothing is launched.

The library must load, export every function declared in include/ssd_bwd.h,
size its workspace, and reject bad arguments with a status code before any
work is enqueued.
"""
import ctypes
import os
import re

import pytest

from state_space_model_mamba_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd_bwd.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(ssd_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = ssd.load_library()
    names = header_functions()
    assert set(names) == set(ssd.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def shape(**kw):
    base = dict(batch=1, seqlen=2048, nheads=128, headdim=64, ngroups=8, dstate=128, chunk_size=256,
                nseqs=1, io_dtype=ssd.SSD_IO_BF16)
    base.update(kw)
    return ssd.make_shape(**base)


def test_workspace_size_and_regions():
    s = shape()
    n = ssd.workspace_size(s)
    nc = 8
    state = 1 * 128 * nc * 64 * 128 * 2   # Hin and dS are held in the I/O dtype (bf16 here)
    assert n >= 2 * state
    off_h, nb_h = ssd.workspace_region(s, ssd.SSD_WS_HIN)
    off_d, nb_d = ssd.workspace_region(s, ssd.SSD_WS_DSTATE)
    off_a, nb_a = ssd.workspace_region(s, ssd.SSD_WS_ACS)
    assert nb_h == nb_d == state and nb_a == 128 * nc * 256 * 4
    for off, nb in ((off_h, nb_h), (off_d, nb_d), (off_a, nb_a)):
        assert off % 256 == 0 and off + nb <= n
    assert len({off_h, off_d, off_a}) == 3
    # ragged tail: one more chunk
    assert ssd.workspace_size(shape(seqlen=2049)) > n
    # fp32 I/O (chunk 128, 16 chunks): fp32 states
    f = shape(io_dtype=ssd.SSD_IO_F32, chunk_size=128)
    assert ssd.workspace_region(f, ssd.SSD_WS_HIN)[1] == 1 * 128 * 16 * 64 * 128 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(nheads=100), -2),          # not a multiple of ngroups
    (dict(chunk_size=96), -2),
    (dict(headdim=48), -2),
    (dict(headdim=16), -2),          # bf16 needs headdim % 32 == 0
    (dict(dstate=24), -2),
    (dict(dstate=48), -2),           # bf16 needs dstate % 32 == 0
    (dict(io_dtype=ssd.SSD_IO_F32, chunk_size=64, headdim=16, dstate=40), -2),
    (dict(dstate=512), -2),
    (dict(io_dtype=7), -1),
    (dict(batch=0), -1),
    (dict(seqlen=0), -1),
    (dict(io_dtype=ssd.SSD_IO_F32, chunk_size=256), -2),  # fp32 stops at chunk 128
    # one chunk of x rows (Q H P) or of B rows (Q G N) beyond 2^31 bytes
    (dict(nheads=65544, ngroups=8), -2),
    (dict(nheads=16400, ngroups=16400, dstate=256), -2),
])
def test_unsupported_shapes_are_rejected(kw, code):
    n = ctypes.c_size_t(0)
    rc = ssd.load_library().ssd_bwd_workspace_size(ctypes.byref(shape(**kw)), ctypes.byref(n))
    assert rc == code
    assert ssd.status_string(rc) != "unknown status"


def test_largest_chunk_of_rows_is_supported():
    # Q H P bf16 elements of exactly 2^31 bytes
    assert ssd.workspace_size(shape(nheads=65536, ngroups=8)) > 0


def test_supported_fp32_shape():
    assert ssd.workspace_size(shape(io_dtype=ssd.SSD_IO_F32, chunk_size=64, headdim=16, dstate=16,
                                    nheads=4, ngroups=1, seqlen=256)) > 0


def _call(s, ptrs, ws_bytes=1 << 40):
    lib = ssd.load_library()
    names = ["x", "dt", "A", "B", "C", "D", "dy", "h0", "seq_idx", "dx", "ddt", "dA", "dB", "dC",
             "dD", "dinit", "ws"]
    args = [ctypes.c_void_p(ptrs.get(n)) if ptrs.get(n) else None for n in names]
    return lib.ssd_bwd(ctypes.byref(s), *args, ctypes.c_size_t(ws_bytes), None)


FAKE = {n: 0x10000 * (i + 1) for i, n in enumerate(
    ["x", "dt", "A", "B", "C", "D", "dy", "dx", "ddt", "dA", "dB", "dC", "dD", "ws"])}


def test_argument_errors_are_reported_before_launch():
    s = shape()
    for missing in ("x", "dt", "A", "B", "C", "dy", "dx", "ddt", "dA", "dB", "dC", "ws"):
        p = dict(FAKE)
        p.pop(missing)
        assert _call(s, p) == -1, missing
    p = dict(FAKE)
    p.pop("D")
    assert _call(s, p) == -1          # dD without D
    p = dict(FAKE)
    p["x"] += 8
    assert _call(s, p) == -4          # misaligned
    assert _call(s, FAKE, ws_bytes=16) == -3
    # initial-state gradients without seq_idx need nseqs == batch
    p = dict(FAKE, dinit=0x990000)
    assert _call(shape(nseqs=3), p) == -1
    bad = shape()
    bad.reserved = 1
    assert _call(bad, FAKE) == -1


def test_version_and_status_strings():
    v = ssd.load_library().ssd_bwd_version()
    assert v >> 16 >= 1
    assert ssd.status_string(0) == "ok"
    assert ssd.status_string(-99) == "unknown status"


def test_frontend_argument_errors_are_reported_before_launch():
    lib = ssd.load_library()
    s = shape()
    names = ["x", "dt", "A", "B", "C", "D", "dy", "h0", "seq_idx", "dx", "ddt", "dA", "dB", "dC", "dD", "dinit"]

    def call(fe, ddt_bias=None, z=None, dz=None):
        args = [ctypes.c_void_p(FAKE.get(n)) if FAKE.get(n) else None for n in names]
        vp = lambda v: ctypes.c_void_p(v) if v else None
        return lib.ssd_bwd_ex(ctypes.byref(s), ctypes.byref(fe) if fe is not None else None, *args[:6], vp(z),
                              *args[6:], vp(ddt_bias), vp(dz), ctypes.c_void_p(FAKE["ws"]),
                              ctypes.c_size_t(1 << 40), None)

    inf = float("inf")
    assert call(ssd.SsdOptions(None, 1, 0.5, 0.1, 0)) == -1            # dt_min > dt_max
    assert call(ssd.SsdOptions(None, 1, float("nan"), inf, 0)) == -1   # NaN bound
    assert call(ssd.SsdOptions(None, 1, -inf, inf, 0), ddt_bias=0x990000) == -1   # ddt_bias without dt_bias
    assert call(None, ddt_bias=0x990000) == -1
    assert call(ssd.SsdOptions(0x990008, 1, -inf, inf, 0)) == -4       # misaligned dt_bias
    assert call(None, z=0x990000) == -1                                 # z without dz
    assert call(None, dz=0x990000) == -1                                # dz without z
    assert call(None, z=0x990000, dz=FAKE["dx"]) == -1                  # dz aliasing dx (dx holds the gated dy)
    assert call(None, z=0x990000, dz=0x9a0008) == -4                    # misaligned dz


def test_launch_geometry_hook_checks_its_arguments():
    lib = ssd.load_library()
    assert lib.ssd_set_launch_geometry(-1, 0) == -1
    assert lib.ssd_set_launch_geometry(0, -3) == -1
    assert lib.ssd_set_launch_geometry(0, 0) == 0


def test_group_path_hook_checks_its_argument_and_sizes_the_workspace():
    lib = ssd.load_library()
    assert lib.ssd_set_group_path(3) == -1 and lib.ssd_set_group_path(-1) == -1
    sh = shape()   # 1 x 2048, 128 heads, 8 groups, N = 128: 64 blocks, the fused path by shape
    try:
        sizes = {}
        for path in (0, 1, 2):
            assert lib.ssd_set_group_path(path) == 0
            sizes[path] = ssd.workspace_size(sh)
        assert sizes[0] == sizes[1] < sizes[2]   # the split path holds dCB and its transpose
    finally:
        lib.ssd_set_group_path(0)


def test_many_heads_per_group_take_the_split_path_with_head_slices():
    # 64 blocks of (batch, group, chunk), but 64 heads in the one group: the split
    # path by shape, its dCB kernel cut into 4 head slices (256 blocks) whose fp32
    # sums take a workspace region of their own
    lib = ssd.load_library()
    sh = shape(seqlen=16384, nheads=64, ngroups=1, dstate=256, nseqs=7)
    try:
        sizes = {}
        for path in (0, 1, 2):
            assert lib.ssd_set_group_path(path) == 0
            sizes[path] = ssd.workspace_size(sh)
        assert sizes[0] == sizes[2] > sizes[1]
        nc, tiles = 64, 256 * (256 + 16) // 2
        assert sizes[2] - sizes[1] >= 4 * nc * tiles * 4 + 2 * nc * 256 * 256 * 2   # slices' sums, dCB and dCB^T
    finally:
        lib.ssd_set_group_path(0)
