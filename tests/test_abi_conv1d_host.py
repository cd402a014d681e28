"""Host-side checks of the causal-conv1d C ABI (include/causal_conv1d.h): no GPU
needed, nothing is launched.  Every declared function is exported, the
workspace is sized, and bad arguments come back as status codes before any
work is enqueued."""
import ctypes
import os
import re

import pytest

from state_space_model_mamba_amd import conv1d, ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "causal_conv1d.h")


def header_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(conv1d_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = conv1d.load_library()
    names = header_functions()
    assert set(names) == set(conv1d.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_size():
    s = conv1d.make_shape(2, 1000, 96, 4, "silu", ssd.SSD_IO_F32)
    # one slot of (width + 1) * channels floats per 512-row block of each batch row
    assert conv1d.workspace_size(s) == 2 * 2 * 5 * 96 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(width=1), -2), (dict(width=5), -2), (dict(channels=12), -2), (dict(activation=2), -2),
    (dict(seqlen=0), -2), (dict(io_dtype=7), -2),
])
def test_unsupported_shapes_are_rejected(kw, code):
    base = dict(batch=1, seqlen=64, channels=16, width=4, activation="silu", io_dtype=ssd.SSD_IO_BF16)
    base.update(kw)
    s = conv1d.make_shape(**base)
    n = ctypes.c_size_t(0)
    assert conv1d.load_library().conv1d_bwd_workspace_size(ctypes.byref(s), ctypes.byref(n)) == code


FAKE = {k: 0x100000 * (i + 1) for i, k in enumerate(["x", "w", "b", "dout", "dx", "dw", "db", "ws"])}


def _bwd(s, p, ws_bytes=1 << 30):
    vp = ctypes.c_void_p
    return conv1d.load_library().conv1d_bwd(ctypes.byref(s), vp(p.get("x")), vp(p.get("w")), vp(p.get("b")), None,
                                            vp(p.get("dout")), vp(p.get("dx")), vp(p.get("dw")), vp(p.get("db")),
                                            vp(p.get("ws")), ctypes.c_size_t(ws_bytes), None)


def test_argument_errors_are_reported_before_launch():
    s = conv1d.make_shape(1, 64, 16, 4, "silu", ssd.SSD_IO_BF16)
    for missing in ("x", "w", "dout", "dx", "dw", "ws"):
        p = dict(FAKE)
        p.pop(missing)
        assert _bwd(s, p) == -1, missing
    p = dict(FAKE)
    p["dx"] += 8
    assert _bwd(s, p) == -4
    assert _bwd(s, FAKE, ws_bytes=16) == -3
    assert _bwd(s, dict(FAKE, dx=FAKE["x"])) == -1
    bad = conv1d.make_shape(1, 64, 16, 4, "silu", ssd.SSD_IO_BF16)
    bad.reserved = 1
    assert _bwd(bad, FAKE) == -1
    vp = ctypes.c_void_p
    lib = conv1d.load_library()
    assert lib.conv1d_fwd(ctypes.byref(s), vp(FAKE["x"]), None, None, None, vp(FAKE["dx"]), None) == -1
    assert lib.conv1d_fwd(ctypes.byref(s), vp(FAKE["x"] + 4), vp(FAKE["w"]), None, None, vp(FAKE["dx"]), None) == -4
