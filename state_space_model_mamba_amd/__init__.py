"""Deterministic Mamba-2 SSD chunked-scan backward for MI355X (gfx950).

The computation runs in the HIP library ``libssd_bwd.so`` (built from
``csrc/``); ``ssd`` is its thin ctypes binding.  Importing this package does
not load the library; ``ssd_bwd`` does, and raises if it is missing.
"""
from .workloads import WORKLOADS, Workload, make_inputs  # noqa: F401


def ssd_bwd(*args, **kwargs):
    from .ssd import ssd_bwd as _impl
    return _impl(*args, **kwargs)
