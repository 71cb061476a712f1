"""Locating and loading libpa.so (no torch import here, so the host-side
bookkeeping can be used without it)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

_cdll = None


class LibraryMissing(RuntimeError):
    pass


def cdll(path: str = LIB_PATH) -> ctypes.CDLL:
    """The loaded library (once per process); raises if it has not been built."""
    global _cdll
    if _cdll is not None:
        return _cdll
    if not os.path.exists(path):
        raise LibraryMissing(
            f"{path} is missing: build it with `python -m paged_kv_cache_47_amd.build` (there is no fallback)")
    _cdll = ctypes.CDLL(path)
    return _cdll
