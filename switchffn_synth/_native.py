"""ctypes loaders for the generator's host (C) and device (HIP) fillers."""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libswitchffn_synth_host.so")
DEV_LIB = os.path.join(_HERE, "libswitchffn_synth_dev.so")

_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is missing; run __graft_entry__.build() first")
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_fill_host.restype = ctypes.c_int
        lib.synth_fill_host.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                        ctypes.c_int, ctypes.c_int]
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is missing; run __graft_entry__.build() first")
        # torch first, so that this library binds to torch's HIP runtime rather than
        # loading a second one (torch bundles libamdhip64 under the same soname).
        import torch  # noqa: F401
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_error_string.restype = ctypes.c_char_p
        lib.synth_error_string.argtypes = [ctypes.c_int]
        lib.synth_fill_device.restype = ctypes.c_int
        lib.synth_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                          ctypes.c_int, ctypes.c_void_p]
        _dev = lib
    return _dev


def fill_host(out: np.ndarray, start: int, seed: int, stream: int, sigma: float, bf16: bool,
              nthreads: int) -> None:
    assert out.flags.c_contiguous and out.dtype == (np.uint16 if bf16 else np.float32)
    rc = _load_host().synth_fill_host(out.ctypes.data, out.size, start, seed, stream, sigma,
                                      int(bf16), nthreads)
    if rc != 0:
        raise RuntimeError(f"synth_fill_host failed ({rc})")


def fill_device(ptr: int, n: int, start: int, seed: int, stream: int, sigma: float, bf16: bool,
                hip_stream: int) -> None:
    lib = _load_dev()
    rc = lib.synth_fill_device(ptr, n, start, seed, stream, sigma, int(bf16), hip_stream)
    if rc != 0:
        why = lib.synth_error_string(rc).decode() if rc > 0 else "bad arguments"
        raise RuntimeError(f"synth_fill_device failed ({rc}: {why})")
