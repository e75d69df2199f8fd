"""ctypes handles on the compiled fillers (host C/OpenMP and device HIP) of the seeded streams."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "_synth_host.so")
DEVICE_LIB = os.path.join(_HERE, "_synth_fill.so")

_host = None
_device = None


def host_lib():
    """The C/OpenMP filler, or None if it has not been built."""
    global _host
    if _host is None and os.path.exists(HOST_LIB):
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_fill_normal_host.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_uint64, ctypes.c_float, ctypes.c_int]
        lib.synth_fill_normal_host.restype = ctypes.c_int
        _host = lib
    return _host


def device_lib():
    """The HIP filler; raises if it has not been built."""
    global _device
    if _device is None:
        import torch  # noqa: F401  (map torch's HIP runtime first, so the filler binds to it)
        if not os.path.exists(DEVICE_LIB):
            raise RuntimeError(f"device filler not built: {DEVICE_LIB} (run __graft_entry__.build())")
        lib = ctypes.CDLL(DEVICE_LIB)
        lib.synth_fill_normal_device.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_uint64, ctypes.c_float, ctypes.c_int,
                                                 ctypes.c_void_p]
        lib.synth_fill_normal_device.restype = ctypes.c_int
        _device = lib
    return _device
