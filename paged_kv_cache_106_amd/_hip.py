"""HIP events without a system-scope fence, through the HIP runtime torch has
already loaded (one runtime per process).

A default event record releases to system scope: the GPU writes back and
invalidates its caches, which on MI355X leaves a gap of several microseconds
in the stream.  The engine's events only order work on the device and tell
the host that a kernel has finished reading pinned memory, and the
benchmark's only take timestamps, so none of them needs that fence
(hipEventDisableSystemFence).  Passed to libpa's entry points, an event is
recorded by the kernel launch itself (hipExtLaunchKernel), with no marker
packet in the stream at all.
"""
import ctypes
import os

import torch

_hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
_hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
_hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
_hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
_hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                     ctypes.c_void_p]
_hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
_hip.hipGetErrorString.restype = ctypes.c_char_p

HIP_EVENT_DISABLE_TIMING = 0x2
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def _check(err, what):
    if err != 0:
        raise RuntimeError(f"{what}: {_hip.hipGetErrorString(err).decode()}")


class Event:
    """hipEvent_t created with hipEventDisableSystemFence."""

    def __init__(self, timing=False):
        self._e = ctypes.c_void_p()
        flags = HIP_EVENT_DISABLE_SYSTEM_FENCE | (0 if timing else HIP_EVENT_DISABLE_TIMING)
        _check(_hip.hipEventCreateWithFlags(ctypes.byref(self._e), flags), "hipEventCreateWithFlags")

    @property
    def handle(self):
        """The hipEvent_t, for the library's event arguments."""
        return self._e.value

    def record(self, stream):
        _check(_hip.hipEventRecord(self._e, ctypes.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def synchronize(self):
        _check(_hip.hipEventSynchronize(self._e), "hipEventSynchronize")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end`; both recorded and complete."""
        ms = ctypes.c_float()
        _check(_hip.hipEventElapsedTime(ctypes.byref(ms), self._e, end._e), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if getattr(self, "_e", None):
            _hip.hipEventDestroy(self._e)
