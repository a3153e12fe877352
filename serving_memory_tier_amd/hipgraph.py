"""HIP stream capture, graph replay and timing events, on the HIP runtime this
process already runs (ctypes).

The library binds to torch's HIP runtime by soname; a second copy of the
runtime would not know torch's streams, so the runtime is located through the
process's own mappings.  The hot-path entry points allocate nothing, take no
host-side wait and issue no memset, so a step (table updates, resolve, move,
offload) captures into a graph as it stands.
"""

from __future__ import annotations

import ctypes

_CAPTURE_RELAXED = 2
_H2D = 1
_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence


def _runtime() -> ctypes.CDLL:
    paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps")
                    if "libamdhip64" in ln and ln.split()[-1].startswith("/")})
    return ctypes.CDLL(paths[0] if paths else "libamdhip64.so.7")


class HipRuntime:
    """Events, one captured graph, and raw async copies on a given stream."""

    def __init__(self):
        ct = ctypes
        self.ct = ct
        self.hip = hip = _runtime()
        hip.hipEventCreate.argtypes = [ct.POINTER(ct.c_void_p)]
        hip.hipEventCreateWithFlags.argtypes = [ct.POINTER(ct.c_void_p), ct.c_uint]
        hip.hipEventRecord.argtypes = [ct.c_void_p, ct.c_void_p]
        hip.hipStreamWaitEvent.argtypes = [ct.c_void_p, ct.c_void_p, ct.c_uint]
        hip.hipEventElapsedTime.argtypes = [ct.POINTER(ct.c_float), ct.c_void_p, ct.c_void_p]
        hip.hipEventDestroy.argtypes = [ct.c_void_p]
        hip.hipStreamBeginCapture.argtypes = [ct.c_void_p, ct.c_int]
        hip.hipStreamEndCapture.argtypes = [ct.c_void_p, ct.POINTER(ct.c_void_p)]
        hip.hipGraphInstantiate.argtypes = [ct.POINTER(ct.c_void_p), ct.c_void_p, ct.c_void_p,
                                            ct.c_void_p, ct.c_size_t]
        hip.hipGraphLaunch.argtypes = [ct.c_void_p, ct.c_void_p]
        hip.hipGraphUpload.argtypes = [ct.c_void_p, ct.c_void_p]
        hip.hipGraphExecDestroy.argtypes = [ct.c_void_p]
        hip.hipGraphDestroy.argtypes = [ct.c_void_p]
        hip.hipMemcpyAsync.argtypes = [ct.c_void_p, ct.c_void_p, ct.c_size_t, ct.c_int,
                                       ct.c_void_p]
        hip.hipMemcpy2DAsync.argtypes = [ct.c_void_p, ct.c_size_t, ct.c_void_p, ct.c_size_t,
                                         ct.c_size_t, ct.c_size_t, ct.c_int, ct.c_void_p]
        self.made = []
        self.graph = self.exec = None

    # -- events -------------------------------------------------------------
    def new_event(self, system_fence: bool = True):
        """An event; ``system_fence`` False: its records release to device
        scope only (hipEventDisableSystemFence), for events that only time
        kernels -- the system-scope release costs each record about a
        microsecond that would be counted as kernel time."""
        e = self.ct.c_void_p()
        rc = (self.hip.hipEventCreate(self.ct.byref(e)) if system_fence else
              self.hip.hipEventCreateWithFlags(self.ct.byref(e), _EVENT_DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed")
        self.made.append(e)
        return e

    def record(self, e, stream: int) -> None:
        if self.hip.hipEventRecord(e, self.ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def wait(self, stream: int, e) -> None:
        """Work enqueued on ``stream`` after this waits for event ``e``."""
        if self.hip.hipStreamWaitEvent(self.ct.c_void_p(stream), e, 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    # -- capture and replay ---------------------------------------------------
    def begin_capture(self, stream: int) -> None:
        if self.exec is not None:
            raise RuntimeError("destroy the previous graph first")
        if self.hip.hipStreamBeginCapture(self.ct.c_void_p(stream), _CAPTURE_RELAXED) != 0:
            raise RuntimeError("hipStreamBeginCapture failed")

    def end_capture(self, stream: int) -> None:
        ct = self.ct
        g, ge = ct.c_void_p(), ct.c_void_p()
        if self.hip.hipStreamEndCapture(ct.c_void_p(stream), ct.byref(g)) != 0:
            raise RuntimeError("hipStreamEndCapture failed")
        if self.hip.hipGraphInstantiate(ct.byref(ge), g, None, None, 0) != 0:
            self.hip.hipGraphDestroy(g)
            raise RuntimeError("hipGraphInstantiate failed")
        self.graph, self.exec = g, ge

    def upload(self, stream: int) -> None:
        """Move the graph's launch resources to the device ahead of its first
        launch, which otherwise pays for that itself."""
        if self.hip.hipGraphUpload(self.exec, self.ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipGraphUpload failed")

    def launch(self, stream: int) -> None:
        if self.hip.hipGraphLaunch(self.exec, self.ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipGraphLaunch failed")

    def destroy_graph(self) -> None:
        if self.exec is not None:
            self.hip.hipGraphExecDestroy(self.exec)
            self.hip.hipGraphDestroy(self.graph)
            self.graph = self.exec = None

    # -- copies ---------------------------------------------------------------
    def memcpy_h2d(self, dst: int, src: int, nbytes: int, stream: int) -> None:
        ct = self.ct
        if self.hip.hipMemcpyAsync(ct.c_void_p(dst), ct.c_void_p(src), nbytes, _H2D,
                                   ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipMemcpyAsync failed")

    def memcpy2d_h2d(self, dst: int, dpitch: int, src: int, spitch: int, width: int,
                     height: int, stream: int) -> None:
        """`height` rows of `width` bytes, `spitch` apart in host memory and
        `dpitch` apart on the device, as one copy."""
        ct = self.ct
        if self.hip.hipMemcpy2DAsync(ct.c_void_p(dst), dpitch, ct.c_void_p(src), spitch, width,
                                     height, _H2D, ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipMemcpy2DAsync failed")

    def close(self) -> None:
        self.destroy_graph()
        for e in self.made:
            self.hip.hipEventDestroy(e)
        self.made = []
