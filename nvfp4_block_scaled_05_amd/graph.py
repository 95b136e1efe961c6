"""HIP-graph capture of a sequence of library calls, through the library's
own C entry points (nvfp4_graph_begin / _end / _launch / _destroy).

The pages run the DiT forward as one CUDA graph launch instead of one launch
per kernel ("英伟达B200狂飙10.2倍！AI绘图告别龟速！", nmedialink.com, section
"CUDA Graphs"; the 8-GPU latency in the time-breakdown paragraph of "NVIDIA
介绍用TensorRT LLM VisualGen加速Blackwell上的FLUX 3 Image Klein…", sns.style).
Here a callable that enqueues NVFP4 / bf16 linear calls on the current stream
is run eagerly on a side stream (warm-up: device checks, workspaces), then
run once more between nvfp4_graph_begin and nvfp4_graph_end on that stream;
each ``replay()`` enqueues the recorded kernels, with their recorded pointers,
on the current stream.  torch supplies only the side stream here.

The callable must not allocate device memory while it is captured (pass
``out=`` and workspaces; the warm-up run creates any default workspace).
What a replay reads and writes are the tensors the callable used during
capture: refresh inputs in place (``tensor.copy_``) before a replay; outputs
returned by the callable are overwritten by every replay.  The library's
kernels clear or keep consistent their own flags and counters (no memset
nodes), so replays are independent of one another.
"""

import ctypes

from ._binding import check, load

__all__ = ["Captured", "capture"]


class Captured:
    """A captured call sequence.  ``outputs`` is what the callable returned
    during capture; ``replay()`` reruns the sequence and returns it."""

    def __init__(self, handle, outputs, keep):
        self._handle = handle
        self.outputs = outputs
        self._keep = keep                 # the capture stream outlives the graph

    def replay(self):
        import torch
        check(load().nvfp4_graph_launch(self._handle, torch.cuda.current_stream().cuda_stream),
              "nvfp4_graph_launch")
        return self.outputs

    def __del__(self):
        if self._handle:
            load().nvfp4_graph_destroy(self._handle)
            self._handle = None


def capture(fn, warmup=1):
    """Capture ``fn()`` (which enqueues work on the current stream) into a
    HIP graph after ``warmup`` eager runs on a side stream."""
    import torch
    lib = load()
    side = torch.cuda.Stream()          # default priority; capturable (not the null stream)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    handle = ctypes.c_void_p()
    with torch.cuda.stream(side):
        check(lib.nvfp4_graph_begin(side.cuda_stream), "nvfp4_graph_begin")
        try:
            outputs = fn()
        finally:
            rc = lib.nvfp4_graph_end(side.cuda_stream, ctypes.byref(handle))
    check(rc, "nvfp4_graph_end")
    torch.cuda.synchronize()
    return Captured(handle.value, outputs, side)
