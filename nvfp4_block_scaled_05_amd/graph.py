"""HIP-graph capture of a sequence of library calls.

The pages run the DiT forward as one CUDA graph launch instead of one launch
per kernel ("英伟达B200狂飙10.2倍！AI绘图告别龟速！", nmedialink.com, section
"CUDA Graphs"; the 8-GPU latency in the time-breakdown paragraph of "NVIDIA
介绍用TensorRT LLM VisualGen加速Blackwell上的FLUX 3 Image Klein…", sns.style).
Here the same is done on HIP through ``torch.cuda.CUDAGraph``: a callable
that enqueues NVFP4 / bf16 linear calls on the current stream is run once
eagerly (warm-up: device checks, allocator pools), then captured, and each
``replay()`` relaunches the recorded kernels with their recorded pointers.

What a replay reads and writes are the tensors the callable used during
capture: refresh inputs in place (``tensor.copy_``) before a replay; outputs
returned by the callable are overwritten by every replay.  The library's
kernels clear their own flags and counters (no memset nodes), so replays are
independent of one another.
"""

__all__ = ["Captured", "capture"]


class Captured:
    """A captured call sequence.  ``outputs`` is what the callable returned
    during capture; ``replay()`` reruns the sequence and returns it."""

    def __init__(self, graph, outputs):
        self.graph = graph
        self.outputs = outputs

    def replay(self):
        self.graph.replay()
        return self.outputs


def capture(fn, warmup=1):
    """Capture ``fn()`` (which enqueues work on the current stream) into a
    HIP graph after ``warmup`` eager runs on a side stream."""
    import torch
    side = torch.cuda.Stream()          # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outputs = fn()
    torch.cuda.synchronize()
    return Captured(graph, outputs)
