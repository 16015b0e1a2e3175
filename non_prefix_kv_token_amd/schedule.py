"""Two-stream schedule of the per-layer calls of a request.

The assembly of a layer's working buffer (gather, scatter and deferred RoPE)
depends only on the selection and that layer's rows, not on the attention of
the layer before it.  The CacheTune page (Sec. 4.2, App. B.2) runs positional
recovery and the buffer fill on a stream of their own and hands each layer's
buffer to that layer's attention through per-layer events, so that work for
the next layer proceeds while the current one computes.  With two
assembled-cache buffers, ``run_layers`` therefore issues the assembly of
layer l on a side stream and the attention of layer l on the caller's
current stream: the assembly of layer l + 1 can run while the attention of
layer l still occupies the GPU (in particular in the attention kernel's
tail, where compute units idle).

Ordering is kept with events only; nothing here computes or allocates device
memory, and the same calls made in order on one stream give the same
results bit for bit:

* the side stream first waits for everything already issued on the current
  stream (the scoring and the selection, and every earlier reader of both
  buffers);
* the attention of layer l waits for the assembly of layer l;
* the assembly into buffer b waits for the attention that last read b.

The side stream joins back into the current stream before the function
returns (the current stream waited for the last assembly), so the function
can be captured into a HIP graph on the current stream.  Both streams keep
the default priority.

``run_assemblies`` is the same hand-off without the attention: the path that
only assembles every layer (score, top-r, assembly) issues even layers on the
current stream into buffer 0 and odd layers on the side stream into buffer 1.
Neighbouring layers' assemblies write different buffers and read only the
selection and their own rows, so each launch's ramp-down overlaps the next
one's ramp-up; a layer two apart writes the same buffer on the same stream.
"""
from __future__ import annotations

from typing import Callable


def run_layers(n_layers: int, assemble: Callable[[int, int], None], attend: Callable[[int, int], None],
               side) -> None:
    """Issue ``assemble(l, b)`` on ``side`` and ``attend(l, b)`` on the current
    stream for l < n_layers, with b = l % 2 the assembled-cache buffer."""
    import torch

    main = torch.cuda.current_stream()
    side.wait_stream(main)
    last_read = [None, None]
    for l in range(n_layers):
        b = l % 2
        if last_read[b] is not None:
            side.wait_event(last_read[b])
        with torch.cuda.stream(side):
            assemble(l, b)
        ready = torch.cuda.Event()
        ready.record(side)
        main.wait_event(ready)
        attend(l, b)
        done = torch.cuda.Event()
        done.record(main)
        last_read[b] = done


def run_assemblies(n_layers: int, assemble: Callable[[int, int], None], side) -> None:
    """Issue ``assemble(l, b)`` for l < n_layers with b = l % 2: buffer 0 on
    the current stream, buffer 1 on ``side``, after everything already issued
    on the current stream; the current stream then waits for the side one."""
    import torch

    main = torch.cuda.current_stream()
    side.wait_stream(main)
    for l in range(n_layers):
        if l % 2 == 0:
            assemble(l, 0)
        else:
            with torch.cuda.stream(side):
                assemble(l, 1)
    main.wait_stream(side)
