"""Host logic of the two-stream layer schedules (``schedule.run_layers``,
``schedule.run_assemblies``),
checked on the CPU with recording stand-ins for torch's streams and events:
for every layer the assembly and the attention land on the right streams and
buffers, and the event waits give exactly the orderings the schedule needs
(selection before any assembly, assembly l before attention l, attention l
before the assembly that next overwrites its buffer, the side stream joined
back into the current stream at the end)."""
import contextlib
import sys
import types

import pytest

import non_prefix_kv_token_amd.schedule as schedule


class _Log:
    def __init__(self):
        self.ops = []  # (stream name, op, payload)
        self.current = None


class _Event:
    def __init__(self, log):
        self.log, self.stream, self.pos = log, None, None

    def record(self, stream):
        self.stream, self.pos = stream.name, len(stream.queue)
        stream.queue.append(("record", self))


class _Stream:
    def __init__(self, log, name):
        self.log, self.name, self.queue = log, name, []

    def wait_stream(self, other):
        ev = _Event(self.log)
        ev.record(other)
        self.wait_event(ev)

    def wait_event(self, ev):
        self.queue.append(("wait", ev))


def _fake_torch(log, main):
    cuda = types.SimpleNamespace()
    cuda.current_stream = lambda: log.current
    cuda.Event = lambda: _Event(log)

    @contextlib.contextmanager
    def stream(s):
        prev, log.current = log.current, s
        try:
            yield
        finally:
            log.current = prev

    cuda.stream = stream
    log.current = main
    return types.SimpleNamespace(cuda=cuda)


def _happens_before(streams, a, b):
    """Whether op a = (stream, index) must complete before op b starts: a is
    in the backward closure of b over stream order and event waits (a wait
    at index j on an event recorded at index p of stream s2 orders every op
    of s2 before p ahead of every op after j)."""
    reach = {}  # stream -> ops [0, reach) that precede b
    todo = [b]
    while todo:
        s, upto = todo.pop()
        lo = reach.get(s, 0)
        if upto <= lo:
            continue
        reach[s] = upto
        for kind, obj in streams[s].queue[lo:upto]:
            if kind == "wait":
                todo.append((obj.stream, obj.pos))
    return a[1] < reach.get(a[0], 0)


@pytest.mark.parametrize("n_layers", [1, 2, 5])
def test_run_layers_streams_buffers_and_order(monkeypatch, n_layers):
    log = _Log()
    main, side = _Stream(log, "main"), _Stream(log, "side")
    monkeypatch.setitem(sys.modules, "torch", _fake_torch(log, main))
    main.queue.append(("op", "select"))
    calls = []

    def assemble(l, b):
        calls.append(("assemble", l, b, log.current.name))
        log.current.queue.append(("op", ("assemble", l, b)))

    def attend(l, b):
        calls.append(("attend", l, b, log.current.name))
        log.current.queue.append(("op", ("attend", l, b)))

    schedule.run_layers(n_layers, assemble, attend, side)
    streams = {"main": main, "side": side}

    def where(op):
        for name, s in streams.items():
            for i, (kind, obj) in enumerate(s.queue):
                if kind == "op" and obj == op:
                    return name, i
        raise AssertionError(f"{op} not issued")

    # each layer: assembly on the side stream, attention on the current one,
    # buffer l % 2, issued in layer order
    assert calls == [c for l in range(n_layers)
                     for c in (("assemble", l, l % 2, "side"), ("attend", l, l % 2, "main"))]
    sel = where("select")
    for l in range(n_layers):
        a, t = where(("assemble", l, l % 2)), where(("attend", l, l % 2))
        assert _happens_before(streams, sel, a), f"layer {l}: assembly may start before the selection"
        assert _happens_before(streams, a, t), f"layer {l}: attention may start before its assembly"
        if l >= 2:  # the assembly overwrites the buffer attention l-2 read
            prev = where(("attend", l - 2, l % 2))
            assert _happens_before(streams, prev, a), f"layer {l}: buffer overwritten while still read"
    # the side stream's last op is ordered before whatever the current stream issues next
    main.queue.append(("op", "after"))
    assert _happens_before(streams, where(("assemble", n_layers - 1, (n_layers - 1) % 2)), where("after"))
    # and no more ordering than needed: assembly l + 1 is not made to wait for attention l
    if n_layers >= 2:
        assert not _happens_before(streams, where(("attend", 0, 0)), where(("assemble", 1, 1)))


@pytest.mark.parametrize("n_layers", [1, 2, 5])
def test_run_assemblies_streams_buffers_and_order(monkeypatch, n_layers):
    log = _Log()
    main, side = _Stream(log, "main"), _Stream(log, "side")
    monkeypatch.setitem(sys.modules, "torch", _fake_torch(log, main))
    main.queue.append(("op", "select"))
    calls = []

    def assemble(l, b):
        calls.append((l, b, log.current.name))
        log.current.queue.append(("op", ("assemble", l, b)))

    schedule.run_assemblies(n_layers, assemble, side)
    streams = {"main": main, "side": side}

    def where(op):
        for name, s in streams.items():
            for i, (kind, obj) in enumerate(s.queue):
                if kind == "op" and obj == op:
                    return name, i
        raise AssertionError(f"{op} not issued")

    # even layers on the current stream into buffer 0, odd ones on the side stream into buffer 1
    assert calls == [(l, l % 2, "main" if l % 2 == 0 else "side") for l in range(n_layers)]
    sel = where("select")
    main.queue.append(("op", "after"))
    for l in range(n_layers):
        a = where(("assemble", l, l % 2))
        assert _happens_before(streams, sel, a), f"layer {l}: assembly may start before the selection"
        if l >= 2:  # the same buffer two layers back is written first
            assert _happens_before(streams, where(("assemble", l - 2, l % 2)), a)
        assert _happens_before(streams, a, where("after")), f"layer {l}: not joined into the current stream"
    if n_layers >= 2:  # neighbours may overlap
        assert not _happens_before(streams, where(("assemble", 0, 0)), where(("assemble", 1, 1)))
