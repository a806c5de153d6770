"""bench.py's timed loop on the host (no GPU): with a fake event clock, the
per-stage times it reports must equal the intervals between the boundaries the
library would record, when it records only some of them (the first step's
start, every step's later boundaries, minus those a call marks back to back)."""
import importlib.util
import os
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


class _Clock:
    t = 0.0


class _Event:
    def __init__(self, enable_timing=True):
        self.t = None

    def record(self):
        self.t = _Clock.t

    def elapsed_time(self, other):
        return other.t - self.t


def _fake_torch():
    cuda = types.SimpleNamespace(Event=_Event, synchronize=lambda: None)
    return types.SimpleNamespace(cuda=cuda)


def _run(same_as_previous, stage_ms, steps=7, warmup=2):
    """A step enqueues stages of the given lengths; the library records event b
    (when given) at the end of stage b - 1 (event 0 at the step's start)."""
    bench = _bench()
    calls = []

    def step(events):
        calls.append(events)
        if events is not None and events[0] is not None:
            events[0].record()
        for b, ms in enumerate(stage_ms, start=1):
            _Clock.t += ms
            if events is not None and events[b] is not None:
                events[b].record()

    _Clock.t = 0.0
    ms_per_step, stages = bench.time_steps(_fake_torch(), step, steps, warmup, len(stage_ms) + 1,
                                           same_as_previous=same_as_previous)
    return calls, stages


def test_stages_with_two_events_per_step():
    calls, stages = _run((2,), [2.0, 0.0, 0.1])
    timed = calls[2:]
    assert calls[0] is None and calls[1] is None           # warm-up: no events
    assert timed[0][0] is not None                          # the first timed step's start
    assert all(c[0] is None for c in timed[1:])             # later starts: the previous end
    assert all(c[2] is None for c in timed)                 # back to back with event 1
    assert all(c[1] is not None and c[3] is not None for c in timed)
    assert abs(stages[0] - 2.0) < 1e-12 and stages[1] == 0.0 and abs(stages[2] - 0.1) < 1e-12


def test_stages_with_every_boundary():
    calls, stages = _run((), [0.01, 3.5, 0.05])
    assert all(c[1] is not None and c[2] is not None and c[3] is not None for c in calls[2:])
    for got, want in zip(stages, [0.01, 3.5, 0.05]):
        assert abs(got - want) < 1e-12
