"""The decode batch's ring of pinned slot stages, on the CPU with stand-in events.

A stage may be rewritten only once the step that last read it has finished.  DecodeBatch keeps
STAGES stages and records a completion event after every STAGE_EVENT_EVERY-th step; before step n
reuses stage n % STAGES it waits on the first recorded event at or after step n - STAGES.
"""
import types

import pytest

from paged_kv_cache_53_amd.runtime import DecodeBatch


class FakeEvent:
    def __init__(self, step, log):
        self.step, self.log = step, log

    def synchronize(self):
        self.log.append(self.step)


def _run(n_steps):
    waits, readers = [], {}
    b = types.SimpleNamespace(STAGES=DecodeBatch.STAGES, STAGE_EVENT_EVERY=DecodeBatch.STAGE_EVENT_EVERY,
                              step_events={})
    for n in range(n_steps):
        before = len(waits)
        stage = DecodeBatch._stage_for(b, n)
        if n >= b.STAGES:
            # the wait covers the step that last read this stage, and no step that has not been issued
            assert len(waits) == before + 1
            assert readers[stage] <= waits[-1] < n
        else:
            assert len(waits) == before
        readers[stage] = n
        if (n + 1) % b.STAGE_EVENT_EVERY == 0:      # what DecodeBatch.step records
            b.step_events[n] = FakeEvent(n, waits)
        assert len(b.step_events) <= b.STAGES // b.STAGE_EVENT_EVERY + 1
    return waits


def test_every_stage_reuse_waits_for_its_last_reader():
    waits = _run(200)
    assert len(waits) == 200 - DecodeBatch.STAGES
    assert waits == sorted(waits)


def test_ring_never_waits_more_than_it_must():
    # with events every E steps and S stages, a reuse waits for a step at most E - 1 past the reader
    waits = _run(64)
    for n, w in zip(range(DecodeBatch.STAGES, 64), waits):
        assert w - (n - DecodeBatch.STAGES) < DecodeBatch.STAGE_EVENT_EVERY


def test_ring_sizes_are_consistent():
    assert DecodeBatch.STAGES % DecodeBatch.STAGE_EVENT_EVERY == 0
    assert DecodeBatch.STAGE_EVENT_EVERY < DecodeBatch.STAGES
