"""Pins of oracle/ring.py against the closed form of a sliding window."""

from hypothesis import given, settings, strategies as st

import numpy as np

from oracle.ring import RingModel


@settings(max_examples=300, deadline=None)
@given(cap=st.sampled_from([1, 3, 4, 18, 96]),
       sizes=st.lists(st.integers(1, 200), min_size=1, max_size=12))
def test_window_is_last_capacity_frames(cap, sizes):
    r = RingModel(cap)
    total = 0
    for n in sizes:
        sizes_n = min(n, 2 * cap)
        r.append([("frame", total + i) for i in range(sizes_n)])
        total += sizes_n
        # closed form: the retained frames are exactly [total - valid, total)
        valid = min(total, cap)
        assert r.valid_frames() == valid
        assert [f for f, _ in r.retained()] == list(range(total - valid, total))
        assert r.frames_written == total
        slots = r.expected_slots()
        # retained frames occupy slots 0..valid-1, each exactly once
        assert sorted(slots) == list(range(valid))
        for s, (f, p) in slots.items():
            assert p == ("frame", f) and f % cap == s


def test_append_larger_than_capacity_keeps_tail():
    r = RingModel(4)
    r.append(list(range(10)))
    assert [p for _, p in r.retained()] == [6, 7, 8, 9]
    assert r.expected_slots() == {2: (6, 6), 3: (7, 7), 0: (8, 8), 1: (9, 9)}


def test_evicted_then_retained_is_every_frame_in_order():
    # every appended frame either left the window (in append order) or is retained
    rng = np.random.default_rng(7)
    for cap in (1, 3, 4, 18):
        ring = RingModel(cap)
        total = 0
        for _ in range(12):
            n = int(rng.integers(1, 2 * cap + 1))
            ring.append([total + i for i in range(n)])
            total += n
            seen = [f for f, _ in ring.evicted] + [f for f, _ in ring.retained()]
            assert seen == list(range(total))
            assert all(p == f for f, p in ring.evicted)
            assert len(ring.evicted) == max(0, total - cap)
