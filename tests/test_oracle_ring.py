"""Pins for oracle/ring.py: the slot map and held frames against a FIFO simulation, and
the visible-frame set against the eviction rule."""
import collections

import pytest

from oracle import ring


def fifo_simulation(n_frames, C, S, W):
    """Frame-by-frame cache simulation with an explicit FIFO of window frames: sink frames
    get slots 0..S-1 in arrival order; a window frame takes the next free window slot or,
    when the window is full, the slot of the frame it pushes out of the FIFO."""
    sink = []
    fifo = collections.deque()
    slot_of = {}
    free = list(range(S, S + W))
    snapshots = []
    for f in range(n_frames):
        if len(sink) < S:
            slot_of[f] = len(sink)
            sink.append(f)
        else:
            if len(fifo) == W:
                old = fifo.popleft()
                slot = slot_of.pop(old)
            else:
                slot = free.pop(0)
            slot_of[f] = slot
            fifo.append(f)
        if (f + 1) % C == 0:
            slots = [-1] * (S + W)
            for fr, sl in slot_of.items():
                slots[sl] = fr
            snapshots.append((f + 1, slots, sorted(sink + list(fifo))))
    return snapshots


@pytest.mark.parametrize("S", range(0, 5))
@pytest.mark.parametrize("W", range(1, 13))
@pytest.mark.parametrize("C", range(1, 5))
def test_ring_vs_fifo(S, W, C):
    n = 600 if (S + W) < 8 else 300
    for F, slots, held in fifo_simulation(n * C, C, S, W):
        assert ring.slot_map(F, S, W) == slots
        assert ring.held_frames(F, S, W) == held
        nv = ring.valid_slots(F, S, W)
        assert all(x >= 0 for x in slots[:nv]) and all(x < 0 for x in slots[nv:])


def test_long_stream_constant_memory():
    """10^4 frames: the number of slots never grows and only the last W frames plus the
    sink are held (cache size depends only on the window)."""
    S, W, C = 3, 9, 3
    for F in range(0, 10_000, C):
        held = ring.held_frames(F, S, W)
        assert len(held) <= S + W
        if F >= S + W:
            assert held == list(range(S)) + list(range(F - W, F))


@pytest.mark.parametrize("S,W,C", [(3, 6, 3), (3, 9, 3), (2, 5, 3), (0, 4, 2), (4, 3, 1)])
def test_visible_committed_frames_are_exactly_the_held_frames(S, W, C):
    for c in range(40):
        s = c * C
        vis = ring.visible_frames(c, C, S, W)
        assert vis == sorted(set(vis))
        assert [f for f in vis if f >= s] == list(range(s, s + C))
        committed = [f for f in vis if f < s]
        assert committed == ring.held_frames(s, S, W)


def test_visible_counts_layer_config():
    # 1560-token frames, chunk 3, sink 3, window 9: 3, 6, 9, 12, 15, 15, ... frames
    counts = [len(ring.visible_frames(c, 3, 3, 9)) for c in range(8)]
    assert counts == [3, 6, 9, 12, 15, 15, 15, 15]
    # tiny: 16-token frames, chunk 3, sink 3, window 6: 3, 6, 9, 12, 12, ...
    counts = [len(ring.visible_frames(c, 3, 3, 6)) for c in range(8)]
    assert counts == [3, 6, 9, 12, 12, 12, 12, 12]
