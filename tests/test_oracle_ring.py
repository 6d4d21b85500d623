"""Pins for oracle/ring.py: the slot map and held frames against a frame-by-frame slot
simulation (single shot and multi-shot), and the visible-frame set against the eviction
rule."""
import collections

import pytest

from oracle import ring


def slot_simulation(n_frames, C, S, W, shot_starts=()):
    """Frame-by-frame cache with explicit slot lists. Window slots 0..W-1 are handed out in
    order and then reused by FIFO: a frame takes the slot of the frame it pushes out of the
    window. A pushed-out frame that is one of the current shot's first S frames moves to sink
    slot W + (its index in the shot). A new shot (at a frame in `shot_starts`) forgets the
    previous shot's sink frames. Yields (frames committed, slot -> frame, held frames) at
    every chunk boundary."""
    fifo = collections.deque()
    slot_of = {}
    sink = {}
    free = list(range(W))
    shot = 0
    snapshots = []
    for f in range(n_frames):
        if f in shot_starts:
            shot = f
            sink = {}
        if len(fifo) == W:
            old = fifo.popleft()
            slot = slot_of.pop(old)
            if shot <= old < shot + S:
                sink[old] = W + (old - shot)
        else:
            slot = free.pop(0)
        slot_of[f] = slot
        fifo.append(f)
        if (f + 1) % C == 0:
            F = f + 1
            if F in shot_starts:        # a shot starting at the next frame is already open
                shot_now, sink_now = F, {}
            else:
                shot_now, sink_now = shot, sink
            slots = [-1] * (S + W)
            for fr, sl in list(slot_of.items()) + list(sink_now.items()):
                slots[sl] = fr
            snapshots.append((F, shot_now, slots, sorted(list(fifo) + list(sink_now))))
    return snapshots


@pytest.mark.parametrize("S", range(0, 5))
@pytest.mark.parametrize("W", range(1, 13))
@pytest.mark.parametrize("C", range(1, 5))
def test_ring_vs_simulation_single_shot(S, W, C):
    n = 600 if (S + W) < 8 else 300
    for F, B, slots, held in slot_simulation(n * C, C, S, W):
        assert B == 0
        assert ring.slot_map(F, S, W) == slots
        assert ring.held_frames(F, S, W) == held
        nv = ring.valid_slots(F, S, W)
        assert nv == len(held)
        assert all(x >= 0 for x in slots[:nv]) and all(x < 0 for x in slots[nv:])


@pytest.mark.parametrize("S", range(0, 5))
@pytest.mark.parametrize("W", range(1, 11))
@pytest.mark.parametrize("C", range(1, 4))
def test_ring_vs_simulation_multi_shot(S, W, C):
    # shots of 1, 2, 5 and 17 chunks, and two boundaries in a row
    starts = {c * C for c in (1, 3, 8, 25, 26, 40)}
    for F, B, slots, held in slot_simulation(60 * C, C, S, W, starts):
        assert ring.slot_map(F, S, W, B) == slots, (F, B)
        assert ring.held_frames(F, S, W, B) == held
        nv = ring.valid_slots(F, S, W, B)
        assert nv == len(held)
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
@pytest.mark.parametrize("shot_chunk", [None, 1, 4, 7])
def test_visible_committed_frames_are_exactly_the_held_frames(S, W, C, shot_chunk):
    B = 0
    for c in range(40):
        s = c * C
        if shot_chunk is not None and c == shot_chunk:
            B = s
        vis = ring.visible_frames(c, C, S, W, B)
        assert vis == sorted(set(vis))
        assert [f for f in vis if f >= s] == list(range(s, s + C))
        committed = [f for f in vis if f < s]
        assert committed == ring.held_frames(s, S, W, B)


def test_visible_counts_layer_config():
    # 1560-token frames, chunk 3, sink 3, window 9: 3, 6, 9, 12, 15, 15, ... frames
    counts = [len(ring.visible_frames(c, 3, 3, 9)) for c in range(8)]
    assert counts == [3, 6, 9, 12, 15, 15, 15, 15]
    # tiny: 16-token frames, chunk 3, sink 3, window 6: 3, 6, 9, 12, 12, ...
    counts = [len(ring.visible_frames(c, 3, 3, 6)) for c in range(8)]
    assert counts == [3, 6, 9, 12, 12, 12, 12, 12]


def test_new_shot_resets_the_sink():
    """Layer config, shot boundary at chunk 10 (frame 30): the first chunk of the new shot
    sees only the window (frames 21..29) and itself; three chunks later the new shot's first
    chunk is its sink and the old sink frames 0..2 are gone."""
    C, S, W = 3, 3, 9
    assert ring.visible_frames(10, C, S, W, 0) == [0, 1, 2] + list(range(21, 33))
    assert ring.visible_frames(10, C, S, W, 30) == list(range(21, 33))
    assert ring.visible_frames(11, C, S, W, 30) == list(range(24, 36))
    assert ring.visible_frames(14, C, S, W, 30) == [30, 31, 32] + list(range(33, 45))
    assert ring.held_frames(42, S, W, 30) == [30, 31, 32] + list(range(33, 42))
    # the old shot's sink is still visible while inside the window of a short shot
    assert ring.visible_frames(2, C, S, W, 3) == list(range(0, 9))
