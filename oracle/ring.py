"""The per-layer KV cache as frames and slots.

[LL] 方法 §3 高效长推理: attention is limited to a fixed local window, so a layer's KV
cache size depends only on the window; the first frame-chunk is pinned as global sink
tokens, kept in the cache for good and joined to every layer's keys and values.
[DIST] 序列并行与注意力汇聚的协同设计: for multi-shot videos the sink is reset at every shot
boundary (the multi-shot sink option).

Readings taken (the pages give no formula):
  * sink = the first S frames of the current shot (frames B..B+S-1, B = the shot's first
    frame; B = 0 for a single shot), never evicted while the shot lasts; a shot boundary
    drops the previous shot's sink and pins the next S frames instead;
  * window = the W committed frames right before the current chunk, whatever shot they
    belong to;
  * the visible set is a set union: a frame in both the sink and the window counts once;
  * inside a chunk attention is bidirectional, across chunks it is causal.

Slot layout (a layout choice, not from the pages): W window slots come first, then S sink
slots. Every committed frame f enters window slot f mod W, evicting frame f-W; when the
evicted frame is a sink frame of the current shot it moves to sink slot W + (f-W-B). So a
layer holds exactly its visible committed frames, and they fill the slot prefix.
"""
from __future__ import annotations


def visible_frames(chunk: int, C: int, S: int, W: int, shot_start: int = 0) -> list[int]:
    """Frames whose keys the queries of chunk `chunk` attend to, ascending.

    s = chunk*C is the chunk's first frame, B = shot_start <= s the first frame of its shot;
    V = {B <= f < B+S} U {max(0, s-W) <= f < s} U {s <= f < s+C}, capped below s+C.
    """
    s = chunk * C
    B = shot_start
    if B > s:
        raise ValueError("the shot starts after the chunk")
    vis = set(range(B, min(B + S, s + C)))
    vis |= set(range(max(0, s - W), s))
    vis |= set(range(s, s + C))
    return sorted(vis)


def n_spilled(F: int, S: int, W: int, shot_start: int = 0) -> int:
    """Sink frames of the current shot that have left the window (so sit in sink slots)."""
    return min(max(F - W - shot_start, 0), S)


def held_frames(F: int, S: int, W: int, shot_start: int = 0) -> list[int]:
    """Frames a layer holds after F frames were committed, ascending: the current shot's sink
    frames that have left the window, then the window [max(0, F-W), F)."""
    B = shot_start
    return list(range(B, B + n_spilled(F, S, W, B))) + list(range(max(0, F - W), F))


def slot_of_frame(f: int, F: int, S: int, W: int, shot_start: int = 0) -> int:
    """Slot of held frame f after F frames were committed: window frames sit in slot f mod W,
    spilled sink frames in slot W + (f - B)."""
    if f >= F - W:
        return f % W
    return W + (f - shot_start)


def slot_map(F: int, S: int, W: int, shot_start: int = 0) -> list[int]:
    """slot -> frame id held there (-1 if empty), for W+S slots."""
    out = [-1] * (S + W)
    for f in held_frames(F, S, W, shot_start):
        out[slot_of_frame(f, F, S, W, shot_start)] = f
    return out


def valid_slots(F: int, S: int, W: int, shot_start: int = 0) -> int:
    """Number of held frames. Their slots always form the prefix [0, n) of the slot range:
    the window slots fill first, and a frame is only spilled once the window is full."""
    return min(F, W) + n_spilled(F, S, W, shot_start)


def chunk_of_frame(f: int, C: int) -> int:
    return f // C
