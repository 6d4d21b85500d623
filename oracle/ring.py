"""The per-layer KV cache as frames and slots.

[LL] 方法 §3 高效长推理: attention is limited to a fixed local window, so a layer's KV
cache size depends only on the window; the first frame-chunk is pinned as global sink
tokens, kept in the cache for good and joined to every layer's keys and values.

Readings taken (the pages give no formula):
  * sink = frames 0..S-1 (the first chunk when S = C), never evicted;
  * window = the W committed frames right before the current chunk;
  * the visible set is a set union: a frame in both the sink and the window counts once;
  * inside a chunk attention is bidirectional, across chunks it is causal.
"""
from __future__ import annotations


def visible_frames(chunk: int, C: int, S: int, W: int) -> list[int]:
    """Frames whose keys the queries of chunk `chunk` attend to, ascending.

    s = chunk*C is the chunk's first frame;
    V = {f < S} U {max(0, s-W) <= f < s} U {s <= f < s+C}.
    """
    s = chunk * C
    vis = set(range(min(S, s + C)))
    vis |= set(range(max(0, s - W), s))
    vis |= set(range(s, s + C))
    return sorted(vis)


def slot_of_frame(f: int, S: int, W: int) -> int:
    """Slot that frame f occupies: sink frames keep their own slot, window frames rotate
    through W slots after the sink, so writing frame f evicts frame f-W."""
    if f < S:
        return f
    return S + (f - S) % W


def held_frames(F: int, S: int, W: int) -> list[int]:
    """Frames a layer holds after F frames were committed, ascending:
    {f < min(F,S)} U [max(S, F-W), F)."""
    return list(range(min(F, S))) + list(range(max(S, F - W), F))


def slot_map(F: int, S: int, W: int) -> list[int]:
    """slot -> frame id held there (-1 if empty), for S+W slots."""
    out = [-1] * (S + W)
    for f in held_frames(F, S, W):
        out[slot_of_frame(f, S, W)] = f
    return out


def valid_slots(F: int, S: int, W: int) -> int:
    """Number of filled slots. They always form the prefix [0, n) of the slot range."""
    return min(F, S) + min(max(F - S, 0), W)


def chunk_of_frame(f: int, C: int) -> int:
    return f // C
