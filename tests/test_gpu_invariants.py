"""Properties of the rolling cache that the pages state outright, checked on the GPU between runs
of the library itself (no oracle in the comparison, so every check is bitwise):

- the sink frames are kept for good: once the first chunk is committed, the first S frames'
  bytes never change while the stream runs, in their window slots and, once the window has
  wrapped, in the sink slots W..W+S-1 they are moved to (LongLive page, frame-sink section);
- a prompt switch's recache rebuilds the cache from the held frames' new K/V alone: after it,
  the cache bytes and every later output are the same whatever the cache held before, and the
  same as a fresh cache that was streamed those new K/V (LongLive page, KV-recache section)."""
import numpy as np
import pytest

from _parity import log
from windowed_attention_kv_amd import synth

pytestmark = pytest.mark.gpu

SHAPE = synth.shrink(synth.CONFIGS["layer"], name="invariants", heads=2, tokens_per_frame=64)


def _cache(kv_format):
    from windowed_attention_kv_amd import Cache
    s = SHAPE
    return Cache(1, s.heads, s.head_dim, s.tokens_per_frame, s.chunk_frames, s.sink_frames,
                 s.window_frames, dtype=s.dtype, kv_format=kv_format)


def _export(cache):
    """The layer's cache bytes in slot order, as host byte arrays."""
    import torch
    planes = cache.export(0)
    torch.cuda.synchronize()
    return [p.contiguous().view(torch.uint8).cpu().numpy() for p in planes]


def _rows_per_frame(cache):
    """Rows of each exported plane per frame (dense planes are [rows, H, D]; FP4 planes
    [rows * H, bytes])."""
    T, H = SHAPE.tokens_per_frame, SHAPE.heads
    return T if cache.kv_format == "dense" else T * H


def _logical(cache, planes):
    """Exported planes with their frames put in committed order (oldest first)."""
    _, slots = cache.state(0)
    order = [s for _, s in sorted((f, s) for s, f in enumerate(slots) if f >= 0)]
    r = _rows_per_frame(cache)
    return [np.concatenate([p[s * r:(s + 1) * r] for s in order]) for p in planes]


def _stream(cache, n_chunks, salt):
    for c in range(n_chunks):
        _, k, v = synth.chunk_inputs(SHAPE, 0, 0, c, salt=salt)
        cache.commit(0, k.torch("cuda"), v.torch("cuda"))


def _frame_bytes(cache, planes, frame):
    """The bytes of committed frame `frame` in every exported plane, wherever its slot is."""
    _, slots = cache.state(0)
    s = slots.index(frame)
    r = _rows_per_frame(cache)
    return [p[s * r:(s + 1) * r].copy() for p in planes]


@pytest.mark.parametrize("kv_format", ["dense", "fp4"])
def test_sink_frames_never_change_while_streaming(kv_format):
    """The first S frames are written by the first commit, move from their window slots to the
    sink slots when the window wraps, and keep the same bytes for the rest of the stream."""
    import torch
    log(f"case: sink bytes over a stream, {kv_format}")
    cache = _cache(kv_format)
    S, W = SHAPE.sink_frames, SHAPE.window_frames
    first = None
    moved = False
    for c in range(10):
        q, k, v = (t.torch("cuda") for t in synth.chunk_inputs(SHAPE, 0, 0, c, salt=31))
        cache.attn_chunk(0, q, k, v)
        cache.commit(0, k, v)
        planes = _export(cache)
        now = [_frame_bytes(cache, planes, f) for f in range(S)]
        if first is None:
            first = now
        for f in range(S):
            for i, (x, y) in enumerate(zip(now[f], first[f])):
                assert np.array_equal(x, y), f"chunk {c}: bytes of sink frame {f}, plane {i}"
        F, slots = cache.state(0)
        moved = moved or slots[W:] == list(range(S))
    assert F == 10 * SHAPE.chunk_frames
    assert moved, "the window never wrapped: the sink frames were not moved"
    torch.cuda.synchronize()


@pytest.mark.parametrize("kv_format", ["dense", "fp4"])
def test_recache_forgets_the_old_contents(kv_format):
    """Two caches with different histories (12 and 21 frames of unrelated K/V) are recached
    with the same inputs; a third cache is streamed the recache's K/V from empty. All three
    then hold the same bytes frame for frame, and the recache outputs and the next chunk's
    outputs are bitwise the same. The frame counts are chosen so that the window's oldest frame
    sits in the same slot in all three, so the kernels sweep the keys in the same order."""
    import torch
    log(f"case: recache independence, {kv_format}")
    s = SHAPE
    C, S, W, T = s.chunk_frames, s.sink_frames, s.window_frames, s.tokens_per_frame
    a, b, fresh = _cache(kv_format), _cache(kv_format), _cache(kv_format)
    _stream(a, 4, salt=41)
    _stream(b, 7, salt=42)
    held = S + W
    n = held * T
    assert a.held_rows(0) == b.held_rows(0) == n
    q, k, v, qx, kt, vt = (t.torch("cuda") for t in synth.recache_inputs(s, 0, n, 48))
    oa, oxa = a.recache(0, q, k, v, qx, kt, vt)
    ob, oxb = b.recache(0, q, k, v, qx, kt, vt)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob), "recache self-attention depends on the old cache contents"
    assert torch.equal(oxa, oxb), "recache cross-attention depends on the old cache contents"
    for c in range(held // C):
        rows = slice(c * C * T, (c + 1) * C * T)
        fresh.commit(0, k[rows], v[rows])
    logical = [_logical(x, _export(x)) for x in (a, b, fresh)]
    for i in range(len(logical[0])):
        assert np.array_equal(logical[0][i], logical[1][i]), f"plane {i}: a != b after recache"
        assert np.array_equal(logical[0][i], logical[2][i]), f"plane {i}: recache != fresh"
    slots = [x.state(0)[1] for x in (a, b, fresh)]
    oldest = [sl.index(min(sl[:W])) for sl in slots]
    assert oldest[0] == oldest[1] == oldest[2], f"window starts at slots {oldest}"
    for c in range(2):
        qq, kk, vv = (t.torch("cuda") for t in synth.chunk_inputs(s, 0, 0, 20 + c, salt=43))
        outs = [x.attn_chunk(0, qq, kk, vv) for x in (a, b, fresh)]
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"chunk {c} after recache: a != b"
        assert torch.equal(outs[0], outs[2]), f"chunk {c} after recache: recache != fresh"
        for x in (a, b, fresh):
            x.commit(0, kk, vv)
