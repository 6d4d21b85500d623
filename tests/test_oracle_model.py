"""Pins for oracle/model.py: the cache-path chunk attention against brute force over the full
history, and the invariants of the method:
  I1 window >= sequence length reduces to block-causal full attention (torch SDPA)
  I2 softmax rows sum to 1 (in test_oracle_attention)
  I3 evicted frames have zero influence
  I4 recache output equals recomputation from scratch
"""
import math

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import fp4, ring
from oracle.model import LayerModel, bruteforce_chunk
from windowed_attention_kv_amd import synth

from test_oracle_attention import sdpa


def _stream(shape, n_chunks, layer=0, **kw):
    """Chunk inputs for a stream: list of (q, k, v) synth Tensors."""
    return [synth.chunk_inputs(shape, layer, 0, c, **kw) for c in range(n_chunks)]


def _model(shape, **kw):
    return LayerModel(shape.sink_frames, shape.window_frames, shape.chunk_frames,
                      shape.tokens_per_frame, shape.heads, shape.head_dim, **kw)


SMALL_LAYER = synth.shrink(synth.CONFIGS["layer"], heads=2, tokens_per_frame=64, chunks=12)


@pytest.mark.parametrize("shape", [synth.CONFIGS["tiny"], SMALL_LAYER], ids=["tiny", "layer-small"])
def test_cache_path_vs_bruteforce(shape):
    m = _model(shape)
    chunks = _stream(shape, shape.chunks)
    hist_k, hist_v = [], []
    scale = 1 / math.sqrt(shape.head_dim)
    for c, (q, k, v) in enumerate(chunks):
        o = m.attn_chunk(q.values, k.values, v.values)
        hk = np.concatenate(hist_k + [k.values]).astype(np.float64)
        hv = np.concatenate(hist_v + [v.values]).astype(np.float64)
        ref = bruteforce_chunk(q.values, hk, hv, c, shape.chunk_frames, shape.sink_frames,
                               shape.window_frames, shape.tokens_per_frame, scale)
        assert np.max(np.abs(o - ref)) <= 1e-12, c
        m.commit(k.values, v.values)
        hist_k.append(k.values)
        hist_v.append(v.values)


def test_window_covering_everything_is_block_causal_attention():
    """I1: with W >= all frames the stream equals block-causal attention over the whole
    sequence (torch SDPA with a block mask)."""
    shape = synth.shrink(synth.CONFIGS["tiny"], window_frames=100)
    m = _model(shape)
    chunks = _stream(shape, 6)
    outs = []
    for q, k, v in chunks:
        outs.append(m.attn_chunk(q.values, k.values, v.values))
        m.commit(k.values, v.values)
    Q = np.concatenate([c[0].values for c in chunks]).astype(np.float64)
    K = np.concatenate([c[1].values for c in chunks]).astype(np.float64)
    V = np.concatenate([c[2].values for c in chunks]).astype(np.float64)
    grp = np.arange(Q.shape[0]) // shape.n_query
    ref = sdpa(Q, K, V, 1 / math.sqrt(shape.head_dim), grp[None, :] <= grp[:, None])
    assert np.max(np.abs(np.concatenate(outs) - ref)) <= 1e-12


def test_first_chunk_is_plain_attention():
    shape = synth.CONFIGS["tiny"]
    q, k, v = synth.chunk_inputs(shape, 0, 0, 0)
    o = _model(shape).attn_chunk(q.values, k.values, v.values)
    ref = sdpa(q.values.astype(np.float64), k.values.astype(np.float64),
               v.values.astype(np.float64), 1 / 8)
    assert np.max(np.abs(o - ref)) <= 1e-12


@pytest.mark.parametrize("shots", [(2,), (5,), (1, 2), (4, 9)])
def test_multi_shot_cache_path_vs_bruteforce(shots):
    """Multi-shot sink: new_shot() before the chunks in `shots`; every chunk matches brute
    force over the whole history with the sink taken from the chunk's own shot."""
    shape = SMALL_LAYER
    C = shape.chunk_frames
    m = _model(shape)
    chunks = _stream(shape, shape.chunks)
    hist_k, hist_v = [], []
    scale = 1 / math.sqrt(shape.head_dim)
    B = 0
    for c, (q, k, v) in enumerate(chunks):
        if c in shots:
            m.new_shot()
            B = c * C
        o = m.attn_chunk(q.values, k.values, v.values)
        hk = np.concatenate(hist_k + [k.values]).astype(np.float64)
        hv = np.concatenate(hist_v + [v.values]).astype(np.float64)
        ref = bruteforce_chunk(q.values, hk, hv, c, C, shape.sink_frames, shape.window_frames,
                               shape.tokens_per_frame, scale, shot_start=B)
        assert np.max(np.abs(o - ref)) <= 1e-12, c
        m.commit(k.values, v.values)
        hist_k.append(k.values)
        hist_v.append(v.values)


def test_new_shot_drops_the_old_sink():
    """After a shot boundary the old shot's sink frames stop mattering once they are out of
    the window, and the new shot's first chunk matters for every later chunk of the shot."""
    shape = synth.CONFIGS["tiny"]          # S = 3, W = 6, C = 3
    chunks = _stream(shape, 12)
    m1, m2, m3 = _model(shape), _model(shape), _model(shape)
    for c, (q, k, v) in enumerate(chunks):
        if c == 4:
            for m in (m1, m2, m3):
                m.new_shot()
        if c >= 4:
            a = m1.attn_chunk(q.values, k.values, v.values)
            b = m2.attn_chunk(q.values, k.values, v.values)
            np.testing.assert_array_equal(a, b)       # old sink (chunk 0) is gone
        if c >= 5:
            d = m3.attn_chunk(q.values, k.values, v.values)
            assert np.max(np.abs(a - d)) > 1e-3, c    # the new sink (chunk 4) is seen
        for m, kk, vv in ((m1, k.values, v.values),
                          (m2, k.values * (1.5 if c == 0 else 1.0), v.values + (1.0 if c == 0 else 0.0)),
                          (m3, k.values * (1.5 if c == 4 else 1.0), v.values + (1.0 if c == 4 else 0.0))):
            m.commit(kk, vv)


def test_evicted_frames_have_no_influence():
    """I3: the outputs do not change, bit for bit, when evicted frames are perturbed
    (cache path: poisoned with NaN; brute force: replaced by large finite values)."""
    shape = synth.CONFIGS["tiny"]
    S, W, C, T = 3, 6, 3, 16
    m = _model(shape)
    chunks = _stream(shape, 8)
    for c, (q, k, v) in enumerate(chunks):
        if c == 7:
            base = m.attn_chunk(q.values, k.values, v.values)
            held = set(m.held())
            for f in list(m.k):
                if f not in held:
                    m.k[f] = np.full_like(m.k[f], np.nan)
                    m.v[f] = np.full_like(m.v[f], np.nan)
            again = m.attn_chunk(q.values, k.values, v.values)
            np.testing.assert_array_equal(base, again)
            hk = np.concatenate([x[1].values for x in chunks]).astype(np.float64)
            hv = np.concatenate([x[2].values for x in chunks]).astype(np.float64)
            ref = bruteforce_chunk(q.values, hk, hv, c, C, S, W, T, 1 / 8)
            evicted = [f for f in range(c * C) if f not in held]
            assert evicted, "the stream must have evicted something by chunk 7"
            for f in evicted:
                hk[f * T:(f + 1) * T] = 1e6
                hv[f * T:(f + 1) * T] = -1e6
            ref2 = bruteforce_chunk(q.values, hk, hv, c, C, S, W, T, 1 / 8)
            np.testing.assert_array_equal(ref, ref2)
        m.commit(k.values, v.values)


def test_every_chunk_depends_on_the_sink():
    shape = synth.CONFIGS["tiny"]
    chunks = _stream(shape, 8)
    m1, m2 = _model(shape), _model(shape)
    for c, (q, k, v) in enumerate(chunks):
        if c >= 1:
            a = m1.attn_chunk(q.values, k.values, v.values)
            b = m2.attn_chunk(q.values, k.values, v.values)
            assert np.max(np.abs(a - b)) > 1e-3, c
        m1.commit(k.values, v.values)
        kk = k.values.copy()
        vv = v.values.copy()
        if c == 0:
            kk = kk * 1.5
            vv = vv + 1.0
        m2.commit(kk, vv)


def _recache_setup(shape, n_chunks, salt=0):
    m = _model(shape)
    for q, k, v in _stream(shape, n_chunks, salt=salt):
        m.commit(k.values, v.values)
    return m


@pytest.mark.parametrize("n_chunks", [1, 2, 4, 10])
def test_recache_equals_streaming_from_scratch(n_chunks):
    """I4: the block-causal prefill over the held frames equals streaming those frames
    chunk by chunk through a fresh cache; the cache afterwards holds the recache K/V."""
    shape = synth.CONFIGS["tiny"]
    m = _recache_setup(shape, n_chunks)
    frames = m.held()
    n = len(frames) * shape.tokens_per_frame
    q, k, v, qx, kt, vt = synth.recache_inputs(shape, 0, n, 20)
    o_self, o_cross = m.recache(q.values, k.values, v.values, qx.values, kt.values, vt.values)
    # fresh stream over the same rows, one chunk per group of held frames
    fresh = _model(shape)
    nq = shape.n_query
    assert n % nq == 0
    for g in range(n // nq):
        sl = slice(g * nq, (g + 1) * nq)
        o = fresh.attn_chunk(q.values[sl], k.values[sl], v.values[sl])
        assert np.max(np.abs(o - o_self[sl])) <= 1e-12, g
        fresh.commit(k.values[sl], v.values[sl])
    # block-causal SDPA
    grp = np.repeat([f // shape.chunk_frames for f in frames], shape.tokens_per_frame)
    ref = sdpa(q.values.astype(np.float64), k.values.astype(np.float64),
               v.values.astype(np.float64), 1 / 8, grp[None, :] <= grp[:, None])
    assert np.max(np.abs(ref - o_self)) <= 1e-12
    ref_x = sdpa(qx.values.astype(np.float64), kt.values.astype(np.float64),
                 vt.values.astype(np.float64), 1 / 8)
    assert np.max(np.abs(ref_x - o_cross)) <= 1e-12
    # frame ids and slots unchanged, values replaced
    K, _ = m.export_dense()
    for i, f in enumerate(frames):
        slot = ring.slot_of_frame(f, m.F, shape.sink_frames, shape.window_frames)
        T = shape.tokens_per_frame
        np.testing.assert_array_equal(K[slot * T:(slot + 1) * T], k.values[i * T:(i + 1) * T])


def test_recache_is_independent_of_old_contents():
    shape = synth.CONFIGS["tiny"]
    a = _recache_setup(shape, 7, salt=0)
    b = _recache_setup(shape, 7, salt=1)
    n = len(a.held()) * shape.tokens_per_frame
    ins = synth.recache_inputs(shape, 0, n, 16)
    ra = a.recache(*(t.values for t in ins))
    rb = b.recache(*(t.values for t in ins))
    np.testing.assert_array_equal(ra[0], rb[0])
    np.testing.assert_array_equal(ra[1], rb[1])
    q, k, v = synth.chunk_inputs(shape, 0, 0, 7, salt=5)
    np.testing.assert_array_equal(a.attn_chunk(q.values, k.values, v.values),
                                  b.attn_chunk(q.values, k.values, v.values))


def test_fp4_store_attends_to_dequantised_history():
    shape = synth.shrink(synth.CONFIGS["layer"], heads=2, tokens_per_frame=32, chunks=6)
    m = _model(shape, kv_format="fp4")
    d = _model(shape)
    u = _model(shape)
    for c, (q, k, v) in enumerate(_stream(shape, 6)):
        if c == 5:
            o = m.attn_chunk(q.values, k.values, v.values)
            ou = u.attn_chunk(q.values, k.values, v.values)
            assert np.max(np.abs(o - ou)) > 1e-4       # quantisation is visible
        m.commit(k.values, v.values, k.bits, v.bits)
        u.commit(k.values, v.values)
        # dense model fed with the round-tripped values must agree exactly
        d.commit(fp4.roundtrip(k.bits), fp4.roundtrip(v.bits))
        np.testing.assert_array_equal(m.k[c * 3], d.k[c * 3])
    q, k, v = synth.chunk_inputs(shape, 0, 0, 6)
    np.testing.assert_array_equal(m.attn_chunk(q.values, k.values, v.values),
                                  d.attn_chunk(q.values, k.values, v.values))
    kp, ks, vp, vs, valid = m.export_fp4()
    assert valid.sum() == 12 * 32 * 2


@pytest.mark.parametrize("D", [128, 64])
def test_rising_score_inputs_move_the_running_max(D):
    """The input recipe of the GPU rescale test (K of frame f scaled by 1 + 2f, 2 heads,
    T = 100, C = 3, S = 3, W = 5, 8 chunks) really moves a row's largest score in the middle of
    its key sweep: sweeping each chunk's keys in cache slot order and then the own chunk, in
    64-key steps, the exact running max (exp2 domain) rises by more than 8 within a step for
    over 1% of (row, step) pairs after the first step. A weight there exceeds 2^8, so any
    rescale rule with that bound must act mid-sweep."""
    T, C, S, W = 100, 3, 3, 5
    shape = synth.shrink(synth.CONFIGS["layer"], name="rising", heads=2, head_dim=D,
                         tokens_per_frame=T, window_frames=W)
    keys, steps, jumps = {}, 0, 0
    for c in range(8):
        q, k, _ = synth.chunk_inputs(shape, 0, 0, c, k_frame_gain=2.0)
        for i in range(C):
            keys[c * C + i] = k.values[i * T:(i + 1) * T]
        order = [f for f in ring.slot_map(c * C, S, W) if f >= 0] + [c * C + i for i in range(C)]
        z = oatt.logits(q.values, np.concatenate([keys[f] for f in order]),
                        1.0 / math.sqrt(D)) * math.log2(math.e)
        run = np.maximum.accumulate(z, axis=-1)
        n = z.shape[-1]
        for t0 in range(64, n, 64):
            before, after = run[..., t0 - 1], run[..., min(t0 + 63, n - 1)]
            steps += before.size
            jumps += int(np.sum(after > before + 8))
    assert jumps > 0.01 * steps, (jumps, steps)


def test_export_fp4_is_the_committed_frames_encoded_in_slot_order():
    """Pin of LayerModel.export_fp4, the reference of every FP4 export comparison. After every
    commit of a multi-shot stream, and after a recache, its planes equal an assembly built
    without the model: each held frame's slot from the frame-by-frame slot simulation of
    test_oracle_ring (explicit window FIFO and sink slots, not ring.slot_map), its codes and
    scales from fp4.quantize of the bf16 bits this test committed for that frame, every other
    row marked empty."""
    from test_oracle_ring import slot_simulation
    shape = synth.shrink(SMALL_LAYER, tokens_per_frame=8, window_frames=4)
    S, W, C, T, H, D = (shape.sink_frames, shape.window_frames, shape.chunk_frames,
                        shape.tokens_per_frame, shape.heads, shape.head_dim)
    shots, n_chunks = (5,), 10
    snaps = {F: slots for F, B, slots, held in
             slot_simulation(n_chunks * C, C, S, W, shot_starts={c * C for c in shots})}
    m = _model(shape, kv_format="fp4")
    bits = {}                # frame -> (K bits [T, H, D], V bits)

    def check():
        slots = snaps[m.F]
        kp, ks, vp, vs, valid = m.export_fp4()
        rows = T * H
        for slot, f in enumerate(slots):
            sl = slice(slot * rows, (slot + 1) * rows)
            assert bool(valid[sl].all()) == (f >= 0) and bool(valid[sl].any()) == (f >= 0)
            if f < 0:
                continue
            for got_p, got_s, b in ((kp, ks, bits[f][0]), (vp, vs, bits[f][1])):
                wp, ws = fp4.quantize(b.reshape(rows, D))
                assert np.array_equal(got_p[sl], wp) and np.array_equal(got_s[sl], ws), (m.F, slot, f)

    for c in range(n_chunks):
        _, k, v = synth.chunk_inputs(shape, 0, 0, c)
        m.commit(k.values, v.values, k.bits, v.bits)
        for i in range(C):
            bits[c * C + i] = (k.bits[i * T:(i + 1) * T], v.bits[i * T:(i + 1) * T])
        if c + 1 in shots:       # the simulation opens a shot at the boundary frame itself
            m.new_shot()
        check()
    held = m.held()
    ins = synth.recache_inputs(shape, 0, len(held) * T, 8)
    q, k, v, qx, kt, vt = ins
    m.recache(q.values, k.values, v.values, qx.values, kt.values, vt.values, k.bits, v.bits)
    for r, f in enumerate(held):
        bits[f] = (k.bits[r * T:(r + 1) * T], v.bits[r * T:(r + 1) * T])
    check()
