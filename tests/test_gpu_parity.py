"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Bit-exact: slot maps, exported cache bytes (dense copies, FP4 packed codes and scales),
ll_kv_quant. Toleranced: attention outputs (bf16: max-abs <= 1e-2 and rel-L2 <= 5e-3; fp32:
1e-5), compared per call against the unrounded oracle.
"""
import math

import numpy as np
import pytest

from _parity import assert_close, log, sample_rows, to_np
from oracle import attention as oatt
from oracle import fp4 as ofp4
from oracle import ring
from oracle.model import LayerModel
from windowed_attention_kv_amd import synth

pytestmark = pytest.mark.gpu


def _cache(shape, kv_format="dense", layers=1):
    from windowed_attention_kv_amd import Cache
    return Cache(layers, shape.heads, shape.head_dim, shape.tokens_per_frame, shape.chunk_frames,
                 shape.sink_frames, shape.window_frames, dtype=shape.dtype, kv_format=kv_format)


def _model(shape, kv_format="dense"):
    return LayerModel(shape.sink_frames, shape.window_frames, shape.chunk_frames,
                      shape.tokens_per_frame, shape.heads, shape.head_dim, kv_format=kv_format)


def _check_export(cache, model, shape, layer=0):
    import torch
    torch.cuda.synchronize()
    F, slots = cache.state(layer)
    assert F == model.F and slots == model.slot_map()
    T, H = shape.tokens_per_frame, shape.heads
    if cache.kv_format == "fp4":
        kp, ks, vp, vs = (x.cpu().numpy() for x in cache.export(layer))
        mkp, mks, mvp, mvs, valid = model.export_fp4()
        for got, want, name in ((kp, mkp, "K packed"), (ks, mks, "K scales"),
                                (vp, mvp, "V packed"), (vs, mvs, "V scales")):
            np.testing.assert_array_equal(got[valid], want[valid], err_msg=name)
    else:
        K, V = (to_np(x) for x in cache.export(layer))
        MK, MV = model.export_dense()
        valid = ~np.isnan(MK[:, 0, 0])
        np.testing.assert_array_equal(K[valid], MK[valid])
        np.testing.assert_array_equal(V[valid], MV[valid])
        assert valid.sum() == ring.valid_slots(model.F, shape.sink_frames, shape.window_frames,
                                               model.B) * T


def run_stream(shape, n_chunks, kv_format="dense", compare=None, rows=None, steps=1,
               export_every=True, shots=(), **kw):
    """Stream n_chunks through the library and the oracle; compare the chunks in `compare`
    (default all) on `rows` (default all) for every denoise step. A new shot starts before
    each chunk in `shots`."""
    cache = _cache(shape, kv_format)
    model = _model(shape, kv_format)
    worst = (0.0, 0.0)
    for c in range(n_chunks):
        if c in shots:
            cache.new_shot()
            model.new_shot()
        for step in range(steps):
            q, k, v = synth.chunk_inputs(shape, 0, step, c, **kw)
            tq, tk, tv = q.torch("cuda"), k.torch("cuda"), v.torch("cuda")
            o = cache.attn_chunk(0, tq, tk, tv)
            if compare is None or c in compare:
                r = rows if rows is not None else np.arange(shape.n_query)
                ref = model.attn_chunk(q.values, k.values, v.values, rows=r)
                ma, rl = assert_close(to_np(o)[r], ref, shape.dtype, f"chunk {c} step {step}")
                worst = (max(worst[0], ma), max(worst[1], rl))
        cache.commit(0, tk, tv)
        model.commit(k.values, v.values, k.bits, v.bits)
        if export_every or c == n_chunks - 1:
            _check_export(cache, model, shape)
    log(f"{shape.name} {kv_format}: worst max-abs {worst[0]:.3e} rel-L2 {worst[1]:.3e}")
    return cache, model


def test_tiny_fp32_stream():
    log("case: tiny fp32 stream, 8 chunks")
    run_stream(synth.CONFIGS["tiny"], 8)


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_ragged_stream(D):
    shape = synth.shrink(synth.CONFIGS["layer"], name=f"ragged-d{D}", heads=3, head_dim=D,
                         tokens_per_frame=100, window_frames=5)
    log(f"case: bf16 ragged stream D={D}")
    run_stream(shape, 9)


def test_bf16_peaked_and_frame_offsets():
    shape = synth.shrink(synth.CONFIGS["layer"], name="peaked", heads=2, tokens_per_frame=72,
                         window_frames=4)
    log("case: bf16 peaked Q/K, V with per-frame offsets")
    run_stream(shape, 7, peaked=True, v_frame_offset=0.25)


@pytest.mark.parametrize("kind", ["bf16-d128", "bf16-d64", "fp4"])
def test_rising_scores_force_rescales(kind):
    """K of frame f scaled by 1 + 2f: the keys of later frames give ever larger scores, so a
    row's largest score keeps jumping while its keys are swept (slot order is not time order,
    and the own chunk comes last). That drives the kernels' running-max rescale of O and the
    row sum in the middle of a sweep, not only on its first tile: on these inputs a row's
    exact running max rises by more than 8 (exp2 domain) within one 64-key step for over 1% of
    (row, step) pairs (pinned on the CPU in test_oracle_model.py)."""
    D = 64 if kind == "bf16-d64" else 128
    shape = synth.shrink(synth.CONFIGS["layer"], name=f"rising-{kind}", heads=2, head_dim=D,
                         tokens_per_frame=100, window_frames=5)
    log(f"case: rising scores {kind}")
    run_stream(shape, 8, kv_format="fp4" if kind == "fp4" else "dense", k_frame_gain=2.0)


def test_denoise_steps_only_last_commits():
    shape = synth.shrink(synth.CONFIGS["layer"], name="steps", heads=2, tokens_per_frame=40,
                         window_frames=4)
    log("case: 4 denoise steps per chunk")
    run_stream(shape, 6, steps=4)


def test_fp32_head_dim_128_and_sink_variants():
    shape = synth.shrink(synth.CONFIGS["tiny"], name="f32-d128", head_dim=128, sink_frames=2,
                         window_frames=4, tokens_per_frame=20)
    log("case: fp32 D=128, S=2, W=4")
    run_stream(shape, 7)


@pytest.mark.parametrize("case", [
    # name, base, overrides, kv_format, chunks
    ("no-sink", "layer", dict(heads=2, tokens_per_frame=20, sink_frames=0, window_frames=3), "dense", 6),
    ("window-equals-chunk", "layer", dict(heads=1, tokens_per_frame=40, window_frames=3), "dense", 6),
    ("one-frame-chunks-d64", "layer", dict(heads=2, head_dim=64, tokens_per_frame=30, chunk_frames=1,
                                           sink_frames=1, window_frames=2), "dense", 8),
    ("one-token-frames", "layer", dict(heads=2, tokens_per_frame=1, window_frames=6), "dense", 10),
    ("fp4-no-sink", "layer", dict(heads=2, tokens_per_frame=24, chunk_frames=2, sink_frames=0,
                                  window_frames=4), "fp4", 7),
    ("fp32-window-one", "tiny", dict(chunk_frames=1, sink_frames=0, window_frames=1), "dense", 5),
], ids=lambda c: c[0])
def test_degenerate_geometries(case):
    """No sink, a window of exactly one chunk, one-frame chunks, one token per frame (3 query
    rows, a few keys: every tile mostly masked), FP4 without a sink, an fp32 window of one
    frame: every chunk compared, cache export bit-exact."""
    name, base, over, kv_format, chunks = case
    shape = synth.shrink(synth.CONFIGS[base], name=name, **over)
    log(f"case: degenerate geometry {name} ({kv_format})")
    run_stream(shape, chunks, kv_format=kv_format)


def test_layer_config_sampled():
    """The 1.3B-DiT-shaped layer: 12 heads x 128, 1560 tokens/frame, chunk 3, sink 3, window 9,
    20 chunks; sampled query rows on fill-up, first wrap and the last chunk."""
    shape = synth.CONFIGS["layer"]
    log("case: layer config, 20 chunks, sampled rows")
    rows = sample_rows(shape.n_query, 48, seed=1)
    run_stream(shape, 20, compare={0, 1, 3, 4, 5, 19}, rows=rows, export_every=False)


@pytest.mark.parametrize("kv_format", ["dense", "fp4"])
def test_three_head_share_sampled(kv_format):
    """The layer shape at 3 heads (one GPU's share of 12 heads over 4 sequence-parallel
    ranks): 57 query blocks on a 256-CU device, so chunk attention runs split into equal key
    ranges with up to 6 pieces per block that are merged on the device; dense and FP4 stores."""
    shape = synth.shrink(synth.CONFIGS["layer"], name="share-h3", heads=3)
    log(f"case: layer config at 3 heads, {kv_format}, 8 chunks, sampled rows")
    rows = sample_rows(shape.n_query, 64, seed=3)
    run_stream(shape, 8, kv_format=kv_format, compare={0, 2, 4, 5, 7}, rows=rows,
               export_every=False)


def test_split_with_many_pieces():
    """One head of 1200 query rows over a 12-frame window of 400-token frames: five query
    blocks on a many-CU device, so once the window is full every block's key tiles are
    spread over dozens of workgroups and merged on the device (ragged tails: 4800 + 1200
    keys are not multiples of the 128-key tile)."""
    shape = synth.shrink(synth.CONFIGS["layer"], name="split-h1", heads=1, tokens_per_frame=400)
    log("case: 1 head, 400-token frames, 8 chunks, all rows")
    run_stream(shape, 8)


def test_side_stream():
    """Every call enqueues on the caller's stream: a stream run entirely on a side stream
    (split schedule at 1 head, FP4 store, commits, the first call's counter clearing) while
    the default stream is kept busy, read back only after that stream is synchronised."""
    import torch
    shape = synth.shrink(synth.CONFIGS["layer"], name="side-stream", heads=1,
                         tokens_per_frame=400, window_frames=6)
    log("case: side stream, split schedule, FP4")
    side = torch.cuda.Stream()
    busy = torch.empty((4096, 4096), device="cuda")
    with torch.cuda.stream(side):
        cache = _cache(shape, "fp4")
    model = _model(shape, "fp4")
    for c in range(8):
        q, k, v = synth.chunk_inputs(shape, 0, 0, c)
        with torch.cuda.stream(side):
            tq, tk, tv = q.torch("cuda"), k.torch("cuda"), v.torch("cuda")
        busy.normal_()                                   # default-stream work in between
        busy = busy @ busy
        with torch.cuda.stream(side):
            o = cache.attn_chunk(0, tq, tk, tv)
            cache.commit(0, tk, tv)
            o_host = o.to("cpu", non_blocking=False)
        side.synchronize()
        ref = model.attn_chunk(q.values, k.values, v.values)
        assert_close(o_host.to(torch.float64).numpy(), ref, "bf16", f"side stream chunk {c}")
        model.commit(k.values, v.values, k.bits, v.bits)
    torch.cuda.synchronize()


def test_value_one_gives_one_and_determinism():
    import torch
    shape = synth.shrink(synth.CONFIGS["layer"], heads=2, tokens_per_frame=90, window_frames=4)
    cache = _cache(shape)
    for c in range(5):
        q, k, v = (t.torch("cuda") for t in synth.chunk_inputs(shape, 0, 0, c))
        ones = torch.ones_like(v)
        o1 = cache.attn_chunk(0, q, k, ones)
        o2 = cache.attn_chunk(0, q, k, ones)
        torch.cuda.synchronize()
        if c > 0:   # history V is also 1
            assert float((o1.float() - 1).abs().max()) <= 2 ** -7
        assert torch.equal(o1, o2)
        a = cache.attn_chunk(0, q, k, v)
        b = cache.attn_chunk(0, q, k, v)
        assert torch.equal(a, b), "attention is not deterministic"
        cache.commit(0, k, ones)


def test_cache_holds_copies_and_evicted_frames_do_not_leak():
    """Poison the caller's buffers after commit and the evicted slots' old frames: the next
    chunks' outputs still match the oracle. V carries a per-frame offset (0.05 per frame) so a
    stale or misrouted frame shows up as a large error; the offset keeps |o| below 2, where
    bf16 output rounding (half an ulp) stays under the 1e-2 max-abs bound."""
    import torch
    shape = synth.shrink(synth.CONFIGS["layer"], heads=2, tokens_per_frame=64, window_frames=3)
    cache = _cache(shape)
    model = _model(shape)
    for c in range(8):
        q, k, v = synth.chunk_inputs(shape, 0, 0, c, v_frame_offset=0.05)
        tq, tk, tv = q.torch("cuda"), k.torch("cuda"), v.torch("cuda")
        o = cache.attn_chunk(0, tq, tk, tv)
        assert_close(to_np(o), model.attn_chunk(q.values, k.values, v.values), "bf16", f"chunk {c}")
        cache.commit(0, tk, tv)
        model.commit(k.values, v.values)
        tk.fill_(float("nan"))
        tv.fill_(float("nan"))
        torch.cuda.synchronize()


def test_kv_quant_exhaustive_bit_exact():
    """Every finite bf16 pattern in blocks whose max drives each scale byte 0..252."""
    import torch
    from windowed_attention_kv_amd import kv_quant
    p = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = p[((p >> 7) & 0xFF) != 0xFF]
    mags = pats & 0x7FFF
    blocks = []
    for field in range(0, 255, 1):
        driver = np.uint16((field << 7) | 0x7F) if field > 0 else np.uint16(0x7F)
        fit = pats[mags <= driver]
        n_blk = -(-fit.size // 15)
        body = np.zeros(n_blk * 15, np.uint16)
        body[:fit.size] = fit
        blocks.append(np.concatenate([np.full((n_blk, 1), driver, np.uint16),
                                      body.reshape(n_blk, 15)], axis=1))
    x = np.concatenate(blocks)                    # [blocks, 16]
    log(f"case: kv_quant on {x.size} elements")
    t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    pk, sc = kv_quant(t)
    wp, ws = ofp4.quantize(x)
    np.testing.assert_array_equal(sc.cpu().numpy(), ws)
    np.testing.assert_array_equal(pk.cpu().numpy(), wp)


def test_kv_quant_random_and_ragged_rows():
    import torch
    from windowed_attention_kv_amd import kv_quant
    for rows, L in ((1, 16), (7, 48), (1000, 128), (12 * 1560, 128)):
        x = synth.bf16_matrix(rows, L, seed=rows + L)
        t = torch.from_numpy(x.bits.view(np.int16)).view(torch.bfloat16).cuda()
        pk, sc = kv_quant(t)
        wp, ws = ofp4.quantize(x.bits)
        np.testing.assert_array_equal(pk.cpu().numpy(), wp)
        np.testing.assert_array_equal(sc.cpu().numpy(), ws)
        # caller-supplied outputs are written in place
        pk2 = torch.empty_like(pk)
        sc2 = torch.empty_like(sc)
        kv_quant(t, pk2, sc2)
        assert torch.equal(pk2, pk) and torch.equal(sc2, sc)


def test_kv_quant_rejects_wrong_outputs():
    """Output buffers that the kernel would overrun are refused before any launch."""
    import pytest
    import torch
    from windowed_attention_kv_amd import kv_quant
    t = torch.zeros((8, 32), dtype=torch.bfloat16, device="cuda")
    good_p = torch.empty((8, 16), dtype=torch.uint8, device="cuda")
    good_s = torch.empty((8, 2), dtype=torch.uint8, device="cuda")
    for p, s in ((good_p[:7], good_s), (good_p, good_s[:, :1]),
                 (good_p.to(torch.int8), good_s), (good_p, good_s.cpu())):
        with pytest.raises(ValueError):
            kv_quant(t, p, s)
    assert all(int(b) == 0 for b in kv_quant(t, good_p, good_s)[0].flatten()[:4])
    # an output that starts off the 8-byte grid the kernel stores on is refused by the library
    from windowed_attention_kv_amd import LLError
    flat = torch.empty(8 * 16 + 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(LLError):
        kv_quant(t, flat[4:].view(8, 16), good_s)


def test_fp4_stream():
    shape = synth.shrink(synth.CONFIGS["layer"], name="fp4-small", heads=2, tokens_per_frame=100,
                         window_frames=5)
    log("case: FP4 KV stream, small")
    run_stream(shape, 8, kv_format="fp4")


def test_fp4_layer_config_sampled():
    shape = synth.CONFIGS["layer"]
    log("case: FP4 KV at the layer config, sampled rows")
    rows = sample_rows(shape.n_query, 32, seed=2)
    run_stream(shape, 7, kv_format="fp4", compare={0, 4, 6}, rows=rows, export_every=False)


def _recache_case(shape, n_chunks, n_text, kv_format="dense", rows=None, after=2):
    cache, model = run_stream(shape, n_chunks, kv_format=kv_format, compare=set(),
                              export_every=False)
    n = len(model.held()) * shape.tokens_per_frame
    ins = synth.recache_inputs(shape, 0, n, n_text)
    q, k, v, qx, kt, vt = ins
    o, ox = cache.recache(0, *(t.torch("cuda") for t in ins))
    ref_o, ref_ox = model.recache(q.values, k.values, v.values, qx.values, kt.values, vt.values,
                                  k.bits, v.bits, rows=rows)
    r = rows if rows is not None else np.arange(n)
    assert_close(to_np(o)[r], ref_o, shape.dtype, "recache self")
    assert_close(to_np(ox)[r], ref_ox, shape.dtype, "recache cross")
    _check_export(cache, model, shape)
    # later chunks see the recached values
    rc = r[r < shape.n_query]
    for c in range(n_chunks, n_chunks + after):
        qq, kk, vv = synth.chunk_inputs(shape, 0, 0, c, salt=7)
        tk, tv = kk.torch("cuda"), vv.torch("cuda")
        oo = cache.attn_chunk(0, qq.torch("cuda"), tk, tv)
        assert_close(to_np(oo)[rc], model.attn_chunk(qq.values, kk.values, vv.values, rows=rc),
                     shape.dtype, f"after recache chunk {c}")
        cache.commit(0, tk, tv)
        model.commit(kk.values, vv.values, kk.bits, vv.bits)


@pytest.mark.parametrize("n_chunks", [1, 3, 10])
def test_recache_small(n_chunks):
    shape = synth.shrink(synth.CONFIGS["layer"], name="recache-small", heads=2,
                         tokens_per_frame=100)
    log(f"case: recache after {n_chunks} chunks")
    _recache_case(shape, n_chunks, n_text=77)


def test_recache_fp32_and_fp4():
    log("case: recache fp32 tiny")
    _recache_case(synth.CONFIGS["tiny"], 9, n_text=20)
    shape = synth.shrink(synth.CONFIGS["layer"], name="recache-fp4", heads=2, tokens_per_frame=64)
    log("case: recache fp4")
    _recache_case(shape, 5, n_text=64, kv_format="fp4")


def test_recache_config_sampled():
    """Recache at the prompt-switch shape: 12 held frames (18720 rows), 512 text tokens."""
    shape = synth.CONFIGS["recache"]
    log("case: recache config, sampled rows")
    rows = sample_rows(12 * shape.tokens_per_frame, 40, seed=3)
    _recache_case(shape, 10, n_text=512, rows=rows, after=1)


def test_interactive_composite_small():
    """The interactive pattern at a small shape: 2 layers x 2 denoise steps x 12 chunks with a
    prompt switch (recache of both layers with new text K/V) before chunks 3, 6 and 9. Every
    chunk output, every recache output and the final caches are checked against one oracle
    model per layer."""
    shape = synth.shrink(synth.CONFIGS["layer"], name="composite", heads=2, tokens_per_frame=64)
    log("case: interactive composite, 2 layers, 12 chunks, switches at 3/6/9")
    L, steps, switches, n_text = 2, 2, (3, 6, 9), 40
    cache = _cache(shape, layers=L)
    models = [_model(shape) for _ in range(L)]
    for c in range(12):
        if c in switches:
            for layer in range(L):
                n = len(models[layer].held()) * shape.tokens_per_frame
                ins = synth.recache_inputs(shape, layer, n, n_text, salt=c)
                q, k, v, qx, kt, vt = ins
                o, ox = cache.recache(layer, *(t.torch("cuda") for t in ins))
                ref_o, ref_ox = models[layer].recache(q.values, k.values, v.values, qx.values,
                                                      kt.values, vt.values, k.bits, v.bits)
                assert_close(to_np(o), ref_o, "bf16", f"switch {c} layer {layer} self")
                assert_close(to_np(ox), ref_ox, "bf16", f"switch {c} layer {layer} cross")
        for step in range(steps):
            for layer in range(L):
                q, k, v = synth.chunk_inputs(shape, layer, step, c)
                tk, tv = k.torch("cuda"), v.torch("cuda")
                o = cache.attn_chunk(layer, q.torch("cuda"), tk, tv)
                assert_close(to_np(o), models[layer].attn_chunk(q.values, k.values, v.values),
                             "bf16", f"chunk {c} step {step} layer {layer}")
                if step == steps - 1:
                    cache.commit(layer, tk, tv)
                    models[layer].commit(k.values, v.values, k.bits, v.bits)
    for layer in range(L):
        _check_export(cache, models[layer], shape, layer)


def _cross_stream(shape, n_chunks, n_text, kv_format="dense", compare=None, rows=None):
    """Stream chunks through ll_attn_chunk_cross: o against the chunk oracle, ox against the
    oracle's plain attention of qx over the text keys, and o bit-identical to ll_attn_chunk's
    (the self part of the fused launch runs the same schedule)."""
    import torch
    cache = _cache(shape, kv_format)
    model = _model(shape, kv_format)
    for c in range(n_chunks):
        q, k, v = synth.chunk_inputs(shape, 0, 0, c)
        xs = synth.recache_inputs(shape, 0, shape.n_query, n_text, salt=100 + c)
        qx, kt, vt = xs[3], xs[4], xs[5]
        tq, tk, tv = q.torch("cuda"), k.torch("cuda"), v.torch("cuda")
        o, ox = cache.attn_chunk_cross(0, tq, tk, tv, qx.torch("cuda"), kt.torch("cuda"),
                                       vt.torch("cuda"))
        o_plain = cache.attn_chunk(0, tq, tk, tv)
        torch.cuda.synchronize()
        assert torch.equal(o, o_plain), f"chunk {c}: fused self part differs from ll_attn_chunk"
        if compare is None or c in compare:
            r = rows if rows is not None else np.arange(shape.n_query)
            assert_close(to_np(o)[r], model.attn_chunk(q.values, k.values, v.values, rows=r),
                         shape.dtype, f"chunk {c} self")
            ref_x = oatt.attention_rows(qx.values, kt.values, vt.values, model.scale, rows=r)
            assert_close(to_np(ox)[r], ref_x, shape.dtype, f"chunk {c} cross")
        cache.commit(0, tk, tv)
        model.commit(k.values, v.values, k.bits, v.bits)


@pytest.mark.parametrize("heads,T,n_text", [(3, 100, 77), (1, 400, 512), (2, 64, 1)])
def test_attn_chunk_cross_fused(heads, T, n_text):
    """bf16 head_dim 128: self and text cross-attention in one launch; (1 head, 400-token
    frames) also runs the split schedule with the cross blocks after it."""
    shape = synth.shrink(synth.CONFIGS["layer"], name=f"cross-h{heads}", heads=heads,
                         tokens_per_frame=T)
    log(f"case: fused cross-attention, {heads} heads, T={T}, {n_text} text keys")
    _cross_stream(shape, 6, n_text)


def test_attn_chunk_cross_other_shapes():
    """head_dim 64 (bf16), fp32 and an FP4 cache: the same results when the self and cross
    parts run as two launches (only a dense bf16 head_dim-128 cache fuses them)."""
    log("case: cross-attention, head_dim 64")
    _cross_stream(synth.shrink(synth.CONFIGS["layer"], name="cross-d64", heads=2, head_dim=64,
                               tokens_per_frame=72), 5, 50)
    log("case: cross-attention, fp32")
    _cross_stream(synth.shrink(synth.CONFIGS["tiny"], name="cross-f32"), 6, 20)
    log("case: cross-attention, FP4 cache")
    _cross_stream(synth.shrink(synth.CONFIGS["layer"], name="cross-fp4", heads=2,
                               tokens_per_frame=64), 6, 64, kv_format="fp4")


def test_attn_chunk_cross_layer_config_sampled():
    """The layer shape with 512 text tokens: 228 self blocks leave 28 of 256 CUs for the
    cross blocks; sampled rows on fill-up and steady chunks."""
    shape = synth.CONFIGS["layer"]
    log("case: fused cross-attention, layer config, sampled rows")
    _cross_stream(shape, 6, 512, compare={0, 5}, rows=sample_rows(shape.n_query, 48, seed=5))


@pytest.mark.parametrize("kind", ["bf16-d128", "bf16-d64", "fp32", "fp4"])
def test_multi_shot_stream(kind):
    """Multi-shot sink: new shots before chunks 3, 4 and 9 of a 14-chunk stream. Every chunk
    matches the oracle and every export is bit-exact, so each sink frame's move from its
    window slot to its sink slot (and the old sink's retirement) is checked."""
    base = synth.CONFIGS["tiny"] if kind == "fp32" else synth.shrink(
        synth.CONFIGS["layer"], heads=2, tokens_per_frame=48,
        head_dim=64 if kind == "bf16-d64" else 128)
    shape = synth.shrink(base, name=f"shots-{kind}")
    log(f"case: multi-shot stream, {kind}")
    run_stream(shape, 14, kv_format="fp4" if kind == "fp4" else "dense", shots=(3, 4, 9))


def test_recache_after_a_new_shot():
    """A prompt switch after a shot boundary: recache over the new shot's sink frames and the
    window (block-causal by chunk), then more chunks of the shot."""
    shape = synth.shrink(synth.CONFIGS["layer"], name="shot-recache", heads=2, tokens_per_frame=64)
    log("case: recache after a new shot")
    cache, model = run_stream(shape, 12, compare=set(), export_every=False, shots=(5,))
    n = len(model.held()) * shape.tokens_per_frame
    assert model.held() == [15, 16, 17] + list(range(27, 36))
    ins = synth.recache_inputs(shape, 0, n, 33)
    q, k, v, qx, kt, vt = ins
    o, ox = cache.recache(0, *(t.torch("cuda") for t in ins))
    ref_o, ref_ox = model.recache(q.values, k.values, v.values, qx.values, kt.values, vt.values,
                                  k.bits, v.bits)
    assert_close(to_np(o), ref_o, "bf16", "recache self after a new shot")
    assert_close(to_np(ox), ref_ox, "bf16", "recache cross after a new shot")
    _check_export(cache, model, shape)
    for c in range(12, 15):
        qq, kk, vv = synth.chunk_inputs(shape, 0, 0, c, salt=9)
        tk, tv = kk.torch("cuda"), vv.torch("cuda")
        oo = cache.attn_chunk(0, qq.torch("cuda"), tk, tv)
        assert_close(to_np(oo), model.attn_chunk(qq.values, kk.values, vv.values), "bf16",
                     f"after recache chunk {c}")
        cache.commit(0, tk, tv)
        model.commit(kk.values, vv.values, kk.bits, vv.bits)
        _check_export(cache, model, shape)


@pytest.mark.parametrize("kv_format", ["dense", "fp4"])
def test_cache_at_the_size_limit(kv_format):
    """The largest cache the library accepts at 2 heads x 128 in bf16: (S+W)*T*H*D*2 =
    2,146,959,360 bytes per K/V plane, just under the 2^31 bound of the kernels' 32-bit byte
    offsets (S=1, W=1023, T=4095, C=1; 4.19M keys per head). All T tokens of a frame carry
    the same K and V rows, and every visible frame has T tokens, so attention over the cache
    equals attention over one key per visible frame: the oracle computes every output row from
    the frame vectors. Checked with the cache partly filled, and after the window has wrapped
    and the sink frame has moved to its sink slot."""
    import torch
    from windowed_attention_kv_amd import Cache
    H, D, T, C, S, W = 2, 128, 4095, 1, 1, 1023
    assert (S + W) * T * H * D * 2 < 2 ** 31 <= (S + W) * (T + 1) * H * D * 2
    n_frames = W + S + 5
    kf = synth.draw((n_frames, H, D), "bf16", 1.0, synth.rng(60, 0, 0, 0, 1))
    vf = synth.draw((n_frames, H, D), "bf16", 0.5, synth.rng(60, 0, 0, 0, 2))
    tkf, tvf = kf.torch("cuda"), vf.torch("cuda")

    def frame(t, f):
        return t[f].expand(T, H, D).contiguous()

    def held(x, f):
        """What the cache holds for committed frame f (one token row, float64)."""
        return ofp4.roundtrip(x.bits[f]) if kv_format == "fp4" else x.values[f].astype(np.float64)

    cache = Cache(1, H, D, T, C, S, W, kv_format=kv_format)
    for c in range(n_frames):
        if c in (600, n_frames - 1):
            log(f"case: cache at the size limit, {kv_format}, chunk {c}")
            q = synth.draw((T, H, D), "bf16", 1.0, synth.rng(60, 0, 0, c, 0))
            o = cache.attn_chunk(0, q.torch("cuda"), frame(tkf, c), frame(tvf, c))
            vis = ring.visible_frames(c, C, S, W)
            K = np.stack([held(kf, f) if f < c else kf.values[f] for f in vis])
            V = np.stack([held(vf, f) if f < c else vf.values[f] for f in vis])
            ref = oatt.attention(q.values, K, V, 1.0 / math.sqrt(D))
            ma, rl = assert_close(to_np(o), ref, "bf16", f"size limit {kv_format} chunk {c}")
            log(f"size limit {kv_format} chunk {c}: max-abs {ma:.3e} rel-L2 {rl:.3e}")
        cache.commit(0, frame(tkf, c), frame(tvf, c))
    F, slots = cache.state(0)
    assert F == n_frames and slots == ring.slot_map(F, S, W)
    del cache
    torch.cuda.empty_cache()
