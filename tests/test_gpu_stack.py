"""GPU parity of the multi-layer workloads: the 30-layer stack at its full length (bf16
and FP4 stores), the prompt-switch recache of every layer of a 30-layer cache, and the batched commit
(ll_cache_commit_layers) against per-layer commits and the oracle."""
import numpy as np
import pytest

from _parity import assert_close, log, sample_rows, to_np
from oracle import fp4 as ofp4
from oracle import ring
from oracle.model import LayerModel
from windowed_attention_kv_amd import synth

pytestmark = pytest.mark.gpu


class _StreamModel(LayerModel):
    """LayerModel for the full-length stack. Frames of the resident input sets are converted
    (under FP4: encoded and decoded) once and shared by every layer and chunk that commits
    them; a committed frame is dropped as soon as the layer no longer holds it, so 80 chunks
    stay within a few hundred MB. keys_for_chunk still asserts that every committed frame a
    chunk sees is held, so a dropped frame that a chunk needed fails loudly. The memo keeps a
    reference to each source frame, so no key can be reused by another buffer."""
    memo = {}

    def _store(self, f, kv, bits, dst, dst_fp4):
        src = bits if self.kv_format == "fp4" else kv
        key = (self.kv_format, src.__array_interface__["data"][0], src.shape)
        if key not in self.memo:
            if self.kv_format == "fp4":
                rows = np.asarray(bits).reshape(self.T * self.H, self.D)
                packed, scales = ofp4.quantize(rows)
                values = ofp4.dequantize(packed, scales).reshape(self.T, self.H, self.D)
                self.memo[key] = (src, (packed, scales), values)
            else:
                self.memo[key] = (src, None, np.asarray(kv, dtype=np.float64))
        _, planes, values = self.memo[key]
        if planes is not None:
            dst_fp4[f] = planes
        dst[f] = values

    def commit(self, k, v, k_bits=None, v_bits=None):
        super().commit(k, v, k_bits, v_bits)
        held = set(self.held())
        for d in (self.k, self.v, self.k_fp4, self.v_fp4):
            for f in [f for f in d if f not in held]:
                del d[f]


def _cache(shape, layers, kv_format="dense"):
    from windowed_attention_kv_amd import Cache
    return Cache(layers, shape.heads, shape.head_dim, shape.tokens_per_frame, shape.chunk_frames,
                 shape.sink_frames, shape.window_frames, dtype=shape.dtype, kv_format=kv_format)


def _model(shape, kv_format="dense", cls=LayerModel):
    return cls(shape.sink_frames, shape.window_frames, shape.chunk_frames,
               shape.tokens_per_frame, shape.heads, shape.head_dim, kv_format=kv_format)


@pytest.mark.parametrize("kv_format", ["dense", "fp4"])
def test_stack_config_sampled(kv_format):
    """The stack workload at its full length, as the bench runs it: one 30-layer cache (bf16
    or FP4 store); per chunk 4 denoise steps over all layers, then one batched commit of the
    last step's K/V into all 30 layers; 80 chunks (fill-up, the window's wrap, the sink
    retiring into its slots, and 76 chunks of steady state). Layers 0, 15 and 29 are checked
    against per-layer oracles on sampled rows at steps 0 and 3 of chunks 0, 1, 4, 5, 15, 39, 40
    and 79: at step 0 they take fresh seeded inputs, every other call takes one of five
    resident input sets, chosen so that consecutive chunks of a layer commit different sets.
    At the end every layer's exported slots equal, bit for bit, the K/V committed into each
    slot (under FP4: the oracle's encoding of it)."""
    import torch
    shape = synth.CONFIGS["layer"]
    L, steps, n_chunks = 30, 4, 80
    C, S, W, T = shape.chunk_frames, shape.sink_frames, shape.window_frames, shape.tokens_per_frame
    n, H, D = shape.n_query, shape.heads, shape.head_dim
    fp4 = kv_format == "fp4"
    sampled_layers, sampled_chunks = (0, 15, 29), {0, 1, 4, 5, 15, 39, 40, 79}
    rows = sample_rows(n, 16, seed=11 if fp4 else 9)
    log(f"case: {kv_format} stack, 30 layers x 4 steps x 80 chunks, sampled layers/chunks/rows")
    pool_host = [synth.chunk_inputs(shape, 100 + i, 0, 0) for i in range(5)]
    pool = [tuple(t.torch("cuda") for t in trip) for trip in pool_host]

    def pick(c, st, layer):
        return (c + 2 * st + layer) % len(pool)

    cache = _cache(shape, L, kv_format)
    models = {l: _model(shape, kv_format, _StreamModel) for l in sampled_layers}
    committed = {}          # (layer, chunk) -> input set committed
    for c in range(n_chunks):
        for st in range(steps):
            for layer in range(L):
                check = layer in models and c in sampled_chunks and st in (0, steps - 1)
                fresh = check and st == 0
                host = synth.chunk_inputs(shape, layer, st, c) if fresh else pool_host[pick(c, st, layer)]
                dev = tuple(t.torch("cuda") for t in host) if fresh else pool[pick(c, st, layer)]
                o = cache.attn_chunk(layer, *dev)
                if check:
                    q, k, v = host
                    ref = models[layer].attn_chunk(q.values, k.values, v.values, rows=rows)
                    assert_close(to_np(o[torch.as_tensor(rows, device="cuda")]), ref, "bf16",
                                 f"{kv_format} layer {layer} chunk {c} step {st}")
        last = [pick(c, steps - 1, layer) for layer in range(L)]
        cache.commit_layers(0, [pool[i][1] for i in last], [pool[i][2] for i in last])
        for layer in range(L):
            committed[(layer, c)] = last[layer]
        for layer, m in models.items():
            _, k, v = pool_host[last[layer]]
            m.commit(k.values, v.values, k.bits, v.bits)
    torch.cuda.synchronize()
    F = n_chunks * C
    slot_frames = ring.slot_map(F, S, W)
    want = {}               # (input set, frame of the chunk, K|V) -> expected slot contents

    def expected(idx, i, which):
        if (idx, i, which) not in want:
            src = pool_host[idx][1 + which]
            if fp4:
                want[(idx, i, which)] = ofp4.quantize(src.bits[i * T:(i + 1) * T].reshape(T * H, D))
            else:
                want[(idx, i, which)] = pool[idx][1 + which][i * T:(i + 1) * T]
        return want[(idx, i, which)]

    for layer in range(L):
        planes = cache.export(layer)
        Fs, slots = cache.state(layer)
        assert Fs == F and slots == slot_frames
        if fp4:
            kp, ks, vp, vs = (x.cpu().numpy() for x in planes)
        for slot, f in enumerate(slot_frames):
            idx, i = committed[(layer, f // C)], f % C
            if fp4:
                sl = slice(slot * T * H, (slot + 1) * T * H)
                for got_p, got_s, which, name in ((kp, ks, 0, "K"), (vp, vs, 1, "V")):
                    wp, ws = expected(idx, i, which)
                    assert np.array_equal(got_p[sl], wp), (layer, slot, f, name, "codes")
                    assert np.array_equal(got_s[sl], ws), (layer, slot, f, name, "scales")
            else:
                for got, which, name in ((planes[0], 0, "K"), (planes[1], 1, "V")):
                    assert torch.equal(got[slot * T:(slot + 1) * T], expected(idx, i, which)), \
                        (layer, slot, f, name)
        if fp4 and layer in models:
            mkp, mks, mvp, mvs, valid = models[layer].export_fp4()
            for got, ref in ((kp, mkp), (ks, mks), (vp, mvp), (vs, mvs)):
                assert np.array_equal(got[valid], ref[valid]), layer


def test_recache_30_layers_sampled():
    """The prompt-switch recache on every layer of a filled 30-layer cache (12 held frames =
    18720 rows, 512 text tokens): layers 0, 15 and 29 take seeded inputs and are compared on
    sampled rows (self and cross) against per-layer oracles, the others take resident random
    inputs; afterwards every layer's export equals its recache K/V slot by slot, and one more
    chunk on the sampled layers attends to the recached values."""
    import torch
    shape = synth.CONFIGS["recache"]
    L, n_text = 30, 512
    C, S, W, T = shape.chunk_frames, shape.sink_frames, shape.window_frames, shape.tokens_per_frame
    n, H, D = shape.n_query, shape.heads, shape.head_dim
    sampled = (0, 15, 29)
    log("case: recache of 30 layers, 18720 rows + 512 text keys, sampled layers/rows")
    cache = _cache(shape, L)
    g = torch.Generator(device="cuda")
    g.manual_seed(23)
    fill = [(torch.randn((n, H, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
            for _ in range(2)]
    models = {l: _model(shape) for l in sampled}
    zeros = np.zeros((n, H, D), np.float32)
    for c in range(10):
        cache.commit_layers(0, [fill[0]] * L, [fill[1]] * L)
        for m in models.values():
            m.commit(zeros, zeros)
    held = models[0].held()
    assert held == [0, 1, 2] + list(range(21, 30))
    rows_all = len(held) * T
    rows = sample_rows(rows_all, 40, seed=13)
    big = [(torch.randn((rows_all, H, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
           for _ in range(4)]
    txt = [(torch.randn((n_text, H, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
           for _ in range(2)]
    new_kv = {}
    for layer in range(L):
        if layer in models:
            ins = synth.recache_inputs(shape, layer, rows_all, n_text)
            dev = [t.torch("cuda") for t in ins]
            o, ox = cache.recache(layer, *dev)
            q, k, v, qx, kt, vt = ins
            ref_o, ref_ox = models[layer].recache(q.values, k.values, v.values, qx.values,
                                                  kt.values, vt.values, rows=rows)
            assert_close(to_np(o)[rows], ref_o, "bf16", f"layer {layer} recache self")
            assert_close(to_np(ox)[rows], ref_ox, "bf16", f"layer {layer} recache cross")
            new_kv[layer] = (dev[1], dev[2])
        else:
            cache.recache(layer, big[0], big[1], big[2], big[3], txt[0], txt[1])
            new_kv[layer] = (big[1], big[2])
    torch.cuda.synchronize()
    slot_frames = ring.slot_map(10 * C, S, W)
    rank = {f: r for r, f in enumerate(held)}
    for layer in range(L):
        K, V = cache.export(layer)
        nk, nv = new_kv[layer]
        for slot, f in enumerate(slot_frames):
            r = rank[f]
            assert torch.equal(K[slot * T:(slot + 1) * T], nk[r * T:(r + 1) * T]), (layer, slot, f)
            assert torch.equal(V[slot * T:(slot + 1) * T], nv[r * T:(r + 1) * T]), (layer, slot, f)
    crow = sample_rows(n, 24, seed=14)
    for layer, m in models.items():
        q, k, v = synth.chunk_inputs(shape, layer, 0, 10, salt=5)
        o = cache.attn_chunk(layer, q.torch("cuda"), k.torch("cuda"), v.torch("cuda"))
        assert_close(to_np(o)[crow], m.attn_chunk(q.values, k.values, v.values, rows=crow), "bf16",
                     f"layer {layer} chunk after the recache")


@pytest.mark.parametrize("kv_format", ["dense", "fp4"])
def test_commit_layers_equals_per_layer_commits(kv_format):
    """ll_cache_commit_layers against ll_cache_commit at the layer shape: 6 layers, one of them
    a chunk ahead and two with a new shot partway (so the batch mixes frame counts and moves
    sink frames out of the window in some layers only), 6 chunks; after every batch the
    exported planes of every layer are bit-identical between the two caches."""
    import torch
    shape = synth.CONFIGS["layer"]
    L = 6
    n, H, D = shape.n_query, shape.heads, shape.head_dim
    log(f"case: batched commit vs per-layer commits, {kv_format}, 6 layers")
    a, b = _cache(shape, L, kv_format), _cache(shape, L, kv_format)
    g = torch.Generator(device="cuda")
    g.manual_seed(31)
    mk = lambda: (torch.randn((n, H, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    k0, v0 = mk(), mk()
    a.commit(0, k0, v0)
    b.commit(0, k0, v0)
    for c in range(6):
        if c == 2:
            for layer in (1, 4):
                a.new_shot(layer)
                b.new_shot(layer)
        ks = [mk() for _ in range(L)]
        vs = [mk() for _ in range(L)]
        a.commit_layers(0, ks, vs)
        for layer in range(L):
            b.commit(layer, ks[layer], vs[layer])
        torch.cuda.synchronize()
        for layer in range(L):
            F, slots = a.state(layer)
            assert (F, slots) == b.state(layer)
            # rows of empty slots hold whatever the memory held: compare the held slots
            T = shape.tokens_per_frame
            per_slot = T if kv_format == "dense" else T * H
            for x, y in zip(a.export(layer), b.export(layer)):
                for slot, f in enumerate(slots):
                    if f >= 0:
                        sl = slice(slot * per_slot, (slot + 1) * per_slot)
                        assert torch.equal(x[sl], y[sl]), (c, layer, slot, f)


_BATCHED_CASES = {
    # name: (base config, overrides, kv_format)
    "bf16-d128-dense": ("layer", dict(tokens_per_frame=200), "dense"),
    "bf16-d128-fp4": ("layer", dict(tokens_per_frame=200), "fp4"),
    "bf16-d64-dense": ("layer", dict(tokens_per_frame=96, heads=6, head_dim=64), "dense"),
    "bf16-d64-fp4": ("layer", dict(tokens_per_frame=96, heads=6, head_dim=64), "fp4"),
    "f32-d64": ("tiny", dict(), "dense"),
}


@pytest.mark.parametrize("case", list(_BATCHED_CASES))
def test_commit_layers_against_the_oracle(case):
    """Batched commits into 4 layers checked against the oracle's export after every batch,
    through the window's wrap, the sink retiring into its slots and a new shot in one layer;
    bf16 and FP4 stores at head_dim 128 and 64 (16-byte units of 16 and 8 per head row; one or
    two 64-element FP4 groups) and an fp32 cache (the tiny shape). Afterwards one more chunk of
    attention per layer reads the batched-committed cache."""
    import torch
    base, over, kv_format = _BATCHED_CASES[case]
    shape = synth.shrink(synth.CONFIGS[base], name=f"batched-{case}", **over)
    L = 4
    log(f"case: batched commit vs oracle, {case}")
    cache = _cache(shape, L, kv_format)
    models = [_model(shape, kv_format) for _ in range(L)]
    for c in range(7):
        if c == 3:
            cache.new_shot(2)
            models[2].new_shot()
        ins = [synth.chunk_inputs(shape, layer, 0, c, salt=3) for layer in range(L)]
        cache.commit_layers(0, [x[1].torch("cuda") for x in ins], [x[2].torch("cuda") for x in ins])
        for layer in range(L):
            _, k, v = ins[layer]
            models[layer].commit(k.values, v.values, k.bits, v.bits)
        torch.cuda.synchronize()
        for layer in range(L):
            m = models[layer]
            F, slots = cache.state(layer)
            assert F == m.F and slots == m.slot_map()
            if kv_format == "fp4":
                got = [x.cpu().numpy() for x in cache.export(layer)]
                want = m.export_fp4()
                valid = want[4]
                for gg, ww in zip(got, want[:4]):
                    assert np.array_equal(gg[valid], ww[valid]), (c, layer)
            else:
                K, V = (to_np(x) for x in cache.export(layer))
                MK, MV = m.export_dense()
                valid = ~np.isnan(MK[:, 0, 0])
                assert np.array_equal(K[valid], MK[valid]) and np.array_equal(V[valid], MV[valid])
    for layer in range(L):
        q, k, v = synth.chunk_inputs(shape, layer, 0, 7, salt=4)
        o = cache.attn_chunk(layer, q.torch("cuda"), k.torch("cuda"), v.torch("cuda"))
        assert_close(to_np(o), models[layer].attn_chunk(q.values, k.values, v.values), shape.dtype,
                     f"{case} layer {layer} chunk after the batched commits")
