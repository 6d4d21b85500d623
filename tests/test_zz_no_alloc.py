"""ll_attn_chunk_noalloc: chunk attention whose split-schedule workspace is the library's static
device array (for callers that cannot allocate).

Host part (recording backend, no GPU): the call passes the static array's address and its
counter and slot capacity to the attention launch, allocates nothing else, and refuses, before
enqueueing anything, a cache whose split schedule needs more slots than the array holds.
GPU part: through the C ABI, its output is bit-identical to ll_attn_chunk's, and within the
bf16 tolerance of the fp64 oracle, on two calls in a row on one device, the second with a
smaller input; calls between them leave the shared counters at zero.
"""
import ctypes
import os

import numpy as np
import pytest

from _parity import assert_close, log, to_np
from oracle.model import LayerModel
from windowed_attention_kv_amd import _lib, make_desc, synth


@pytest.fixture
def fake():
    if not os.path.exists(_lib.FAKE_PATH):
        pytest.skip("libll_fake.so not built")
    f = _lib.load_fake()
    f.llfake_reset()
    f.llfake_set_cus(256)
    yield f
    f.llfake_set_cus(256)


def _fake_cache(f, heads):
    d = make_desc(1, heads, 128, 1560, 3, 3, 9)
    size = ctypes.c_size_t()
    assert f.ll_cache_size(ctypes.byref(d), ctypes.byref(size)) == 0
    h = ctypes.c_void_p()
    assert f.ll_cache_create(ctypes.byref(d), ctypes.c_void_p(1 << 20), size.value, ctypes.byref(h)) == 0
    return h


def test_noalloc_passes_the_static_workspace(fake):
    P = ctypes.c_void_p(1 << 24)
    h = _fake_cache(fake, 12)
    assert fake.ll_attn_chunk_noalloc(h, 0, P, P, P, P, None) == 0
    buf = (ctypes.c_int64 * 24)()
    kinds = [fake.llfake_record(i, buf) for i in range(fake.llfake_count())]
    assert kinds == [0]                      # one attention launch, no workspace clearing
    fake.llfake_record(0, buf)
    assert buf[16] == 1 and buf[17] == 65536 and buf[18] == 512 and buf[19] == 256
    fake.ll_cache_destroy(h)
    # a device with more compute units needs more piece slots than the array holds
    fake.llfake_set_cus(300)
    h = _fake_cache(fake, 12)
    fake.llfake_reset()
    assert fake.ll_attn_chunk_noalloc(h, 0, P, P, P, P, None) == _lib.LL_EINVAL
    assert b"static workspace" in fake.ll_last_error()
    assert fake.llfake_count() == 0
    # the cache's own workspace still serves ll_attn_chunk on such a device
    assert fake.ll_attn_chunk(h, 0, P, P, P, P, None) == 0
    fake.ll_cache_destroy(h)


def _noalloc(cache, layer, q, k, v, o):
    import torch
    lib = _lib.lib()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    _lib.check(lib, lib.ll_attn_chunk_noalloc(cache.handle, layer, ptr(q), ptr(k), ptr(v), ptr(o),
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    return o


@pytest.mark.gpu
def test_noalloc_matches_attn_chunk_on_two_calls():
    import torch
    from windowed_attention_kv_amd import Cache
    cases = [synth.CONFIGS["layer"],
             synth.shrink(synth.CONFIGS["layer"], name="noalloc-small", heads=3, tokens_per_frame=400)]
    for shape in cases:
        H, D, T, C, S, W = (shape.heads, shape.head_dim, shape.tokens_per_frame, shape.chunk_frames,
                            shape.sink_frames, shape.window_frames)
        log(f"case: ll_attn_chunk_noalloc vs ll_attn_chunk, {H} heads, T={T}")
        cache = Cache(1, H, D, T, C, S, W)
        model = LayerModel(S, W, C, T, H, D)
        for c in range(5):       # fill the window: the next chunk is a steady one
            q, k, v = synth.chunk_inputs(shape, 0, 0, c, salt=41)
            tk, tv = k.torch("cuda"), v.torch("cuda")
            cache.commit(0, tk, tv)
            model.commit(k.values, v.values)
        q, k, v = synth.chunk_inputs(shape, 0, 0, 5, salt=41)
        tq, tk, tv = q.torch("cuda"), k.torch("cuda"), v.torch("cuda")
        o_ref = cache.attn_chunk(0, tq, tk, tv)
        o = _noalloc(cache, 0, tq, tk, tv, torch.empty_like(tq))
        o2 = _noalloc(cache, 0, tq, tk, tv, torch.empty_like(tq))
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "noalloc output differs from ll_attn_chunk"
        assert torch.equal(o2, o_ref), "second noalloc call differs (counters not left at zero)"
        rows = np.unique(np.linspace(0, shape.n_query - 1, 40).astype(int))
        assert_close(to_np(o)[rows], model.attn_chunk(q.values, k.values, v.values, rows=rows),
                     "bf16", f"noalloc {H} heads vs oracle")
        del cache
