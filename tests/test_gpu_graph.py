"""Chunk attention captured in a HIP graph: one denoise step at the layer shape (three layers'
chunk attention, split schedule on) recorded once, through ll_attn_chunk and through
ll_attn_chunk_noalloc, and replayed several times with eager work and synchronisations between
the replays; every replay's outputs are bit-identical to the eager calls'. The first call on a
handle (and on a device, for the static workspace) clears the split counters with a kernel and
sets the kernels' LDS attribute, so it runs before the capture; the captured launches record no
memset, and every launch leaves the counters at zero for the next replay."""
import ctypes

import pytest

from _parity import log
from windowed_attention_kv_amd import _lib, synth

pytestmark = pytest.mark.gpu


def _noalloc(cache, layer, q, k, v, o):
    import torch
    lib = _lib.lib()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    _lib.check(lib, lib.ll_attn_chunk_noalloc(cache.handle, layer, ptr(q), ptr(k), ptr(v), ptr(o),
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))


@pytest.mark.parametrize("entry", ["ll_attn_chunk", "ll_attn_chunk_noalloc"])
def test_denoise_step_replayed_from_a_graph(entry):
    import torch
    from windowed_attention_kv_amd import Cache
    shape = synth.CONFIGS["layer"]
    L = 3
    H, D, T, C, S, W = (shape.heads, shape.head_dim, shape.tokens_per_frame, shape.chunk_frames,
                        shape.sink_frames, shape.window_frames)
    log(f"case: graph replay of {L} layers' chunk attention via {entry}")
    cache = Cache(L, H, D, T, C, S, W)
    for c in range(5):                       # fill the window: the next chunk is a steady one
        for layer in range(L):
            _, k, v = synth.chunk_inputs(shape, layer, 0, c, salt=51)
            cache.commit(layer, k.torch("cuda"), v.torch("cuda"))
    ins = [tuple(t.torch("cuda") for t in synth.chunk_inputs(shape, layer, 0, 5, salt=51))
           for layer in range(L)]
    outs = [torch.empty_like(q) for q, _, _ in ins]

    def step():
        for layer, ((q, k, v), o) in enumerate(zip(ins, outs)):
            if entry == "ll_attn_chunk":
                cache.attn_chunk(layer, q, k, v, out=o)
            else:
                _noalloc(cache, layer, q, k, v, o)

    step()                                   # eager: first calls, reference outputs
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.zero_()                        # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for layer, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}, layer {layer} differs from the eager call"
        step()                               # an eager step between replays as well
        torch.cuda.synchronize()
        for layer, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"eager step after replay {rep}, layer {layer}"
    del graph
