"""Window+sink chunk attention over a rolling per-layer KV cache, for MI355X (gfx950).

Thin Python binding over the C ABI of include/ll.h (libll.so). Every step of the path runs
in the library's HIP kernels; this module only checks and marshals torch tensors (device
memory and streams). There is no fallback: if the library is missing, calls raise.

    cache = Cache(layers=1, heads=12, head_dim=128, tokens_per_frame=1560, chunk_frames=3,
                  sink_frames=3, window_frames=9)            # bf16, dense KV
    o = cache.attn_chunk(0, q, k, v)                          # [C*T, H, D] each
    cache.commit(0, k, v)
    o, ox = cache.recache(0, q, k, v, qx, k_text, v_text)
    packed, scales = kv_quant(x)                              # FP4 e2m1 + e8m0/16
"""
from __future__ import annotations

import ctypes

from ._lib import (LL_ABI_VERSION, LL_BF16, LL_F32, LL_KV_DENSE, LL_KV_FP4, CacheDesc, LLError,
                   check, lib)

__all__ = ["Cache", "kv_quant", "LLError", "make_desc"]


def _torch():
    import torch
    return torch


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_desc(layers, heads, head_dim, tokens_per_frame, chunk_frames, sink_frames,
              window_frames, dtype="bf16", kv_format="dense", scale=None) -> CacheDesc:
    d = CacheDesc()
    d.abi_version = LL_ABI_VERSION
    d.num_layers = layers
    d.num_heads = heads
    d.head_dim = head_dim
    d.tokens_per_frame = tokens_per_frame
    d.chunk_frames = chunk_frames
    d.sink_frames = sink_frames
    d.window_frames = window_frames
    d.dtype = {"f32": LL_F32, "bf16": LL_BF16}[dtype]
    d.kv_format = {"dense": LL_KV_DENSE, "fp4": LL_KV_FP4}[kv_format]
    d.softmax_scale = 0.0 if scale is None else float(scale)
    return d


class Cache:
    """Host handle plus the torch-owned device memory of a window+sink KV cache."""

    def __init__(self, layers, heads, head_dim, tokens_per_frame, chunk_frames, sink_frames,
                 window_frames, dtype="bf16", kv_format="dense", scale=None, device="cuda"):
        torch = _torch()
        self.desc = make_desc(layers, heads, head_dim, tokens_per_frame, chunk_frames,
                              sink_frames, window_frames, dtype, kv_format, scale)
        self.H, self.D, self.T, self.C = heads, head_dim, tokens_per_frame, chunk_frames
        self.S, self.W, self.layers = sink_frames, window_frames, layers
        self.dtype = dtype
        self.kv_format = kv_format
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self._lib = lib()
        size = ctypes.c_size_t()
        check(self._lib, self._lib.ll_cache_size(ctypes.byref(self.desc), ctypes.byref(size)))
        self.nbytes = size.value
        self.mem = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        check(self._lib, self._lib.ll_cache_create(ctypes.byref(self.desc),
                                                   ctypes.c_void_p(self.mem.data_ptr()),
                                                   self.nbytes, ctypes.byref(h)))
        self.handle = h

    # -- helpers -----------------------------------------------------------------------
    def _check(self, t, rows, name):
        if t.device != self.device or t.dtype != self.tdtype or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous {self.tdtype} tensor on {self.device}")
        if tuple(t.shape) != (rows, self.H, self.D):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {(rows, self.H, self.D)}")
        return ctypes.c_void_p(t.data_ptr())

    @property
    def n_chunk(self) -> int:
        return self.C * self.T

    def _empty(self, rows):
        return _torch().empty((rows, self.H, self.D), dtype=self.tdtype, device=self.device)

    # -- the hot path ----------------------------------------------------------------------
    def attn_chunk(self, layer, q, k, v, out=None):
        n = self.n_chunk
        o = self._empty(n) if out is None else out
        check(self._lib, self._lib.ll_attn_chunk(self.handle, layer, self._check(q, n, "q"),
                                                 self._check(k, n, "k"), self._check(v, n, "v"),
                                                 self._check(o, n, "o"), _stream(self.device)))
        return o

    def attn_chunk_cross(self, layer, q, k, v, qx, k_text, v_text, out=None, out_x=None):
        """attn_chunk plus the text cross-attention ox = softmax(scale qx K_text^T) V_text in
        one call (one launch for bf16 head_dim 128). Returns (o, ox)."""
        n = self.n_chunk
        nt = k_text.shape[0]
        o = self._empty(n) if out is None else out
        ox = self._empty(n) if out_x is None else out_x
        check(self._lib, self._lib.ll_attn_chunk_cross(
            self.handle, layer, self._check(q, n, "q"), self._check(k, n, "k"),
            self._check(v, n, "v"), self._check(qx, n, "qx"), self._check(k_text, nt, "k_text"),
            self._check(v_text, nt, "v_text"), nt, self._check(o, n, "o"), self._check(ox, n, "ox"),
            _stream(self.device)))
        return o, ox

    def commit(self, layer, k, v):
        n = self.n_chunk
        check(self._lib, self._lib.ll_cache_commit(self.handle, layer, self._check(k, n, "k"),
                                                   self._check(v, n, "v"), _stream(self.device)))

    def commit_layers(self, first_layer, ks, vs):
        """Commit one chunk's K/V into layers first_layer .. first_layer + len(ks) - 1 with
        one launch (ks[i], vs[i] go to layer first_layer + i)."""
        n = self.n_chunk
        if len(ks) != len(vs) or not ks:
            raise ValueError("commit_layers: ks and vs must be non-empty and of equal length")
        kp = (ctypes.c_void_p * len(ks))(*[self._check(t, n, "k").value for t in ks])
        vp = (ctypes.c_void_p * len(vs))(*[self._check(t, n, "v").value for t in vs])
        check(self._lib, self._lib.ll_cache_commit_layers(self.handle, first_layer, len(ks), kp, vp,
                                                          _stream(self.device)))

    def new_shot(self, layer=None):
        """Shot boundary (multi-shot sink): the next committed frame of `layer` (default:
        every layer) starts a new shot whose first S frames become the sink."""
        layers = range(self.layers) if layer is None else [layer]
        for l in layers:
            check(self._lib, self._lib.ll_cache_new_shot(self.handle, l))

    def held_rows(self, layer) -> int:
        F, slots = self.state(layer)
        return sum(1 for f in slots if f >= 0) * self.T

    def recache(self, layer, q, k, v, qx, k_text, v_text, out=None, out_x=None):
        n = self.held_rows(layer)
        nt = k_text.shape[0]
        o = self._empty(n) if out is None else out
        ox = self._empty(n) if out_x is None else out_x
        check(self._lib, self._lib.ll_recache(
            self.handle, layer, self._check(q, n, "q"), self._check(k, n, "k"),
            self._check(v, n, "v"), self._check(qx, n, "qx"), self._check(k_text, nt, "k_text"),
            self._check(v_text, nt, "v_text"), nt, self._check(o, n, "o"),
            self._check(ox, n, "ox"), _stream(self.device)))
        return o, ox

    # -- inspection ---------------------------------------------------------------------------
    def state(self, layer):
        F = ctypes.c_int64()
        slots = (ctypes.c_int32 * (self.S + self.W))()
        check(self._lib, self._lib.ll_cache_state(self.handle, layer, ctypes.byref(F), slots))
        return F.value, list(slots)

    def export(self, layer):
        """dense: (K, V) [(S+W)*T, H, D]; fp4: (K packed, K scales, V packed, V scales) with
        [(S+W)*T*H, D/2] and [(S+W)*T*H, D/16] uint8 planes. Slot order."""
        torch = _torch()
        rows = (self.S + self.W) * self.T
        s = _stream(self.device)
        if self.kv_format == "fp4":
            kp = torch.empty((rows * self.H, self.D // 2), dtype=torch.uint8, device=self.device)
            vp = torch.empty_like(kp)
            ks = torch.empty((rows * self.H, self.D // 16), dtype=torch.uint8, device=self.device)
            vs = torch.empty_like(ks)
            check(self._lib, self._lib.ll_cache_export(
                self.handle, layer, ctypes.c_void_p(kp.data_ptr()), ctypes.c_void_p(vp.data_ptr()),
                ctypes.c_void_p(ks.data_ptr()), ctypes.c_void_p(vs.data_ptr()), s))
            return kp, ks, vp, vs
        K = self._empty(rows)
        V = self._empty(rows)
        check(self._lib, self._lib.ll_cache_export(self.handle, layer, ctypes.c_void_p(K.data_ptr()),
                                                   ctypes.c_void_p(V.data_ptr()), None, None, s))
        return K, V

    def reset(self):
        check(self._lib, self._lib.ll_cache_reset(self.handle))

    def close(self):
        if getattr(self, "handle", None):
            self._lib.ll_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kv_quant(x, packed=None, scales=None):
    """FP4 e2m1 codes (2 per byte) and e8m0 scales (one per 16 along the last dim) of a
    contiguous bf16 CUDA tensor whose last dimension is a multiple of 16."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("kv_quant expects a contiguous bf16 CUDA tensor")
    L = x.shape[-1] if x.dim() else 0
    rows = x.numel() // L if L else 0
    if packed is None:
        packed = torch.empty((rows, L // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, L // 16), dtype=torch.uint8, device=x.device)
    # caller-supplied outputs are written in full by the kernel: check them before the launch
    for name, t, width in (("packed", packed, L // 2), ("scales", scales, L // 16)):
        if t.dtype != torch.uint8 or t.device != x.device or not t.is_contiguous() \
                or t.numel() != rows * width:
            raise ValueError(f"kv_quant: {name} must be a contiguous uint8 tensor on {x.device} "
                             f"with {rows * width} elements")
    l = lib()
    check(l, l.ll_kv_quant(ctypes.c_void_p(x.data_ptr()), rows, L,
                           ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                           _stream(x.device)))
    return packed, scales


def flops_per_pair(head_dim: int) -> int:
    """Algorithmic flops of one visible (query, key) pair of one head: 2D for q.k and 2D for
    the p*v accumulation."""
    return 4 * head_dim


def attn_flops(n_query: int, n_keys: int, heads: int, head_dim: int) -> float:
    return float(n_query) * n_keys * heads * flops_per_pair(head_dim)
