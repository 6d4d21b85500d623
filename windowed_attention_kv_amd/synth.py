"""Seeded synthetic inputs shared by the tests, the bench and the oracle side.

This module holds no part of the attention, cache or codec arithmetic: it only draws
random tensors from fixed seeds and rounds them to the storage type (bf16 by integer
round-to-nearest-even on the fp32 bit pattern), so that the HIP path and the oracle are
fed bit-identical values.

Shapes follow the five workloads of the window+sink chunk-attention hot path:

  tiny    1 layer, 2 heads x 64, 16 tokens/frame, chunk 3 frames, sink 3, window 6, 8 chunks, fp32
  layer   1 layer, 12 heads x 128, 1560 tokens/frame, chunk 3, sink 3, window 9, 20 chunks, bf16
  stack   the layer shape x 30 layers x 4 denoise steps x 80 chunks
  recache 30 layers, prefill over sink(3)+window(9) frames (18720 rows) + 512 text tokens
  fp4     the stack with an e2m1/e8m0 KV store

The pages these follow measure on VBench / VBench-Long prompt suites and a private
interactive set; nothing from those suites is used here: the tensors below stand in for
the activations such prompts would produce, with the shapes of a 1.3B-parameter DiT.
"""
from __future__ import annotations

import dataclasses

import numpy as np

# tensor ids inside a seed tuple
Q, K, V, QX, K_TEXT, V_TEXT = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    cfg_id: int
    layers: int
    heads: int
    head_dim: int
    tokens_per_frame: int
    chunk_frames: int
    sink_frames: int
    window_frames: int
    chunks: int
    dtype: str          # "f32" or "bf16"
    value_scale: float  # std of the drawn values
    steps: int = 1      # denoise steps per chunk (only the last commits)
    n_text: int = 0     # text tokens for the recache cross-attention
    kv_format: str = "dense"

    @property
    def n_query(self) -> int:
        return self.tokens_per_frame * self.chunk_frames

    @property
    def slots(self) -> int:
        return self.sink_frames + self.window_frames


CONFIGS = {
    "tiny": Shape("tiny", 0, 1, 2, 64, 16, 3, 3, 6, 8, "f32", 1.0),
    "layer": Shape("layer", 1, 1, 12, 128, 1560, 3, 3, 9, 20, "bf16", 0.5),
    "stack": Shape("stack", 2, 30, 12, 128, 1560, 3, 3, 9, 80, "bf16", 0.5, steps=4),
    "recache": Shape("recache", 3, 30, 12, 128, 1560, 3, 3, 9, 4, "bf16", 0.5, n_text=512),
    "fp4": Shape("fp4", 4, 30, 12, 128, 1560, 3, 3, 9, 80, "bf16", 0.5, steps=4, kv_format="fp4"),
}


def shrink(shape: Shape, **kw) -> Shape:
    """A copy of `shape` with some fields replaced (used for smaller parity cases)."""
    return dataclasses.replace(shape, **kw)


def rng(cfg_id: int, layer: int, step: int, chunk: int, tensor_id: int, salt: int = 0):
    ss = np.random.SeedSequence([cfg_id, layer, step, chunk, tensor_id, salt])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns, nearest-even on the dropped 16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """One synthetic tensor: `values` are float32 holding exactly the stored values;
    `bits` is the uint16 bf16 pattern (None for fp32 tensors)."""
    values: np.ndarray
    bits: np.ndarray | None

    def torch(self, device="cpu"):
        import torch
        if self.bits is None:
            return torch.from_numpy(np.ascontiguousarray(self.values)).to(device)
        t = torch.from_numpy(np.ascontiguousarray(self.bits).view(np.int16))
        return t.view(torch.bfloat16).to(device)


def draw(shape_rows: tuple, dtype: str, std: float, gen: np.random.Generator,
         offset: np.ndarray | float = 0.0, gain: np.ndarray | float = 1.0) -> Tensor:
    x = gen.standard_normal(shape_rows, dtype=np.float32) * np.float32(std)
    x = (x * np.asarray(gain, dtype=np.float32) + np.asarray(offset, dtype=np.float32)).astype(np.float32)
    if dtype == "f32":
        return Tensor(x, None)
    bits = f32_to_bf16_bits(x)
    return Tensor(bf16_bits_to_f32(bits), bits)


def chunk_inputs(shape: Shape, layer: int, step: int, chunk: int, *, peaked: bool = False,
                 v_frame_offset: float = 0.0, k_frame_gain: float = 0.0, salt: int = 0):
    """Q, K, V of one chunk, each [C*T, H, D].

    peaked: Q and K drawn with twice the std (sharper softmax).
    v_frame_offset: V of frame f gets + f * v_frame_offset, so a wrong or stale frame shows
    up as a large error.
    k_frame_gain: K of frame f is scaled by 1 + f * k_frame_gain, so later frames give ever
    larger scores (the largest score of a row keeps moving as its keys are swept).
    """
    rows = (shape.n_query, shape.heads, shape.head_dim)
    std = shape.value_scale * (2.0 if peaked else 1.0)
    frame = chunk * shape.chunk_frames + np.arange(shape.n_query) // shape.tokens_per_frame
    out = []
    for tid in (Q, K, V):
        g = rng(shape.cfg_id, layer, step, chunk, tid, salt)
        off, gain = 0.0, 1.0
        if tid == V and v_frame_offset:
            off = (frame * v_frame_offset).astype(np.float32)[:, None, None]
        if tid == K and k_frame_gain:
            gain = (1.0 + frame * k_frame_gain).astype(np.float32)[:, None, None]
        out.append(draw(rows, shape.dtype, std if tid != V else shape.value_scale, g, off, gain))
    return tuple(out)


def recache_inputs(shape: Shape, layer: int, n_rows: int, n_text: int, *, salt: int = 0):
    """Q, K, V, Qx ([n_rows, H, D]) and K_text, V_text ([n_text, H, D]) of one recache."""
    big = (n_rows, shape.heads, shape.head_dim)
    txt = (n_text, shape.heads, shape.head_dim)
    res = []
    for tid, rows in ((Q, big), (K, big), (V, big), (QX, big), (K_TEXT, txt), (V_TEXT, txt)):
        g = rng(shape.cfg_id, layer, 1000, 0, tid, salt)
        res.append(draw(rows, shape.dtype, shape.value_scale, g))
    return tuple(res)


def bf16_matrix(rows: int, cols: int, seed: int, std: float = 0.5) -> Tensor:
    """A generic bf16 matrix (codec tests)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([99, seed])))
    return draw((rows, cols), "bf16", std, g)
