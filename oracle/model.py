"""One layer's window+sink KV cache over a stream of chunks, as the method defines it.

[LL] 方法 §3 高效长推理 (short-window attention; frame sink), [LL] 方法 §1 KV 重缓存 (recache at
a prompt switch), [INFRA] §5 (quantisation errors enter the stored history), [DIST]
"NVFP4 量化与 KV Cache 压缩的工程实现" (FP4 KV store).

The model keeps every frame ever committed (it never evicts) and lets the visible-frame set
of `ring.visible_frames` decide what a chunk sees; the slot map of `ring.slot_map` is used
only to lay out `export()`. A cross-check asserts that every committed frame a chunk sees
is one the layer still holds, tying the visible set to the eviction rule.

Readings taken:
  * multi-shot sink ([DIST] 序列并行与注意力汇聚的协同设计): new_shot() marks the next committed
    frame as the first of a new shot; its first S frames become the sink and the previous
    shot's sink frames stop being visible unless they are still in the window;
  * the own chunk is attended bidirectionally and unquantised; only committed history is
    stored in FP4 (quantisation happens on commit);
  * only the last denoise step of a chunk commits (earlier steps leave no trace);
  * recache rows are the held frames in ascending frame id; a query in frame fq sees key
    frame fk iff chunk(fk) <= chunk(fq); its cross-attention uses separate queries qx and
    all n_text text keys, unmasked; after the recache the held frames keep their ids and
    slots and take the recache K/V as values.
"""
from __future__ import annotations

import math

import numpy as np

from . import attention as att
from . import fp4
from . import ring


class LayerModel:
    def __init__(self, S: int, W: int, C: int, T: int, H: int, D: int,
                 scale: float | None = None, kv_format: str = "dense"):
        self.S, self.W, self.C, self.T, self.H, self.D = S, W, C, T, H, D
        self.scale = 1.0 / math.sqrt(D) if scale is None else scale
        self.kv_format = kv_format
        self.F = 0
        self.B = 0           # first frame of the current shot
        self.k = {}          # frame -> stored K values [T,H,D] float64
        self.v = {}
        self.k_fp4 = {}      # frame -> (packed [T*H, D/2], scales [T*H, D/16]) under FP4
        self.v_fp4 = {}

    # -- storage ---------------------------------------------------------------------
    def _store(self, f: int, kv, bits, dst: dict, dst_fp4: dict):
        if self.kv_format == "fp4":
            if bits is None:
                raise ValueError("the FP4 store needs the bf16 bit patterns")
            rows = np.asarray(bits).reshape(self.T * self.H, self.D)
            packed, scales = fp4.quantize(rows)
            dst_fp4[f] = (packed, scales)
            dst[f] = fp4.dequantize(packed, scales).reshape(self.T, self.H, self.D)
        else:
            dst[f] = np.asarray(kv, dtype=np.float64).copy()

    @property
    def chunk(self) -> int:
        return self.F // self.C

    def held(self) -> list[int]:
        return ring.held_frames(self.F, self.S, self.W, self.B)

    def new_shot(self):
        """The next committed frame starts a new shot (multi-shot sink)."""
        self.B = self.F

    # -- chunk attention -----------------------------------------------------------------
    def keys_for_chunk(self, k_own, v_own):
        """Concatenated keys/values the current chunk attends to, with their frame ids."""
        s = self.F
        held = set(self.held())
        ks, vs, fr = [], [], []
        for f in ring.visible_frames(self.chunk, self.C, self.S, self.W, self.B):
            if f < s:
                assert f in held, f"chunk {self.chunk} sees frame {f} that was evicted"
                ks.append(self.k[f])
                vs.append(self.v[f])
            else:
                i = f - s
                ks.append(np.asarray(k_own, dtype=np.float64)[i * self.T:(i + 1) * self.T])
                vs.append(np.asarray(v_own, dtype=np.float64)[i * self.T:(i + 1) * self.T])
            fr.append(f)
        return np.concatenate(ks), np.concatenate(vs), fr

    def attn_chunk(self, q, k, v, rows=None) -> np.ndarray:
        """O for the chunk's queries (all, or the subset `rows`)."""
        K, V, _ = self.keys_for_chunk(k, v)
        return att.attention_rows(q, K, V, self.scale, rows=rows)

    # -- commit --------------------------------------------------------------------------
    def commit(self, k, v, k_bits=None, v_bits=None):
        """Store the chunk's K/V as frames F..F+C-1 (the final denoise step's values)."""
        for i in range(self.C):
            f = self.F + i
            sl = slice(i * self.T, (i + 1) * self.T)
            self._store(f, None if k is None else np.asarray(k)[sl],
                        None if k_bits is None else np.asarray(k_bits)[sl], self.k, self.k_fp4)
            self._store(f, None if v is None else np.asarray(v)[sl],
                        None if v_bits is None else np.asarray(v_bits)[sl], self.v, self.v_fp4)
        self.F += self.C

    # -- recache -------------------------------------------------------------------------
    def recache_mask(self, frames: list[int]):
        """mask_fn for the block-causal prefill over `frames` (ascending)."""
        row_chunk = np.repeat(np.array([ring.chunk_of_frame(f, self.C) for f in frames]), self.T)

        def mask_fn(r):
            return row_chunk[None, :] <= row_chunk[np.asarray(r)][:, None]
        return mask_fn

    def recache(self, q, k, v, qx, k_text, v_text, k_bits=None, v_bits=None,
                rows=None, update=True):
        """(o_self, o_cross) over the held frames; then the held frames take k, v."""
        frames = self.held()
        if not frames:
            raise ValueError("recache of an empty layer")
        n = len(frames) * self.T
        if np.asarray(q).shape[0] != n:
            raise ValueError(f"recache expects {n} rows")
        o_self = att.attention_rows(q, k, v, self.scale, rows=rows,
                                    mask_fn=self.recache_mask(frames))
        o_cross = att.attention_rows(qx, k_text, v_text, self.scale, rows=rows)
        if update:
            for i, f in enumerate(frames):
                sl = slice(i * self.T, (i + 1) * self.T)
                self._store(f, np.asarray(k)[sl],
                            None if k_bits is None else np.asarray(k_bits)[sl], self.k, self.k_fp4)
                self._store(f, np.asarray(v)[sl],
                            None if v_bits is None else np.asarray(v_bits)[sl], self.v, self.v_fp4)
        return o_self, o_cross

    # -- inspection ------------------------------------------------------------------------
    def slot_map(self) -> list[int]:
        return ring.slot_map(self.F, self.S, self.W, self.B)

    def export_dense(self):
        """Slot-order K, V [(S+W)*T, H, D]; empty slots are NaN."""
        shape = ((self.S + self.W) * self.T, self.H, self.D)
        K = np.full(shape, np.nan)
        Vv = np.full(shape, np.nan)
        for slot, f in enumerate(self.slot_map()):
            if f >= 0:
                K[slot * self.T:(slot + 1) * self.T] = self.k[f]
                Vv[slot * self.T:(slot + 1) * self.T] = self.v[f]
        return K, Vv

    def export_fp4(self):
        """Slot-order packed [(S+W)*T*H, D/2] and scales [(S+W)*T*H, D/16] for K and V,
        and a bool [(S+W)*T*H] mask of the filled rows."""
        NS, T, H, D = self.S + self.W, self.T, self.H, self.D
        kp = np.zeros((NS * T * H, D // 2), np.uint8)
        ks = np.zeros((NS * T * H, D // 16), np.uint8)
        vp, vs = kp.copy(), ks.copy()
        valid = np.zeros(NS * T * H, bool)
        for slot, f in enumerate(self.slot_map()):
            if f >= 0:
                sl = slice(slot * T * H, (slot + 1) * T * H)
                kp[sl], ks[sl] = self.k_fp4[f]
                vp[sl], vs[sl] = self.v_fp4[f]
                valid[sl] = True
        return kp, ks, vp, vs, valid


def bruteforce_chunk(q, hist_k, hist_v, chunk: int, C: int, S: int, W: int, T: int,
                     scale: float, rows=None, shot_start: int = 0) -> np.ndarray:
    """Chunk attention over the WHOLE history (every frame ever produced, own chunk
    included, frame-major [n_frames*T, H, D]) with an explicit frame mask: key frame fk is
    visible to the chunk iff it is a sink frame of the chunk's shot (the shot's first S
    frames), one of the W frames before the chunk, or in the chunk. Nothing is evicted;
    masked keys contribute exactly zero."""
    s = chunk * C
    n_frames = np.asarray(hist_k).shape[0] // T
    fk = np.arange(n_frames)
    B = shot_start
    vis = ((fk >= B) & (fk < B + S)) | ((fk >= s - W) & (fk < s)) | ((fk >= s) & (fk < s + C))
    vis &= fk < s + C
    key_vis = np.repeat(vis, T)

    def mask_fn(r):
        return np.broadcast_to(key_vis[None, :], (len(r), key_vis.size))
    return att.attention_rows(q, hist_k, hist_v, scale, rows=rows, mask_fn=mask_fn)
