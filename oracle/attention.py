"""Explicit masked softmax attention in float64.

For one head h, query i and keys j:
    z_ij = scale * sum_d q[i,h,d] * k[j,h,d]           (logits)
    p_ij = exp(z_ij - m_i) / sum_j exp(z_ij - m_i),  m_i = max_j z_ij
    o[i,h,:] = sum_j p_ij * v[j,h,:]
Masked keys get z = -inf and so p = 0 exactly.

Used for the chunk attention of [LL] 方法 §3 (window + sink keys), for the block-causal
recache prefill of [LL] 方法 §1 KV 重缓存, and for its cross-attention to the prompt
(text) keys and values of the DiT cross-attention layers described there.

Query rows are independent under the definition, so the functions accept a subset of rows
(`rows`) to keep large sampled checks affordable; the arithmetic per row is the same.
"""
from __future__ import annotations

import numpy as np


def logits(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """q [Nq,H,D], k [Nk,H,D] -> z [H,Nq,Nk] in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    # per head: z_h = Q_h K_h^T (library matmul as the contraction step)
    qh = np.transpose(q, (1, 0, 2))          # [H,Nq,D]
    kh = np.transpose(k, (1, 2, 0))          # [H,D,Nk]
    return scale * np.matmul(qh, kh)


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row softmax over the last axis; rows that are all -inf are not allowed."""
    m = np.max(z, axis=-1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row sees no key")
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q, k, v, scale: float, mask: np.ndarray | None = None,
              return_probs: bool = False):
    """o [Nq,H,D] = softmax(scale q k^T, masked) v.

    mask: bool [Nq,Nk] (True = key visible to that query), shared by all heads.
    """
    z = logits(q, k, scale)
    if mask is not None:
        z = np.where(np.asarray(mask, dtype=bool)[None, :, :], z, -np.inf)
    p = softmax_rows(z)                      # [H,Nq,Nk]
    vh = np.transpose(np.asarray(v, dtype=np.float64), (1, 0, 2))   # [H,Nk,D]
    o = np.transpose(np.matmul(p, vh), (1, 0, 2))                 # [Nq,H,D]
    return (o, p) if return_probs else o


def attention_rows(q, k, v, scale: float, rows=None, mask_fn=None, block: int = 256):
    """attention() for the query rows `rows` (default: all), `block` rows at a time.

    mask_fn(rows_array) -> bool [len(rows), Nk] gives the visibility of those rows.
    Returns [len(rows), H, D].
    """
    q = np.asarray(q)
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows)
    out = np.empty((len(rows), q.shape[1], q.shape[2]), dtype=np.float64)
    for s in range(0, len(rows), block):
        r = rows[s:s + block]
        m = None if mask_fn is None else mask_fn(r)
        out[s:s + block] = attention(q[r], k, v, scale, m)
    return out
