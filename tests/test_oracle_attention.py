"""Pins for oracle/attention.py: library routine (torch CPU fp64 scaled_dot_product_attention,
run, not re-implemented), closed forms and the softmax normalisation invariant."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as att


def _rand(shape, seed, std=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * std


def sdpa(q, k, v, scale, mask=None):
    """torch CPU fp64 SDPA on [N,H,D] arrays; mask bool [Nq,Nk] True = visible."""
    tq = torch.from_numpy(np.transpose(q, (1, 0, 2)).copy())[None]
    tk = torch.from_numpy(np.transpose(k, (1, 0, 2)).copy())[None]
    tv = torch.from_numpy(np.transpose(v, (1, 0, 2)).copy())[None]
    am = None if mask is None else torch.from_numpy(np.asarray(mask, bool))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale)
    return np.transpose(o[0].numpy(), (1, 0, 2))


@pytest.mark.parametrize("nq,nk,H,D", [(48, 48, 2, 64), (37, 200, 3, 128), (5, 1, 1, 16)])
def test_unmasked_vs_sdpa(nq, nk, H, D):
    q, k, v = _rand((nq, H, D), 1), _rand((nk, H, D), 2), _rand((nk, H, D), 3)
    scale = 1 / math.sqrt(D)
    o = att.attention(q, k, v, scale)
    ref = sdpa(q, k, v, scale)
    assert np.max(np.abs(o - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_block_causal_mask_vs_sdpa():
    T, C, G, H, D = 8, 3, 4, 2, 32
    n = T * C * G
    q, k, v = _rand((n, H, D), 4), _rand((n, H, D), 5), _rand((n, H, D), 6)
    grp = np.arange(n) // (T * C)
    mask = grp[None, :] <= grp[:, None]
    o = att.attention(q, k, v, 0.3, mask)
    ref = sdpa(q, k, v, 0.3, mask)
    assert np.max(np.abs(o - ref)) <= 1e-12


def test_rows_subset_equals_full():
    q, k, v = _rand((70, 2, 16), 7), _rand((90, 2, 16), 8), _rand((90, 2, 16), 9)
    full = att.attention(q, k, v, 0.25)
    rows = np.array([0, 3, 69, 17])
    sub = att.attention_rows(q, k, v, 0.25, rows=rows, block=3)
    # BLAS may group the sums differently for fewer rows: equal up to rounding
    assert np.max(np.abs(sub - full[rows])) <= 1e-14


def test_probabilities_sum_to_one():
    q, k, v = _rand((40, 3, 64), 10, 3.0), _rand((300, 3, 64), 11, 3.0), _rand((300, 3, 64), 12)
    mask = _rand((40, 300), 13) > 0.7
    mask[:, 0] = True
    _, p = att.attention(q, k, v, 0.125, mask, return_probs=True)
    assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-14
    assert np.all(p[:, ~mask] == 0.0)


def test_closed_forms():
    H, D = 2, 8
    v = _rand((5, H, D), 14)
    # identical keys: uniform weights -> mean of V
    q = _rand((3, H, D), 15)
    k = np.repeat(_rand((1, H, D), 16), 5, axis=0)
    np.testing.assert_allclose(att.attention(q, k, v, 0.7), np.broadcast_to(v.mean(0), (3, H, D)),
                               rtol=0, atol=1e-14)
    # V == 1 -> O == 1
    np.testing.assert_allclose(att.attention(q, _rand((5, H, D), 17), np.ones((5, H, D)), 0.7),
                               1.0, rtol=0, atol=1e-14)
    # a single visible key returns its value row
    mask = np.zeros((3, 5), bool)
    mask[:, 2] = True
    np.testing.assert_array_equal(att.attention(q, _rand((5, H, D), 18), v, 0.7, mask),
                                  np.broadcast_to(v[2], (3, H, D)))
    # two keys, worked by hand: q.k1 = 2, q.k2 = 0 (per head), scale 0.5
    q = np.zeros((1, 1, 2))
    q[0, 0] = [1.0, 1.0]
    k = np.array([[[1.0, 1.0]], [[1.0, -1.0]]])
    v = np.array([[[10.0, 0.0]], [[0.0, 4.0]]])
    w1 = math.exp(1.0) / (math.exp(1.0) + math.exp(0.0))
    o = att.attention(q, k, v, 0.5)
    np.testing.assert_allclose(o[0, 0], [10.0 * w1, 4.0 * (1 - w1)], rtol=1e-15)


def test_key_order_does_not_matter():
    q, k, v = _rand((10, 2, 16), 20), _rand((50, 2, 16), 21), _rand((50, 2, 16), 22)
    perm = np.random.Generator(np.random.PCG64(23)).permutation(50)
    a = att.attention(q, k, v, 0.25)
    b = att.attention(q, k[perm], v[perm], 0.25)
    assert np.max(np.abs(a - b)) <= 1e-14
