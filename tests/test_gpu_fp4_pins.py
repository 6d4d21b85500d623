"""GPU pins of the FP4 store's decode inside chunk attention, and FP4 at head_dim 64.

Every byte value at every scale byte: the committed V rows are built so that each e8m0 scale
byte the encoder can produce (0..252, from the block maxima of finite bf16 inputs) occurs in
blocks that together hold all 256 code bytes, and the committed K rows are distinct triples of
one-hot dimensions. A query row built on one key's triple scores that key three times as high
as any key sharing two of its dimensions (a gap of more than 300 in the exp2 domain), so its
softmax is that one key: the output row IS the key's V row as the kernel decoded it. Each
element is compared with the fp64 oracle within 2^-16 of its block's scale, which tells every
code at every scale apart, subnormal decodes (scale bytes 0 and 1) included.
"""
import itertools
import math

import numpy as np
import pytest

from _parity import assert_close, log, to_np
from oracle import fp4 as ofp4
from oracle.model import LayerModel
from windowed_attention_kv_amd import synth

pytestmark = pytest.mark.gpu

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
N_SCALES = 253                       # scale bytes 0..252
BLOCKS_PER_SCALE = 37                # 7 free bytes per block -> all 256 byte values


def _code_value(code, sb):
    mag = GRID[code & 7] * 2.0 ** (sb - 127)
    return -mag if code & 8 else mag


def _v_blocks(n_blocks, seed):
    """Scale byte and the 8 code bytes of each of n_blocks blocks. Block byte 0 is 0x77 (two
    6.0 codes, so the block maximum fixes the scale byte); bytes 1..7 of the 37 blocks of one
    scale byte run through all 256 values. Blocks past the 253 x 37 that cover every pair get
    random bytes at scale byte 127."""
    g = np.random.Generator(np.random.PCG64(seed))
    sb = np.full(n_blocks, 127, np.int64)
    by = g.integers(0, 256, size=(n_blocks, 8))
    by[:, 0] = 0x77
    for s in range(N_SCALES):
        for j in range(BLOCKS_PER_SCALE):
            b = s * BLOCKS_PER_SCALE + j
            sb[b] = s
            by[b, 1:] = (j * 7 + np.arange(7)) % 256
    return sb, by


def _blocks_to_bits(sb, by):
    """bf16 bit patterns [n_blocks, 16] holding exactly the blocks' decoded values."""
    codes = np.empty((sb.size, 16), np.int64)
    codes[:, 0::2] = by & 0xF
    codes[:, 1::2] = by >> 4
    vals = np.vectorize(_code_value)(codes, sb[:, None])
    f32 = vals.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), vals)
    return synth.f32_to_bf16_bits(f32), codes


@pytest.mark.parametrize("D", [128, 64])
def test_fp4_decode_of_every_byte_at_every_scale(D):
    import torch
    from windowed_attention_kv_amd import Cache
    H, C, S, W = 2, 3, 3, 9
    bpr = D // 16                                  # blocks per (token, head) row
    need_rows = -(-N_SCALES * BLOCKS_PER_SCALE // bpr)
    T = -(-need_rows // (S + W))
    T = -(-T // 4) * 4
    n_keys = (S + W) * T
    log(f"case: FP4 decode pin, D={D}, T={T}, {n_keys} cache keys per head")
    # K: key j is 32 at the dims of the j-th triple; Q: 80 at its target key's triple
    triples = list(itertools.islice(itertools.combinations(range(D), 3), n_keys))
    kf = np.zeros((n_keys, D), np.float32)
    for j, tr in enumerate(triples):
        kf[j, list(tr)] = 32.0
    # V: head 0 takes the blocks in key order, head 1 the same rows in reverse key order
    sb, by = _v_blocks(n_keys * bpr, seed=D)
    vbits, _ = _blocks_to_bits(sb, by)
    vrow = vbits.reshape(n_keys, D)
    kbits = synth.f32_to_bf16_bits(kf)
    K = np.stack([kbits, kbits], axis=1)                       # [n_keys, H, D]
    V = np.stack([vrow, vrow[::-1]], axis=1)
    sbh = np.stack([sb.reshape(n_keys, bpr), sb.reshape(n_keys, bpr)[::-1]], axis=1)
    # the oracle encoder reproduces the intended codes and scales exactly
    pk, sc = ofp4.quantize(V.reshape(-1, D))
    assert np.array_equal(sc.reshape(n_keys, H, bpr), sbh)
    assert np.array_equal(pk.reshape(n_keys, H, D // 2)[:, 0, :].reshape(-1, 8), by)

    shape = synth.shrink(synth.CONFIGS["layer"], name=f"fp4-pin-d{D}", heads=H, head_dim=D,
                         tokens_per_frame=T, window_frames=W)
    cache = Cache(1, H, D, T, C, S, W, kv_format="fp4")
    model = LayerModel(S, W, C, T, H, D, kv_format="fp4")
    n = C * T
    as_bf16 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    val = lambda bits: synth.bf16_bits_to_f32(bits)
    for c in range((S + W) // C):
        rows = slice(c * n, (c + 1) * n)
        cache.commit(0, as_bf16(K[rows]), as_bf16(V[rows]))
        model.commit(val(K[rows]), val(V[rows]), K[rows], V[rows])
    # own chunk: K = 0 (score 0), V = 0
    zero = np.zeros((n, H, D), np.uint16)
    tz = as_bf16(zero)
    worst_rel = 0.0
    exact = 0
    dec = ofp4.dequantize(pk, sc).reshape(n_keys, H, D)
    for call in range(-(-n_keys // n)):
        target = np.minimum(np.arange(call * n, (call + 1) * n), n_keys - 1)
        qf = np.zeros((n, D), np.float32)
        for i, j in enumerate(target):
            qf[i, list(triples[j])] = 80.0
        qbits = synth.f32_to_bf16_bits(qf)
        Q = np.stack([qbits, qbits], axis=1)
        o = to_np(cache.attn_chunk(0, as_bf16(Q), tz, tz))
        ref = model.attn_chunk(val(Q), val(zero), val(zero))
        # the softmax of every row is its target key: the oracle's output is that key's
        # decoded V row (up to terms below 2^-300 of it)
        assert np.allclose(ref, dec[target], rtol=0, atol=0) or \
            np.all(np.abs(ref - dec[target]) <= 2.0 ** (np.repeat(sbh[target], 16, axis=2) - 127 - 40))
        tol = 2.0 ** (np.repeat(sbh[target], 16, axis=2) - 127 - 16)
        err = np.abs(o - ref)
        bad = err > tol
        assert not bad.any(), (f"call {call}: {int(bad.sum())} decoded values off, first at "
                               f"{np.argwhere(bad)[0]} (scale byte "
                               f"{np.repeat(sbh[target], 16, axis=2)[tuple(np.argwhere(bad)[0])]})")
        exact += int(np.sum(o == dec[target]))
        nz = np.linalg.norm(ref)
        worst_rel = max(worst_rel, float(np.linalg.norm(o - ref) / nz) if nz else 0.0)
    log(f"FP4 decode pin D={D}: {exact} of {n_keys * H * D} values bit-identical to the "
        f"oracle's decode, worst rel-L2 {worst_rel:.2e}")


@pytest.mark.parametrize("kind", ["stream", "rising", "shots", "recache"])
def test_fp4_head_dim_64(kind):
    """The FP4 store at head_dim 64 (the 4-wave kernel's register-staged decode and the
    one-group-per-row quantising commit): a stream past the window wrap and the sink spill,
    rising scores that force mid-sweep rescales, multi-shot sinks, and a recache; every chunk
    compared and every export bit-exact."""
    from test_gpu_parity import _recache_case, run_stream
    shape = synth.shrink(synth.CONFIGS["layer"], name=f"fp4-d64-{kind}", heads=3, head_dim=64,
                         tokens_per_frame=72, window_frames=6)
    log(f"case: FP4 head_dim 64, {kind}")
    if kind == "stream":
        run_stream(shape, 9, kv_format="fp4")
    elif kind == "rising":
        run_stream(shape, 8, kv_format="fp4", k_frame_gain=2.0)
    elif kind == "shots":
        run_stream(shape, 12, kv_format="fp4", shots=(3, 4, 8))
    else:
        _recache_case(shape, 5, n_text=40, kv_format="fp4")
