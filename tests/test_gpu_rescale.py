"""GPU parity when a row's scores jump far above its running max in the middle of a key sweep.

The attention kernels take each 64-key tile's weights against the running max as it stands and
take the tile max (rescaling O and the row sum) only when a lane's weight sum exceeds 2^8.
These cases drive that path with keys whose scores sit ~22 (heads in the upper half) or ~46
(heads in the lower half: weights of ~2^46 against the stale max) above all earlier keys of the
row (exp2 domain), met after normal keys: in the own chunk, and one chunk later in the middle
of the cached window. Whole-block launches (16 heads, 304 query
blocks) and the split schedule (2 heads) are both covered."""
import numpy as np
import pytest

from _parity import assert_close, log, sample_rows, to_np
from oracle.model import LayerModel
from windowed_attention_kv_amd import synth

pytestmark = pytest.mark.gpu


def _bf16(x):
    bits = synth.f32_to_bf16_bits(np.asarray(x, np.float32))
    return synth.Tensor(synth.bf16_bits_to_f32(bits), bits)


@pytest.mark.parametrize("case", ["whole-blocks", "split"])
def test_score_jumps_far_above_the_running_max(case):
    from windowed_attention_kv_amd import Cache
    H, T = (16, 1560) if case == "whole-blocks" else (2, 200)
    D, C, S, W = 128, 3, 1, 3
    n = C * T
    g = np.random.Generator(np.random.PCG64(71 if case == "whole-blocks" else 72))
    log(f"case: score jumps, {case}, {H} heads x {n} rows")
    cache = Cache(1, H, D, T, C, S, W)
    model = LayerModel(S, W, C, T, H, D)

    def normal(std=0.5, mean=0.0):
        return _bf16(mean + std * g.standard_normal((n, H, D)))

    # fill the sink and window with normal keys
    for _ in range(2):
        k, v = normal(), normal(mean=0.3)
        cache.commit(0, k.torch("cuda"), v.torch("cuda"))
        model.commit(k.values, v.values, k.bits, v.bits)
    # the test chunk: queries along +1; frame 1 of its own K scores far above everything the
    # rows met before it (K ~ 3 in heads 0..H/2-1: ~46 above; K ~ 1.5 in the others: ~22)
    q = _bf16(1.0 + 0.25 * g.standard_normal((n, H, D)))
    kx = 0.5 * g.standard_normal((n, H, D))
    lo = slice(T, 2 * T)
    kx[lo, : H // 2] = 3.0 + 0.25 * g.standard_normal((T, H // 2, D))
    kx[lo, H // 2:] = 1.5 + 0.25 * g.standard_normal((T, H - H // 2, D))
    k = _bf16(kx)
    v = normal(mean=0.3)
    rows = sample_rows(n, 24, seed=73)
    o = cache.attn_chunk(0, q.torch("cuda"), k.torch("cuda"), v.torch("cuda"))
    ref = model.attn_chunk(q.values, k.values, v.values, rows=rows)
    assert_close(to_np(o)[rows], ref, "bf16", f"{case}: jump in the own chunk")
    cache.commit(0, k.torch("cuda"), v.torch("cuda"))
    model.commit(k.values, v.values, k.bits, v.bits)
    # next chunk: the large keys are now a cached frame, met in the middle of the sweep
    q2 = _bf16(1.0 + 0.25 * g.standard_normal((n, H, D)))
    k2, v2 = normal(), normal(mean=0.3)
    o2 = cache.attn_chunk(0, q2.torch("cuda"), k2.torch("cuda"), v2.torch("cuda"))
    ref2 = model.attn_chunk(q2.values, k2.values, v2.values, rows=rows)
    assert_close(to_np(o2)[rows], ref2, "bf16", f"{case}: jump in the cached window")
