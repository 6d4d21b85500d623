"""Planted mistakes in the oracle (CPU only): each plausible error must make some pin fail.

This checks the pins themselves: a dropped term, an off-by-one window, a wrong tie rule or
a wrong slot formula is caught by at least one of the tests in test_oracle_*.py.
"""
import numpy as np
import pytest

import oracle.attention as att_mod
import oracle.fp4 as fp4_mod
import oracle.ring as ring_mod
import test_oracle_attention as t_att
import test_oracle_fp4 as t_fp4
import test_oracle_model as t_model
import test_oracle_ring as t_ring
from windowed_attention_kv_amd import synth


def _window_one_longer(chunk, C, S, W, shot_start=0):
    s = chunk * C
    return sorted(set(range(shot_start, min(shot_start + S, s + C)))
                  | set(range(max(0, s - W - 1), s)) | set(range(s, s + C)))


def _sink_dropped(chunk, C, S, W, shot_start=0):
    s = chunk * C
    return sorted(set(range(max(0, s - W), s)) | set(range(s, s + C)))


def _slot_wrong(f, F, S, W, shot_start=0):
    return (f + 1) % W if f >= F - W else W + (f - shot_start)


def _spill_late(F, S, W, shot_start=0):
    return min(max(F - W - shot_start - 1, 0), S)


def _ties_to_odd(y):
    y = np.asarray(y, dtype=np.float64)
    code = np.zeros(y.shape, dtype=np.int64)
    for c in range(7):
        mid = 0.5 * (fp4_mod.GRID[c] + fp4_mod.GRID[c + 1])
        code = np.where(y >= mid, c + 1, code)
    return code


_orig_scale_bytes = fp4_mod.scale_bytes


def _scale_off_by_one(bits):
    return np.minimum(_orig_scale_bytes(bits).astype(np.int64) + 1, 254).astype(np.uint8)


_orig_logits = att_mod.logits


def _logits_no_scale(q, k, scale):
    return _orig_logits(q, k, 1.0)


def _logits_wrong_head(q, k, scale):
    z = _orig_logits(q, k, scale)
    return z[::-1].copy() if z.shape[0] > 1 else z + 0.1


MUTANTS = [
    ("window+1", ring_mod, "visible_frames", _window_one_longer,
     lambda: t_model.test_cache_path_vs_bruteforce(synth.CONFIGS["tiny"])),
    ("sink dropped", ring_mod, "visible_frames", _sink_dropped,
     lambda: t_model.test_cache_path_vs_bruteforce(synth.CONFIGS["tiny"])),
    ("slot formula", ring_mod, "slot_of_frame", _slot_wrong,
     lambda: t_ring.test_ring_vs_simulation_single_shot(3, 9, 3)),
    ("sink spill one frame late", ring_mod, "n_spilled", _spill_late,
     lambda: t_ring.test_ring_vs_simulation_multi_shot(3, 9, 3)),
    ("fp4 ties to odd", fp4_mod, "encode_magnitude", _ties_to_odd,
     t_fp4.test_exhaustive_vs_brute_force),
    ("fp4 scale off by one", fp4_mod, "scale_bytes", _scale_off_by_one,
     t_fp4.test_grid_matches_ocp_e2m1_table),
    ("logit scale dropped", att_mod, "logits", _logits_no_scale,
     lambda: t_att.test_unmasked_vs_sdpa(48, 48, 2, 64)),
    ("heads mixed up", att_mod, "logits", _logits_wrong_head,
     lambda: t_att.test_unmasked_vs_sdpa(37, 200, 3, 128)),
]


@pytest.mark.parametrize("name,mod,attr,bad,pin", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_mutant(monkeypatch, name, mod, attr, bad, pin):
    pin()                                   # the pin passes on the real oracle
    monkeypatch.setattr(mod, attr, bad)
    with pytest.raises((AssertionError, ValueError, KeyError)):
        pin()
