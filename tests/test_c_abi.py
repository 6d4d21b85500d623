"""The C ABI from a plain-C program (tests/c_abi_stream.c, built by build() with gcc against
include/ll.h and libll.so; no Python, no torch): it streams chunks through one layer with
ll_cache_size / ll_cache_create / ll_attn_chunk / ll_cache_commit / ll_cache_state on device
memory from the HIP runtime, reading its inputs from and writing its outputs to files. The GPU
test compares every chunk's output with the oracle."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

from _parity import assert_close, log
from oracle.model import LayerModel
from windowed_attention_kv_amd import _lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi_stream")


def _need_bin():
    if not os.path.exists(BIN):
        pytest.skip("tests/c_abi_stream not built (run build())")


def test_c_consumer_builds_against_the_header():
    """The program compiled and linked against include/ll.h and libll.so (-Wall -Wextra
    -Werror) and reports the header's ABI version without touching a GPU."""
    _need_bin()
    r = subprocess.run([BIN, "--abi"], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=60)
    assert r.returncode == 0, r.stderr
    assert int(r.stdout.strip()) == _lib.LL_ABI_VERSION


@pytest.mark.gpu
@pytest.mark.parametrize("kv_format", ["dense", "fp4"])
def test_c_consumer_stream_matches_the_oracle(kv_format):
    _need_bin()
    shape = synth.shrink(synth.CONFIGS["layer"], name=f"c-abi-{kv_format}", heads=2,
                         tokens_per_frame=72, window_frames=6)
    chunks = 6
    H, D, T, C, S, W = (shape.heads, shape.head_dim, shape.tokens_per_frame, shape.chunk_frames,
                        shape.sink_frames, shape.window_frames)
    log(f"case: plain-C consumer, {kv_format}, {chunks} chunks")
    model = LayerModel(S, W, C, T, H, D, kv_format=kv_format)
    with tempfile.TemporaryDirectory() as d:
        with open(os.path.join(d, "desc.txt"), "w") as f:
            f.write(f"{H} {D} {T} {C} {S} {W} {chunks} 1 {1 if kv_format == 'fp4' else 0}\n")
        ins = [synth.chunk_inputs(shape, 0, 0, c, salt=61) for c in range(chunks)]
        for c, trip in enumerate(ins):
            for name, t in zip("qkv", trip):
                np.ascontiguousarray(t.bits).tofile(os.path.join(d, f"{name}_{c}.bin"))
        r = subprocess.run([BIN, d], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                           timeout=120)
        assert r.returncode == 0, r.stderr
        assert f"frames committed {chunks * C}" in r.stdout
        for c, (q, k, v) in enumerate(ins):
            bits = np.fromfile(os.path.join(d, f"o_{c}.bin"), dtype=np.uint16).reshape(q.bits.shape)
            o = synth.bf16_bits_to_f32(bits)
            assert_close(o, model.attn_chunk(q.values, k.values, v.values), "bf16",
                         f"C consumer, {kv_format}, chunk {c}")
            model.commit(k.values, v.values, k.bits, v.bits)
