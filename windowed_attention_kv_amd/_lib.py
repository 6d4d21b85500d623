"""ctypes loader for the C ABI in include/ll.h (libll.so, or the CPU-only recording build
libll_fake.so used by host-logic tests). Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libll.so")
# the recording build of the host layer (another build of it, e.g. a sanitizer one, via LL_FAKE_LIB)
FAKE_PATH = os.environ.get("LL_FAKE_LIB") or os.path.join(PKG, "libll_fake.so")

LL_ABI_VERSION = 1
LL_OK, LL_EINVAL, LL_ESTATE, LL_EUNSUPPORTED, LL_EDEVICE = range(5)
LL_F32, LL_BF16 = 0, 1
LL_KV_DENSE, LL_KV_FP4 = 0, 1
STATUS_NAMES = {0: "LL_OK", 1: "LL_EINVAL", 2: "LL_ESTATE", 3: "LL_EUNSUPPORTED", 4: "LL_EDEVICE"}

# every symbol include/ll.h declares
SYMBOLS = ["ll_cache_size", "ll_cache_create", "ll_cache_destroy", "ll_cache_reset",
           "ll_cache_new_shot", "ll_attn_chunk", "ll_attn_chunk_noalloc", "ll_attn_chunk_cross", "ll_cache_commit",
           "ll_cache_commit_layers", "ll_recache", "ll_kv_quant",
           "ll_cache_state", "ll_cache_export", "ll_last_error"]


class CacheDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32),
                ("num_layers", ctypes.c_int32),
                ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32),
                ("chunk_frames", ctypes.c_int32),
                ("sink_frames", ctypes.c_int32),
                ("window_frames", ctypes.c_int32),
                ("dtype", ctypes.c_int32),
                ("kv_format", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class LLError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def _declare(lib):
    lib.ll_cache_size.argtypes = [ctypes.POINTER(CacheDesc), ctypes.POINTER(ctypes.c_size_t)]
    lib.ll_cache_create.argtypes = [ctypes.POINTER(CacheDesc), _P, ctypes.c_size_t, ctypes.POINTER(_P)]
    lib.ll_cache_destroy.argtypes = [_P]
    lib.ll_cache_reset.argtypes = [_P]
    lib.ll_cache_new_shot.argtypes = [_P, _I32]
    lib.ll_attn_chunk.argtypes = [_P, _I32, _P, _P, _P, _P, _P]
    lib.ll_attn_chunk_noalloc.argtypes = [_P, _I32, _P, _P, _P, _P, _P]
    lib.ll_attn_chunk_cross.argtypes = [_P, _I32, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P]
    lib.ll_cache_commit.argtypes = [_P, _I32, _P, _P, _P]
    lib.ll_cache_commit_layers.argtypes = [_P, _I32, _I32, ctypes.POINTER(_P), ctypes.POINTER(_P), _P]
    lib.ll_recache.argtypes = [_P, _I32, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P]
    lib.ll_kv_quant.argtypes = [_P, _I64, _I32, _P, _P, _P]
    lib.ll_cache_state.argtypes = [_P, _I32, ctypes.POINTER(_I64), ctypes.POINTER(_I32)]
    lib.ll_cache_export.argtypes = [_P, _I32, _P, _P, _P, _P, _P]
    lib.ll_last_error.argtypes = []
    lib.ll_last_error.restype = ctypes.c_char_p
    for name in SYMBOLS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = None


def lib():
    """The HIP library. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m windowed_attention_kv_amd.build`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def load_fake():
    """The CPU-only build of the host layer with a recording launch backend (tests only)."""
    if not os.path.exists(FAKE_PATH):
        raise RuntimeError(f"{FAKE_PATH} is missing: build it first")
    f = _declare(ctypes.CDLL(FAKE_PATH))
    f.llfake_reset.argtypes = []
    f.llfake_fail_next.argtypes = [ctypes.c_int]
    f.llfake_set_cus.argtypes = [ctypes.c_int]
    f.llfake_count.restype = ctypes.c_int
    f.llfake_record.argtypes = [ctypes.c_int, ctypes.POINTER(_I64)]
    f.llfake_record.restype = ctypes.c_int
    return f


def check(l, status: int):
    if status != LL_OK:
        raise LLError(status, l.ll_last_error().decode(errors="replace"))
