"""ctypes loader for libkvc.so, the C-ABI library declared in include/kvc.h.

There is no fallback: if the HIP library is missing, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvc.so")

BF16, FP8_E5M2, FP8_E4M3 = 0, 1, 2
OK, EINVAL, ENOSLOT, EUNSUPPORTED, EHIP, ECORRUPT, ESTATE, ESMALLWS = 0, -1, -2, -3, -4, -5, -6, -7
STATUS_COMP_EXHAUSTED, STATUS_RAW_EXHAUSTED, STATUS_MISSING_BLOCK, STATUS_CORRUPT = 1, 2, 4, 8
NUM_BUFFERS = 8
NOALLOC_WS_BYTES = 16 << 20  # KVC_NOALLOC_WS_BYTES
BUFFER_NAMES = ("comp_pool", "raw_pool", "tail", "bases", "block_table", "comp_free", "raw_free", "counters")


class Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "dtype", "num_kv_heads", "num_q_heads", "head_dim", "block_tokens", "group_tokens", "esc_cap_bytes",
        "compressed", "max_seqs", "max_blocks_per_seq", "num_comp_slots", "num_raw_slots", "mode_set",
        "base_versions")]


class Buffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUFFER_NAMES]


class Stats(ctypes.Structure):
    _fields_ = [("comp_tiles", ctypes.c_uint64), ("raw_tiles", ctypes.c_uint64), ("groups", ctypes.c_uint64 * 4),
                ("esc_bytes", ctypes.c_uint64), ("comp_free", ctypes.c_int32), ("raw_free", ctypes.c_int32)]


class KVCError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"kvc error {code}: {msg}")
        self.code = code


# every entry point of include/kvc.h with its ctypes signature
_P = ctypes.POINTER
_vp, _i32, _u64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
SIGNATURES = {
    "kv_buffer_sizes": (ctypes.c_int, [_P(Params), _P(_sz), _P(_sz)]),
    "kv_cache_create": (ctypes.c_int, [_P(Params), _P(Buffers), _u64, _vp, _P(_vp)]),
    "kv_cache_destroy": (None, [_vp]),
    "kv_calibrate": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp]),
    "kv_recalibrate": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp]),
    "kv_encode_append": (ctypes.c_int, [_vp, _P(_i32), _i32, _vp, _vp, _i32, _vp]),
    "kv_decode_blocks": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "kv_prefill_attention": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp, _i32, ctypes.c_float, _vp, _vp]),
    "kv_attention_workspace_bytes": (_sz, [_P(Params), _i32, _i32]),
    "kv_decode_attention": (ctypes.c_int, [_vp, _P(_i32), _i32, _vp, ctypes.c_float, _i32, _vp, _sz, _vp, _vp]),
    "kv_attention_partials": (ctypes.c_int, [_vp, _P(_i32), _i32, _vp, ctypes.c_float, _i32, _vp, _sz, _vp]),
    "kv_attention_combine": (ctypes.c_int, [_vp, _P(_i32), _i32, _vp, ctypes.c_float, _i32, _vp, _sz, _vp, _vp]),
    "kv_decode_attention_noalloc": (ctypes.c_int, [_vp, _P(_i32), _i32, _vp, ctypes.c_float, _i32, _vp, _vp]),
    "kv_decode_step": (ctypes.c_int, [_vp, _P(_i32), _i32, _vp, _vp, _vp, ctypes.c_float, _i32, _vp, _sz, _vp, _vp]),
    "kv_tile_stats": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp]),
    "kv_window_coverage": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "kv_read_probe": (ctypes.c_int, [_vp, ctypes.c_uint64, _i32, _vp, _vp]),
    "kv_admit_fcfs": (ctypes.c_int, [_P(Params), _u64, ctypes.c_double, _P(_i32), _i32, _P(_i32), _P(_i32),
                                     _P(_i32)]),
    "kv_release_seq": (ctypes.c_int, [_vp, _i32, _vp]),
    "kv_seq_length": (ctypes.c_int, [_vp, _i32, _P(_i32)]),
    "kv_get_status": (ctypes.c_int, [_vp, _P(ctypes.c_uint32), _P(Stats), _vp]),
    "kv_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Load libkvc.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m decode_attention_calibrate_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(rc: int):
    if rc != OK:
        raise KVCError(rc, load().kv_last_error().decode())
    return rc
