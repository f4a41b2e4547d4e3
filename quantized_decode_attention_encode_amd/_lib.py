"""ctypes loader for libkvq.so (the C ABI of include/kvq.h).

There is no fallback: if the library has not been built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY may point at another build of the same ABI (e.g. a tuning variant); the default
# is the in-tree library.
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(HERE, "libkvq.so")

KVQ_OK = 0
KVQ_E_INVALID = -1
KVQ_E_UNSUPPORTED = -2
KVQ_E_CAPACITY = -3
KVQ_E_WORKSPACE = -4
KVQ_E_NODEVICE = -5
KVQ_E_HIP = -6
KVQ_MAX_BATCH = 256
KVQ_NOALLOC_SCRATCH_BYTES = 8 << 20


class KVQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status
        self.message = message


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_kv_heads", "n_q_heads", "head_dim", "key_bits", "value_bits", "group", "residual",
        "max_tokens", "n_sink", "method", "skvq_reorder", "skvq_clip_search")] + [("skvq_clip_alpha", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("kitty_n_hi", "kitty_hi_bits")]


METHOD_KIVI, METHOD_SKVQ, METHOD_KITTY = 0, 1, 2


class LayoutInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "lengths_offset", "records_offset", "record_bytes", "rec_key_codes", "rec_value_codes",
        "rec_key_params", "rec_value_params", "window_k_offset", "window_v_offset", "total_bytes",
        "sync_offset", "sink_pos_offset", "sink_k_offset", "sink_v_offset", "perm_offset", "rec_slot_table",
        "kstats_offset")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python quantized_decode_attention_encode_amd/build.py` "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    pcfg = ctypes.POINTER(Config)
    pi32 = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "kvq_probe": (I32, [pi32]),
        "kvq_config_check": (I32, [pcfg]),
        "kvq_kitty_n_hi": (I32, [I32, ctypes.c_double, pi32]),
        "kvq_cache_bytes": (SZ, [pcfg]),
        "kvq_layout": (I32, [pcfg, ctypes.POINTER(LayoutInfo)]),
        "kvq_workspace_bytes": (SZ, [pcfg, I32]),
        "kvq_cache_create": (I32, [pcfg, P, SZ, ctypes.POINTER(P)]),
        "kvq_cache_destroy": (None, [P]),
        "kvq_reset": (I32, [P, P]),
        "kvq_cache_lengths": (I32, [P, pi32, pi32]),
        "kvq_encode": (I32, [P, P, P, I64, pi32, P]),
        "kvq_encode_block": (I32, [P, I32, I32, I32, I32, I32, P, P, P, P]),
        "kvq_prefill": (I32, [P, P, P, I64, pi32, P]),
        "kvq_append": (I32, [P, P, P, P]),
        "kvq_decode_attend": (I32, [P, P, P, I32, F32, P, SZ, I32, P]),
        "kvq_append_decode_attend": (I32, [P, P, P, P, P, I32, F32, P, SZ, I32, P]),
        "kvq_decode_attend_multi": (I32, [P, P, P, I32, I32, F32, P, SZ, I32, P]),
        "kvq_decode_attend_noalloc": (I32, [P, P, P, I32, F32, I32, P]),
        "kvq_profile_enable": (I32, [P, I32]),
        "kvq_profile_read": (I32, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
        "kvq_last_error": (ctypes.c_char_p, []),
        "kvq_status_string": (ctypes.c_char_p, [I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
EXPORTED = ("kvq_probe", "kvq_config_check", "kvq_kitty_n_hi", "kvq_cache_bytes", "kvq_layout", "kvq_workspace_bytes",
            "kvq_cache_create", "kvq_cache_destroy", "kvq_reset", "kvq_cache_lengths", "kvq_encode", "kvq_encode_block",
            "kvq_prefill", "kvq_append", "kvq_decode_attend", "kvq_append_decode_attend", "kvq_decode_attend_multi", "kvq_decode_attend_noalloc",
            "kvq_profile_enable", "kvq_profile_read",
            "kvq_last_error", "kvq_status_string")


def status_name(status: int) -> str:
    return lib.kvq_status_string(status).decode()


def check(status: int) -> None:
    if status != KVQ_OK:
        raise KVQError(status, lib.kvq_last_error().decode())
