"""ctypes loader for libdq.so (argument types of every C ABI entry point)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(PKG, "libdq.so")


class CodecDesc(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("levels", ctypes.c_int32),
                ("container_bytes", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("step64", ctypes.c_int32),
                ("drift_order", ctypes.c_int32)]


_handle = None


def lib():
    """Loads libdq.so once.  Raises (never falls back) when it is missing."""
    global _handle
    if _handle is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} not built: run `python -m kv_cache_entropy_amd.build`")
        L = ctypes.CDLL(LIB)
        vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        L.dq_status_string.restype = ctypes.c_char_p
        L.dq_status_string.argtypes = [ctypes.c_int]
        L.dq_version.restype = ctypes.c_int
        L.dq_version.argtypes = []
        L.dq_set_knob.restype = ctypes.c_int
        L.dq_set_knob.argtypes = [ctypes.c_int, i64]
        L.dq_get_knob.restype = i64
        L.dq_get_knob.argtypes = [ctypes.c_int]
        L.dq_codec_create.argtypes = [ctypes.POINTER(CodecDesc), ctypes.POINTER(vp)]
        L.dq_codec_destroy.argtypes = [vp]
        L.dq_codec_info.argtypes = [vp, ctypes.POINTER(CodecDesc)]
        L.dq_codec_tables.argtypes = [vp, vp, vp, vp, vp]
        L.dq_encode.argtypes = [vp, vp, i64, i64, i64, vp, i64, vp, vp, vp, vp]
        L.dq_encode_kv.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp]
        L.dq_decode_symbols.argtypes = [vp, vp, i64, i32, vp, i64, vp, vp, vp, vp]
        L.dq_attn_decode_workspace.argtypes = [i32, i32, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
        L.dq_attn_decode.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp, i64, vp, vp, i64,
                                     ctypes.c_float, i32, vp, vp, ctypes.c_size_t, vp]
        L.dq_attn_decode_timed.argtypes = L.dq_attn_decode.argtypes + [vp, vp]
        L.dq_attn_decode_noalloc.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp, i64, vp, vp, i64,
                                             ctypes.c_float, i32, vp, vp]
        L.dq_attn_prefill_workspace.argtypes = [i32, i32, i32, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
        L.dq_attn_prefill.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, i64, vp, vp, i64,
                                      ctypes.c_float, i32, vp, vp, ctypes.c_size_t, vp]
        L.dq_attn_decode_paged.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp, i64, vp, i32, vp,
                                           i64, ctypes.c_float, i32, vp, vp, ctypes.c_size_t, vp]
        # (ck, cv, q, B, Hq, k_new, v_new, stride_b, stride_h, kc, kn, vc, vn, S) + where +
        # (seq_len, max_len, sm_scale, out_dtype, out, ws, ws_bytes, k_stats, v_stats, stream)
        app_head = [vp, vp, vp, i32, i32, vp, vp, i64, i64, vp, vp, vp, vp, i64]
        app_tail = [vp, i64, ctypes.c_float, i32, vp, vp, ctypes.c_size_t, vp, vp, vp]
        L.dq_attn_decode_append.argtypes = app_head + [vp] + app_tail
        L.dq_attn_decode_paged_append.argtypes = app_head + [vp, i32] + app_tail
        L.dq_attn_decode_append_timed.argtypes = app_head + [vp] + app_tail + [vp, vp]
        for f in ("dq_codec_create", "dq_codec_destroy", "dq_codec_info", "dq_codec_tables",
                  "dq_encode", "dq_encode_kv", "dq_decode_symbols", "dq_attn_decode_workspace",
                  "dq_attn_decode", "dq_attn_decode_timed", "dq_attn_decode_paged", "dq_attn_decode_noalloc",
                  "dq_attn_prefill_workspace", "dq_attn_prefill", "dq_attn_decode_append",
                  "dq_attn_decode_paged_append", "dq_attn_decode_append_timed"):
            getattr(L, f).restype = ctypes.c_int
        del u64
        _handle = L
    return _handle
