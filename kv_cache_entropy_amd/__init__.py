"""D-Quant hot path on MI355X: driftable rANS KV-cache coding and decode
attention over the coded cache.

Thin binding over the C ABI in include/dq.h (libdq.so, built by
``python -m kv_cache_entropy_amd.build``).  This module only checks and
marshals arguments: every step of the computation runs in the HIP kernels.
torch is used for device memory and the current stream.  If libdq.so is
missing or fails to load, every entry point raises; there is no fallback.

    ck = Codec(levels=8, container_bytes=34, seed=1, kv_heads=8)
    cont, norm = alloc_pool(ck, num_slots, device="cuda")
    encode(ck, k_bf16, slots, cont, norm)
    out = attn_decode(ck, cv, q, kc, kn, vc, vn, seq_start, seq_len, max_len)
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import _lib

HEAD_DIM = 128
MAX_CONTAINER = 132
PAGE_TOKENS = 64
NSTATS = 6 + MAX_CONTAINER + 1

__all__ = ["Codec", "set_knob", "get_knob", "knobs", "alloc_pool", "encode", "encode_kv", "decode_symbols",
           "attn_decode", "attn_decode_noalloc", "attn_decode_paged",
           "attn_prefill", "attn_prefill_workspace_bytes",
           "attn_workspace_bytes", "new_stats", "stats_dict", "DQError", "library_path"]


class DQError(RuntimeError):
    pass


def library_path() -> str:
    return _lib.LIB


def _check(status: int, what: str):
    if status != 0:
        msg = _lib.lib().dq_status_string(status).decode()
        raise DQError(f"{what}: {msg} ({status})")


# Path overrides of the C ABI (dq_set_knob): -1 (or None) = the library's own
# choice.  Tests force each code path with them; results do not depend on them
# except for the split length (floating-point order of the attention sums).
KNOBS = {"split_tokens": 1, "latency_mode": 2, "append_fuse": 3, "encode_wave_max": 4,
         "encode_key_span": 5, "splitk_waves": 6, "work_queue": 7, "slot_table": 8,
         "encode_two_pass": 9, "qk_valu": 10}


def set_knob(name: str, value) -> None:
    _check(_lib.lib().dq_set_knob(KNOBS[name], -1 if value is None else int(value)), f"dq_set_knob({name})")


def get_knob(name: str) -> int:
    return int(_lib.lib().dq_get_knob(KNOBS[name]))


class knobs:
    """Context manager: ``with knobs(split_tokens=64): ...`` forces the given
    paths and restores the previous values on exit."""

    def __init__(self, **kw):
        self._kw = kw
        self._old = {}

    def __enter__(self):
        for k, v in self._kw.items():
            self._old[k] = get_knob(k)
            set_knob(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self._old.items():
            set_knob(k, v)
        return False


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_cuda(name, t, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise DQError(f"{name} must be a CUDA/HIP tensor")
    if dtype is not None and t.dtype != dtype:
        raise DQError(f"{name} must have dtype {dtype}, got {t.dtype}")


class Codec:
    """One coded stream (K or V): level count, container bytes, rotation
    seed, kv heads, cell width (step64 / 64 sigma; 0 = default) and drift
    order (0 magnitude, 1 rate-distortion)."""

    def __init__(self, levels: int, container_bytes: int, seed: int, kv_heads: int,
                 step64: int = 0, drift_order: int = 0):
        L = _lib.lib()
        desc = _lib.CodecDesc(HEAD_DIM, levels, container_bytes, kv_heads,
                              seed & (2**64 - 1), step64, drift_order)
        h = ctypes.c_void_p()
        _check(L.dq_codec_create(ctypes.byref(desc), ctypes.byref(h)), "dq_codec_create")
        self._h = h
        info = _lib.CodecDesc()
        _check(L.dq_codec_info(h, ctypes.byref(info)), "dq_codec_info")
        self.levels = info.levels
        self.C = info.container_bytes
        self.seed = info.seed
        self.kv_heads = info.num_kv_heads
        self.step64 = info.step64
        self.drift_order = info.drift_order

    @property
    def handle(self):
        return self._h

    def tables(self) -> dict:
        import numpy as np
        L = self.levels
        f = np.zeros(L, np.uint16)
        c = np.zeros(L + 1, np.uint16)
        r = np.zeros(L, np.uint16)
        w = np.zeros(2 * self.kv_heads, np.uint64)
        _check(_lib.lib().dq_codec_tables(
            self._h, f.ctypes.data_as(ctypes.c_void_p), c.ctypes.data_as(ctypes.c_void_p),
            r.ctypes.data_as(ctypes.c_void_p), w.ctypes.data_as(ctypes.c_void_p)),
            "dq_codec_tables")
        return {"freq": f, "cum": c, "recon_f16": r, "sign_words": w}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _lib.lib().dq_codec_destroy(h)
            except Exception:
                pass
            self._h = None


def pool_slots(num_slots: int, C: int = 0) -> int:
    """num_slots rounded up to a multiple of 16, so that slots * C is a
    multiple of 16 bytes for every container size (K and V pools with
    different C then share slot numbering)."""
    return (num_slots + 15) // 16 * 16


def alloc_pool(codec: Codec, num_slots: int, device="cuda"):
    """Zeroed (cont uint8 [Hkv, S, C], norm fp16 [Hkv, S]) with S padded so the
    plane size is a multiple of 16 bytes."""
    S = pool_slots(num_slots, codec.C)
    cont = torch.zeros((codec.kv_heads, S, codec.C), dtype=torch.uint8, device=device)
    norm = torch.zeros((codec.kv_heads, S), dtype=torch.float16, device=device)
    return cont, norm


def new_stats(device="cuda") -> torch.Tensor:
    return torch.zeros(NSTATS, dtype=torch.int64, device=device)


def stats_dict(stats: torch.Tensor) -> dict:
    s = [int(v) for v in stats.cpu().tolist()]
    return {"vectors": s[0], "drifted_vectors": s[1], "drifted_symbols": s[2],
            "multilevel_events": s[3], "bad_norms": s[4], "zero_norms": s[5],
            "len_hist": s[6:]}


def encode(codec: Codec, x: torch.Tensor, slots: torch.Tensor, cont: torch.Tensor,
           norm: torch.Tensor, stats: torch.Tensor | None = None):
    """x: bf16 [T, Hkv, 128] (last dim contiguous); slots: int64 [T];
    cont/norm: the pool from alloc_pool; stats: int64 [NSTATS] or None."""
    _need_cuda("x", x, torch.bfloat16)
    _need_cuda("slots", slots, torch.int64)
    _need_cuda("cont", cont, torch.uint8)
    _need_cuda("norm", norm, torch.float16)
    if x.dim() != 3 or x.shape[1] != codec.kv_heads or x.shape[2] != HEAD_DIM or x.stride(2) != 1:
        raise DQError(f"x must be [T, {codec.kv_heads}, 128] with unit inner stride")
    if slots.dim() != 1 or slots.shape[0] != x.shape[0] or not slots.is_contiguous():
        raise DQError("slots must be a contiguous int64 [T]")
    if (cont.dim() != 3 or cont.shape[0] != codec.kv_heads or cont.shape[2] != codec.C
            or not cont.is_contiguous()):
        raise DQError("cont must be a contiguous uint8 [Hkv, S, C]")
    if norm.shape != cont.shape[:2] or not norm.is_contiguous():
        raise DQError("norm must be a contiguous fp16 [Hkv, S]")
    if stats is not None:
        _need_cuda("stats", stats, torch.int64)
        if stats.numel() != NSTATS or not stats.is_contiguous():
            raise DQError(f"stats must be a contiguous int64 [{NSTATS}]")
    _check(_lib.lib().dq_encode(codec.handle, _ptr(x), x.shape[0], x.stride(0), x.stride(1),
                                _ptr(slots), cont.shape[1], _ptr(cont), _ptr(norm),
                                _ptr(stats), _stream(x.device)), "dq_encode")


def encode_kv(ck: Codec, cv: Codec, k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor,
              k_cont: torch.Tensor, k_norm: torch.Tensor, v_cont: torch.Tensor, v_norm: torch.Tensor,
              k_stats: torch.Tensor | None = None, v_stats: torch.Tensor | None = None):
    """encode(ck, k, ...) and encode(cv, v, ...) with shared slots, in one
    launch when both are small batches.  k, v: bf16 [T, Hkv, 128] with the
    same strides."""
    for name, x in (("k", k), ("v", v)):
        _need_cuda(name, x, torch.bfloat16)
        if x.dim() != 3 or x.shape[1] != ck.kv_heads or x.shape[2] != HEAD_DIM or x.stride(2) != 1:
            raise DQError(f"{name} must be [T, {ck.kv_heads}, 128] with unit inner stride")
    if k.shape != v.shape or k.stride() != v.stride():
        raise DQError("k and v must have the same shape and strides")
    _need_cuda("slots", slots, torch.int64)
    if slots.dim() != 1 or slots.shape[0] != k.shape[0] or not slots.is_contiguous():
        raise DQError("slots must be a contiguous int64 [T]")
    for name, codec, cont, norm in (("k", ck, k_cont, k_norm), ("v", cv, v_cont, v_norm)):
        _need_cuda(f"{name}_cont", cont, torch.uint8)
        _need_cuda(f"{name}_norm", norm, torch.float16)
        if (cont.dim() != 3 or cont.shape[0] != codec.kv_heads or cont.shape[2] != codec.C
                or not cont.is_contiguous() or norm.shape != cont.shape[:2] or not norm.is_contiguous()):
            raise DQError(f"{name} pool must be contiguous [Hkv, S, C] / [Hkv, S]")
    if k_cont.shape[1] != v_cont.shape[1]:
        raise DQError("K and V pools must have the same slot count")
    for st in (k_stats, v_stats):
        if st is not None:
            _need_cuda("stats", st, torch.int64)
            if st.numel() != NSTATS or not st.is_contiguous():
                raise DQError(f"stats must be a contiguous int64 [{NSTATS}]")
    _check(_lib.lib().dq_encode_kv(ck.handle, cv.handle, _ptr(k), _ptr(v), k.shape[0], k.stride(0),
                                   k.stride(1), _ptr(slots), k_cont.shape[1], _ptr(k_cont), _ptr(k_norm),
                                   _ptr(v_cont), _ptr(v_norm), _ptr(k_stats), _ptr(v_stats),
                                   _stream(k.device)), "dq_encode_kv")


def decode_symbols(codec: Codec, cont: torch.Tensor, head: int, slots: torch.Tensor):
    """Returns (symbols uint8 [n, 128], final_state int64 [n], consumed int32 [n])."""
    _need_cuda("cont", cont, torch.uint8)
    _need_cuda("slots", slots, torch.int64)
    n = slots.shape[0]
    sym = torch.empty((n, HEAD_DIM), dtype=torch.uint8, device=cont.device)
    fs = torch.empty(n, dtype=torch.int32, device=cont.device)
    cons = torch.empty(n, dtype=torch.int32, device=cont.device)
    _check(_lib.lib().dq_decode_symbols(codec.handle, _ptr(cont), cont.shape[1], head,
                                        _ptr(slots.contiguous()), n, _ptr(sym), _ptr(fs),
                                        _ptr(cons), _stream(cont.device)), "dq_decode_symbols")
    return sym, fs.to(torch.int64) & 0xFFFFFFFF, cons


def attn_workspace_bytes(B: int, Hq: int, Hkv: int, max_len: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.lib().dq_attn_decode_workspace(B, Hq, Hkv, max_len, ctypes.byref(n)),
           "dq_attn_decode_workspace")
    return n.value


def attn_decode(ck: Codec, cv: Codec, q: torch.Tensor, k_cont, k_norm, v_cont, v_norm,
                seq_start: torch.Tensor, seq_len: torch.Tensor, max_len: int,
                sm_scale: float | None = None, out: torch.Tensor | None = None,
                out_dtype=torch.float32, workspace: torch.Tensor | None = None,
                split_events=None):
    """q: bf16 [B, Hq, 128]; pools from alloc_pool; seq_start int64 [B];
    seq_len int32 [B] (1 <= len <= max_len).  Returns out [B, Hq, 128].

    split_events: optional (begin, end) torch.cuda.Event pair, recorded on
    the current stream around the split-K kernel alone."""
    _need_cuda("q", q, torch.bfloat16)
    for name, t, dt in (("k_cont", k_cont, torch.uint8), ("v_cont", v_cont, torch.uint8),
                        ("k_norm", k_norm, torch.float16), ("v_norm", v_norm, torch.float16),
                        ("seq_start", seq_start, torch.int64), ("seq_len", seq_len, torch.int32)):
        _need_cuda(name, t, dt)
        if not t.is_contiguous():
            raise DQError(f"{name} must be contiguous")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise DQError("q must be a contiguous bf16 [B, Hq, 128]")
    if k_cont.shape[1] != v_cont.shape[1]:
        raise DQError("K and V pools must have the same slot count")
    B, Hq, _ = q.shape
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise DQError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (B, Hq, HEAD_DIM) or not out.is_contiguous():
        raise DQError("out has the wrong shape or dtype")
    need = attn_workspace_bytes(B, Hq, ck.kv_heads, max_len)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if sm_scale is None:
        sm_scale = HEAD_DIM ** -0.5
    args = (ck.handle, cv.handle, _ptr(q), B, Hq, _ptr(k_cont), _ptr(k_norm), _ptr(v_cont),
            _ptr(v_norm), k_cont.shape[1], _ptr(seq_start), _ptr(seq_len), max_len,
            ctypes.c_float(sm_scale), 0 if out_dtype == torch.float32 else 1, _ptr(out),
            _ptr(workspace), workspace.numel(), _stream(q.device))
    if split_events is None:
        _check(_lib.lib().dq_attn_decode(*args), "dq_attn_decode")
    else:
        _check(_lib.lib().dq_attn_decode_timed(*args, *_event_handles(split_events)), "dq_attn_decode_timed")
    return out


def attn_decode_noalloc(ck: Codec, cv: Codec, q: torch.Tensor, k_cont, k_norm, v_cont, v_norm,
                        seq_start: torch.Tensor, seq_len: torch.Tensor, max_len: int,
                        sm_scale: float | None = None, out: torch.Tensor | None = None,
                        out_dtype=torch.float32):
    """attn_decode through dq_attn_decode_noalloc: the library's own device
    array is the workspace (no allocation in the call; pass `out` to keep
    this wrapper from allocating the result).  Calls that overlap on one GPU
    race; a shape whose workspace exceeds the array raises DQError."""
    _need_cuda("q", q, torch.bfloat16)
    for name, t, dt in (("k_cont", k_cont, torch.uint8), ("v_cont", v_cont, torch.uint8),
                        ("k_norm", k_norm, torch.float16), ("v_norm", v_norm, torch.float16),
                        ("seq_start", seq_start, torch.int64), ("seq_len", seq_len, torch.int32)):
        _need_cuda(name, t, dt)
        if not t.is_contiguous():
            raise DQError(f"{name} must be contiguous")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise DQError("q must be a contiguous bf16 [B, Hq, 128]")
    if k_cont.shape[1] != v_cont.shape[1]:
        raise DQError("K and V pools must have the same slot count")
    B, Hq, _ = q.shape
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise DQError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (B, Hq, HEAD_DIM) or not out.is_contiguous():
        raise DQError("out has the wrong shape or dtype")
    if sm_scale is None:
        sm_scale = HEAD_DIM ** -0.5
    _check(_lib.lib().dq_attn_decode_noalloc(
        ck.handle, cv.handle, _ptr(q), B, Hq, _ptr(k_cont), _ptr(k_norm), _ptr(v_cont), _ptr(v_norm),
        k_cont.shape[1], _ptr(seq_start), _ptr(seq_len), max_len, ctypes.c_float(sm_scale),
        0 if out_dtype == torch.float32 else 1, _ptr(out), _stream(q.device)), "dq_attn_decode_noalloc")
    return out


def attn_decode_paged(ck: Codec, cv: Codec, q: torch.Tensor, k_cont, k_norm, v_cont, v_norm,
                      pages: torch.Tensor, seq_len: torch.Tensor, max_len: int,
                      sm_scale: float | None = None, out: torch.Tensor | None = None,
                      out_dtype=torch.float32, workspace: torch.Tensor | None = None):
    """attn_decode over a paged pool: pages int32 [B, max_pages], token t of
    sequence b in slot pages[b, t // 64] * 64 + t % 64."""
    _need_cuda("q", q, torch.bfloat16)
    for name, t, dt in (("k_cont", k_cont, torch.uint8), ("v_cont", v_cont, torch.uint8),
                        ("k_norm", k_norm, torch.float16), ("v_norm", v_norm, torch.float16),
                        ("pages", pages, torch.int32), ("seq_len", seq_len, torch.int32)):
        _need_cuda(name, t, dt)
        if not t.is_contiguous():
            raise DQError(f"{name} must be contiguous")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise DQError("q must be a contiguous bf16 [B, Hq, 128]")
    B, Hq, _ = q.shape
    if pages.dim() != 2 or pages.shape[0] != B:
        raise DQError("pages must be int32 [B, max_pages]")
    if k_cont.shape[1] != v_cont.shape[1]:
        raise DQError("K and V pools must have the same slot count")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise DQError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (B, Hq, HEAD_DIM) or not out.is_contiguous():
        raise DQError("out has the wrong shape or dtype")
    need = attn_workspace_bytes(B, Hq, ck.kv_heads, max_len)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if sm_scale is None:
        sm_scale = HEAD_DIM ** -0.5
    _check(_lib.lib().dq_attn_decode_paged(
        ck.handle, cv.handle, _ptr(q), B, Hq, _ptr(k_cont), _ptr(k_norm), _ptr(v_cont),
        _ptr(v_norm), k_cont.shape[1], _ptr(pages), pages.shape[1], _ptr(seq_len), max_len,
        ctypes.c_float(sm_scale), 0 if out_dtype == torch.float32 else 1, _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(q.device)), "dq_attn_decode_paged")
    return out


def _event_handles(events):
    handles = []
    for ev in events:
        if ev.cuda_event == 0:  # torch creates the HIP event on first record
            ev.record()
        handles.append(ctypes.c_void_p(ev.cuda_event))
    return handles


def _attn_decode_append(ck: Codec, cv: Codec, q, k_new, v_new, k_cont, k_norm, v_cont, v_norm,
                        loc, seq_len, max_len, sm_scale, out, out_dtype, workspace, k_stats, v_stats,
                        paged: bool, split_events=None):
    _need_cuda("q", q, torch.bfloat16)
    loc_name, loc_dt = ("pages", torch.int32) if paged else ("seq_start", torch.int64)
    for name, t, dt in (("k_cont", k_cont, torch.uint8), ("v_cont", v_cont, torch.uint8),
                        ("k_norm", k_norm, torch.float16), ("v_norm", v_norm, torch.float16),
                        (loc_name, loc, loc_dt), ("seq_len", seq_len, torch.int32)):
        _need_cuda(name, t, dt)
        if not t.is_contiguous():
            raise DQError(f"{name} must be contiguous")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise DQError("q must be a contiguous bf16 [B, Hq, 128]")
    B, Hq, _ = q.shape
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        _need_cuda(name, x, torch.bfloat16)
        if tuple(x.shape) != (B, ck.kv_heads, HEAD_DIM) or x.stride(2) != 1:
            raise DQError(f"{name} must be [B, {ck.kv_heads}, 128] with unit inner stride")
    if k_new.stride() != v_new.stride():
        raise DQError("k_new and v_new must have the same strides")
    if paged and (loc.dim() != 2 or loc.shape[0] != B):
        raise DQError("pages must be int32 [B, max_pages]")
    if k_cont.shape[1] != v_cont.shape[1]:
        raise DQError("K and V pools must have the same slot count")
    for st in (k_stats, v_stats):
        if st is not None:
            _need_cuda("stats", st, torch.int64)
            if st.numel() != NSTATS or not st.is_contiguous():
                raise DQError(f"stats must be a contiguous int64 [{NSTATS}]")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise DQError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (B, Hq, HEAD_DIM) or not out.is_contiguous():
        raise DQError("out has the wrong shape or dtype")
    need = attn_workspace_bytes(B, Hq, ck.kv_heads, max_len)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if sm_scale is None:
        sm_scale = HEAD_DIM ** -0.5
    head = (ck.handle, cv.handle, _ptr(q), B, Hq, _ptr(k_new), _ptr(v_new), k_new.stride(0),
            k_new.stride(1), _ptr(k_cont), _ptr(k_norm), _ptr(v_cont), _ptr(v_norm), k_cont.shape[1])
    where = (_ptr(loc), loc.shape[1]) if paged else (_ptr(loc),)
    tail = (_ptr(seq_len), max_len, ctypes.c_float(sm_scale), 0 if out_dtype == torch.float32 else 1,
            _ptr(out), _ptr(workspace), workspace.numel(), _ptr(k_stats), _ptr(v_stats), _stream(q.device))
    if split_events is not None and not paged:
        _check(_lib.lib().dq_attn_decode_append_timed(*head, *where, *tail, *_event_handles(split_events)),
               "dq_attn_decode_append_timed")
        return out
    fn = "dq_attn_decode_paged_append" if paged else "dq_attn_decode_append"
    _check(getattr(_lib.lib(), fn)(*head, *where, *tail), fn)
    return out


def attn_decode_append(ck: Codec, cv: Codec, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                       k_cont, k_norm, v_cont, v_norm, seq_start: torch.Tensor, seq_len: torch.Tensor,
                       max_len: int, sm_scale: float | None = None, out: torch.Tensor | None = None,
                       out_dtype=torch.float32, workspace: torch.Tensor | None = None,
                       k_stats: torch.Tensor | None = None, v_stats: torch.Tensor | None = None,
                       split_events=None):
    """A decode step with append in one call: k_new, v_new bf16 [B, Hkv, 128]
    are encoded into slot seq_start[b] + seq_len[b] - 1 (seq_len counts the
    new token) and attended to with the rest of the cache.  Returns out
    [B, Hq, 128]; the pools are updated in place.

    split_events: optional (begin, end) torch.cuda.Event pair, recorded on
    the current stream around the split-K kernel (which runs the encodes)."""
    return _attn_decode_append(ck, cv, q, k_new, v_new, k_cont, k_norm, v_cont, v_norm, seq_start, seq_len,
                               max_len, sm_scale, out, out_dtype, workspace, k_stats, v_stats, paged=False,
                               split_events=split_events)


def attn_decode_paged_append(ck: Codec, cv: Codec, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                             k_cont, k_norm, v_cont, v_norm, pages: torch.Tensor, seq_len: torch.Tensor,
                             max_len: int, sm_scale: float | None = None, out: torch.Tensor | None = None,
                             out_dtype=torch.float32, workspace: torch.Tensor | None = None,
                             k_stats: torch.Tensor | None = None, v_stats: torch.Tensor | None = None):
    """attn_decode_append over a paged pool (pages int32 [B, max_pages])."""
    return _attn_decode_append(ck, cv, q, k_new, v_new, k_cont, k_norm, v_cont, v_norm, pages, seq_len,
                               max_len, sm_scale, out, out_dtype, workspace, k_stats, v_stats, paged=True)


def attn_prefill_workspace_bytes(B: int, Tq: int, Hq: int, Hkv: int, max_len: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.lib().dq_attn_prefill_workspace(B, Tq, Hq, Hkv, max_len, ctypes.byref(n)),
           "dq_attn_prefill_workspace")
    return n.value


def attn_prefill(ck: Codec, cv: Codec, q: torch.Tensor, k_cont, k_norm, v_cont, v_norm,
                 seq_start: torch.Tensor, seq_len: torch.Tensor, max_len: int,
                 sm_scale: float | None = None, out: torch.Tensor | None = None,
                 out_dtype=torch.float32, workspace: torch.Tensor | None = None):
    """Causal chunked-prefill attention: q bf16 [B, Tq, Hq, 128]; the last Tq
    cached tokens of each sequence are the queries.  Returns [B, Tq, Hq, 128]."""
    _need_cuda("q", q, torch.bfloat16)
    for name, t, dt in (("k_cont", k_cont, torch.uint8), ("v_cont", v_cont, torch.uint8),
                        ("k_norm", k_norm, torch.float16), ("v_norm", v_norm, torch.float16),
                        ("seq_start", seq_start, torch.int64), ("seq_len", seq_len, torch.int32)):
        _need_cuda(name, t, dt)
        if not t.is_contiguous():
            raise DQError(f"{name} must be contiguous")
    if q.dim() != 4 or q.shape[3] != HEAD_DIM or not q.is_contiguous():
        raise DQError("q must be a contiguous bf16 [B, Tq, Hq, 128]")
    B, Tq, Hq, _ = q.shape
    if k_cont.shape[1] != v_cont.shape[1]:
        raise DQError("K and V pools must have the same slot count")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise DQError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((B, Tq, Hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (B, Tq, Hq, HEAD_DIM) or not out.is_contiguous():
        raise DQError("out has the wrong shape or dtype")
    need = attn_prefill_workspace_bytes(B, Tq, Hq, ck.kv_heads, max_len)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if sm_scale is None:
        sm_scale = HEAD_DIM ** -0.5
    _check(_lib.lib().dq_attn_prefill(
        ck.handle, cv.handle, _ptr(q), B, Tq, Hq, _ptr(k_cont), _ptr(k_norm), _ptr(v_cont),
        _ptr(v_norm), k_cont.shape[1], _ptr(seq_start), _ptr(seq_len), max_len,
        ctypes.c_float(sm_scale), 0 if out_dtype == torch.float32 else 1, _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(q.device)), "dq_attn_prefill")
    return out
