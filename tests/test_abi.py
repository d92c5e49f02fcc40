"""Host-side checks of the C ABI library (no GPU needed).

* libdq.so loads and exports every function include/dq.h declares;
* codec creation is host-only and its exported tables equal the oracle's bit
  for bit (frequencies, cumulative counts, fp16 reconstruction levels,
  rotation sign words) for the default codecs and a sweep of others;
* invalid descriptors return the documented codes and launch nothing.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_entropy_amd as dq
from kv_cache_entropy_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(_lib.LIB):
        from kv_cache_entropy_amd import build
        build.build()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dq_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "dq_encode" in names and "dq_attn_decode" in names and len(names) >= 10
    L = ctypes.CDLL(_lib.LIB)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = _lib.lib()
    assert L.dq_version() == 105
    assert L.dq_status_string(0) == b"ok"
    for code in (-1, -2, -3, -4, -5):
        assert L.dq_status_string(code) not in (b"ok", b"unknown status")


def test_knobs_set_get_and_reject():
    """dq_set_knob stores a forced path per knob (host only, no GPU), -1
    restores the default, and unknown knobs or values below -1 are rejected."""
    for name in dq.KNOBS:
        assert dq.get_knob(name) == -1
    with dq.knobs(split_tokens=128, latency_mode=1):
        assert dq.get_knob("split_tokens") == 128 and dq.get_knob("latency_mode") == 1
    assert dq.get_knob("split_tokens") == -1 and dq.get_knob("latency_mode") == -1
    L = _lib.lib()
    assert L.dq_set_knob(0, 1) == -1 and L.dq_set_knob(99, 1) == -1 and L.dq_set_knob(1, -2) == -1
    assert L.dq_get_knob(0) == -1


@pytest.mark.parametrize("levels,C,step64", [
    (8, 34, 0), (6, 34, 0), (8, 29, 0), (6, 29, 0),
    (8, 34, 60), (8, 34, 80), (6, 29, 70), (4, 24, 64), (2, 20, 64),
    (10, 40, 64), (12, 48, 60), (16, 60, 25), (16, 60, 50), (6, 132, 30), (8, 64, 40)])
def test_tables_match_oracle(oracle_lib, levels, C, step64):
    O = oracle_lib
    seed = 0xDEADBEEF12345 + levels
    try:
        codec = dq.Codec(levels, C, seed=seed, kv_heads=5, step64=step64)
    except dq.DQError:
        assert O.codec_check(levels, step64 or O.DEFAULT_STEP64.get((levels, C), 0), C) != 0
        return
    oc = O.Codec(levels, C, seed=seed, hkv=5, step64=codec.step64)
    ot = oc.tables()
    t = codec.tables()
    assert (t["freq"].astype(np.uint32) == ot["freq"]).all()
    assert (t["cum"].astype(np.uint32) == ot["cum"]).all()
    assert (t["recon_f16"] == ot["recon_f16"]).all()
    assert (t["sign_words"] == oc.sign_words()).all()


def test_defaults_match_oracle(oracle_lib):
    for (levels, C), step in oracle_lib.DEFAULT_STEP64.items():
        assert dq.Codec(levels, C, seed=1, kv_heads=1).step64 == step


def test_codec_acceptance_matches_oracle(oracle_lib):
    O = oracle_lib
    for levels in (2, 4, 6, 8, 10, 16):
        for C in (8, 20, 29, 34, 48):
            for step64 in (20, 40, 64, 73, 83, 84, 100, 160):
                want = O.codec_check(levels, step64, C)
                L = _lib.lib()
                desc = _lib.CodecDesc(128, levels, C, 1, 0, step64, 0)
                h = ctypes.c_void_p()
                got = L.dq_codec_create(ctypes.byref(desc), ctypes.byref(h))
                if got == 0:
                    L.dq_codec_destroy(h)
                assert got == want, (levels, C, step64)


def test_invalid_descriptors():
    L = _lib.lib()
    h = ctypes.c_void_p()
    bad = [
        (_lib.CodecDesc(64, 8, 34, 1, 0, 0, 0), -2),     # head_dim
        (_lib.CodecDesc(128, 7, 34, 1, 0, 0, 0), -1),    # odd levels
        (_lib.CodecDesc(128, 18, 34, 1, 0, 0, 0), -1),   # too many levels
        (_lib.CodecDesc(128, 8, 4, 1, 0, 73, 0), -1),    # container too small
        (_lib.CodecDesc(128, 8, 133, 1, 0, 73, 0), -1),  # container too large
        (_lib.CodecDesc(128, 8, 34, 0, 0, 0, 0), -1),    # no kv heads
        (_lib.CodecDesc(128, 8, 34, 1, 0, 0, 7), -1),    # drift order not 0 or 1
        (_lib.CodecDesc(128, 8, 40, 1, 0, 0, 0), -1),    # no default width
        (_lib.CodecDesc(128, 8, 34, 1, 0, 2000, 0), -1),  # width out of range
        (_lib.CodecDesc(128, 8, 29, 1, 0, 84, 0), -3),   # outer cells too close
    ]
    for desc, code in bad:
        assert L.dq_codec_create(ctypes.byref(desc), ctypes.byref(h)) == code
    assert L.dq_codec_create(None, ctypes.byref(h)) == -1
    assert L.dq_codec_destroy(None) == 0


def test_host_argument_checks_launch_nothing():
    """Argument errors are reported before any HIP call, so they are
    testable without a GPU."""
    L = _lib.lib()
    c = dq.Codec(8, 34, seed=1, kv_heads=2)
    vp = ctypes.c_void_p
    fake = vp(256)  # never dereferenced: every call below fails validation
    # null codec / negative sizes
    assert L.dq_encode(None, fake, 1, 256, 128, fake, 16, fake, fake, None, None) == -1
    assert L.dq_encode(c.handle, fake, -1, 256, 128, fake, 16, fake, fake, None, None) == -1
    assert L.dq_encode(c.handle, fake, 0, 256, 128, fake, 16, fake, fake, None, None) == 0
    # misaligned x / strides
    assert L.dq_encode(c.handle, vp(258), 1, 256, 128, fake, 16, fake, fake, None, None) == -1
    assert L.dq_encode(c.handle, fake, 1, 255, 128, fake, 16, fake, fake, None, None) == -1
    # decode: bad head
    assert L.dq_decode_symbols(c.handle, fake, 16, 2, fake, 1, fake, None, None, None) == -1
    assert L.dq_decode_symbols(c.handle, fake, 16, 0, fake, 0, fake, None, None, None) == 0
    # attention: mismatched heads, bad group, misalignment
    v3 = dq.Codec(6, 34, seed=2, kv_heads=3)
    v2 = dq.Codec(6, 34, seed=2, kv_heads=2)
    args = [fake, 1, 4, fake, fake, fake, fake, 16, fake, fake, 64, ctypes.c_float(0.1), 0,
            fake, fake, 1 << 20, None]
    assert L.dq_attn_decode(c.handle, v3.handle, *args) == -1
    bad_group = list(args)
    bad_group[2] = 16  # Hq / Hkv = 8
    assert L.dq_attn_decode(c.handle, v2.handle, *bad_group) == -2
    misaligned = list(args)
    misaligned[3] = vp(264)  # k_cont not 16-byte aligned
    assert L.dq_attn_decode(c.handle, v2.handle, *misaligned) == -1
    bad_pool = list(args)
    bad_pool[7] = 15  # 15 * 34 not a multiple of 16
    assert L.dq_attn_decode(c.handle, v2.handle, *bad_pool) == -1


def test_paged_attention_argument_checks():
    L = _lib.lib()
    c = dq.Codec(8, 34, seed=1, kv_heads=2)
    v = dq.Codec(6, 34, seed=2, kv_heads=2)
    vp = ctypes.c_void_p
    fake = vp(256)
    base = [c.handle, v.handle, fake, 1, 4, fake, fake, fake, fake, 64, fake, 2, fake, 128,
            ctypes.c_float(0.1), 0, fake, fake, 1 << 20, None]
    nopages = list(base)
    nopages[10] = None
    assert L.dq_attn_decode_paged(*nopages) == -1
    zero = list(base)
    zero[11] = 0  # max_pages
    assert L.dq_attn_decode_paged(*zero) == -1
    short = list(base)
    short[13] = 129  # max_len > max_pages * 64
    assert L.dq_attn_decode_paged(*short) == -1


def test_append_argument_checks():
    """The decode-with-append entry points reject missing or misaligned new
    tokens and a missing page table before touching the device."""
    L = _lib.lib()
    c = dq.Codec(8, 34, seed=1, kv_heads=2)
    v = dq.Codec(6, 34, seed=2, kv_heads=2)
    vp = ctypes.c_void_p
    fake = vp(256)
    # ck cv q B Hq k_new v_new stride_b stride_h kc kn vc vn S seq_start seq_len max_len
    # sm_scale out_dtype out ws ws_bytes k_stats v_stats stream
    base = [c.handle, v.handle, fake, 1, 4, fake, fake, 256, 128, fake, fake, fake, fake, 64, fake, fake, 128,
            ctypes.c_float(0.1), 0, fake, fake, 1 << 20, None, None, None]
    for idx in (5, 6):
        bad = list(base)
        bad[idx] = None
        assert L.dq_attn_decode_append(*bad) == -1
        bad[idx] = vp(257)  # bf16 needs 2-byte alignment
        assert L.dq_attn_decode_append(*bad) == -1
    paged = base[:14] + [fake, 2] + base[15:]
    nopages = list(paged)
    nopages[14] = None
    assert L.dq_attn_decode_paged_append(*nopages) == -1
    short = list(paged)
    short[17] = 129  # max_len > max_pages * 64
    assert L.dq_attn_decode_paged_append(*short) == -1


def test_drift_order_codec():
    c = dq.Codec(6, 34, seed=1, kv_heads=2, drift_order=1)
    assert c.drift_order == 1
    assert dq.Codec(6, 34, seed=1, kv_heads=2).drift_order == 0
    with pytest.raises(dq.DQError):
        dq.Codec(6, 34, seed=1, kv_heads=2, drift_order=2)
