"""dq_attn_decode_noalloc: decode attention with the library's own device
array as the workspace, for callers that cannot allocate.  Through the C ABI
(ctypes), against dq_attn_decode on the same inputs (same kernels, so the
same bytes), on two calls in a row, the second smaller, each with fresh
data; plus the oracle on the first call and the size rejection."""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_entropy_amd as dq
import synth
from kv_cache_entropy_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(B, Hq, hkv, lens, seed, C=(34, 34)):
    ck = dq.Codec(8, C[0], seed=seed, kv_heads=hkv)
    cv = dq.Codec(6, C[1], seed=seed + 1, kv_heads=hkv)
    lens = np.asarray(lens, np.int64)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    T = int(lens.sum())
    K = synth.kv_tensor("outlier", T, hkv, seed=seed + 2, device=DEV)
    V = synth.kv_tensor("student_t5", T, hkv, seed=seed + 3, device=DEV)
    slots = torch.arange(T, dtype=torch.int64, device=DEV)
    kc, kn = dq.alloc_pool(ck, T, DEV)
    vc, vn = dq.alloc_pool(cv, T, DEV)
    dq.encode(ck, K, slots, kc, kn)
    dq.encode(cv, V, slots, vc, vn)
    q = synth.q_tensor(B, Hq, seed=seed + 4, device=DEV)
    ss = torch.from_numpy(starts).to(DEV)
    sl = torch.from_numpy(lens.astype(np.int32)).to(DEV)
    return dict(ck=ck, cv=cv, q=q, kc=kc, kn=kn, vc=vc, vn=vn, ss=ss, sl=sl, max_len=int(lens.max()),
                starts=starts, lens=lens, K=K, V=V)


def _noalloc(c, out):
    B, Hq, _ = c["q"].shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return _lib.lib().dq_attn_decode_noalloc(
        c["ck"].handle, c["cv"].handle, p(c["q"]), B, Hq, p(c["kc"]), p(c["kn"]), p(c["vc"]), p(c["vn"]),
        c["kc"].shape[1], p(c["ss"]), p(c["sl"]), c["max_len"], ctypes.c_float(128 ** -0.5), 0, p(out),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_workspace_call_twice(oracle_lib):
    O = oracle_lib
    first = _case(4, 32, 8, [3000, 1, 2049, 777], seed=301)
    second = _case(2, 8, 2, [500, 65], seed=302, C=(29, 34))
    for i, c in enumerate((first, second)):
        print(f"no-alloc call {i}: B={c['q'].shape[0]} lens={c['lens'].tolist()}", flush=True)
        got = torch.full(c["q"].shape, float("nan"), dtype=torch.float32, device=DEV)
        assert _noalloc(c, got) == 0
        ref = dq.attn_decode(c["ck"], c["cv"], c["q"], c["kc"], c["kn"], c["vc"], c["vn"], c["ss"], c["sl"],
                             c["max_len"])
        torch.cuda.synchronize()
        assert torch.equal(got, ref), float((got - ref).abs().max())
        if i == 0:
            ock = O.Codec(8, 34, seed=301, hkv=8)
            ocv = O.Codec(6, 34, seed=302, hkv=8)
            S = c["kc"].shape[1]
            okc, okn, _ = O.encode(ock, synth.bf16_bits(c["K"]), num_slots=S)
            ovc, ovn, _ = O.encode(ocv, synth.bf16_bits(c["V"]), num_slots=S)
            want = O.attention(ock, ocv, synth.bf16_bits(c["q"]), okc, okn, ovc, ovn, c["starts"],
                               c["lens"].astype(np.int32))
            g = got.double().cpu().numpy()
            err = float(np.abs(g - want).max())
            rel = float(np.linalg.norm(g - want) / np.linalg.norm(want))
            assert err <= 2e-3 and rel <= 1e-3, (err, rel)


def test_noalloc_rejects_oversized_workspace():
    """A shape whose workspace would exceed the library's array returns
    DQ_ERR_WORKSPACE before anything is launched, and the next call that
    fits still works."""
    c = _case(2, 8, 2, [300, 200], seed=303)
    B, Hq, _ = c["q"].shape
    need = dq.attn_workspace_bytes(B, Hq, 2, 1 << 30)
    assert need > (64 << 20)
    big = dict(c, max_len=1 << 30)
    out = torch.zeros(c["q"].shape, dtype=torch.float32, device=DEV)
    assert _noalloc(big, out) == -4
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    assert _noalloc(c, out) == 0
    ref = dq.attn_decode(c["ck"], c["cv"], c["q"], c["kc"], c["kn"], c["vc"], c["vn"], c["ss"], c["sl"],
                         c["max_len"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
