"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Containers, norms, decoded symbols and drift statistics must be bit-exact;
attention output (fp32) must be within max-abs 2e-3 and relative-L2 1e-3 of
the oracle's fp64 result on the same containers.  Inputs come from the seeded
generator in synth/ (drawn on the GPU, copied to the host for the oracle).
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_entropy_amd as dq
import synth

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2 = 2e-3, 1e-3
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _np_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _codecs(O, levels, C, seed, hkv, step64=0, order=0):
    g = dq.Codec(levels, C, seed=seed, kv_heads=hkv, step64=step64, drift_order=order)
    o = O.Codec(levels, C, seed=seed, hkv=hkv, step64=g.step64, order=order)
    return g, o


@pytest.fixture(params=["wave", "lane", "lane_one_pass"])
def encode_path(request, knob):
    """Small batches run the wave-per-vector kernel, large ones the
    lane-per-vector kernels (two passes by default: no-drift vectors first,
    then the drift search on the rest; or the search inline in one pass);
    force each in turn on the same inputs."""
    knob("encode_wave_max", "1000000000" if request.param == "wave" else "0")
    knob("encode_two_pass", "0" if request.param == "lane_one_pass" else "-1")
    return request.param


def _encode_both(O, gc, oc, x, slots, num_slots):
    cont, norm = dq.alloc_pool(gc, num_slots, DEV)
    st = dq.new_stats(DEV)
    dq.encode(gc, x, slots, cont, norm, st)
    torch.cuda.synchronize()
    S = cont.shape[1]
    ocont, onorm, ost = O.encode(oc, _np_bits(x), slots.cpu().numpy(), num_slots=S)
    return cont, norm, st, ocont, onorm, ost


def _assert_encode_equal(cont, norm, st, ocont, onorm, ost, label):
    gcont = cont.cpu().numpy()
    gnorm = _np_bits(norm)
    bad = np.argwhere((gcont != ocont).any(axis=2))
    assert len(bad) == 0, f"{label}: {len(bad)} containers differ, first {bad[:5].tolist()}"
    assert (gnorm == onorm).all(), f"{label}: norms differ"
    assert dq.stats_dict(st) == O_stats(ost), f"{label}: stats differ"


def O_stats(ost):
    import oracle
    return oracle.stats_dict(ost)


@pytest.mark.parametrize("levels,C", [(8, 34), (6, 34), (8, 29), (6, 29)])
@pytest.mark.parametrize("kind", ["iid", "outlier", "student_t5", "iid_scaled"])
def test_encode_bit_exact(oracle_lib, encode_path, levels, C, kind):
    O = oracle_lib
    _say(f"encode {levels}/{C} {kind} {encode_path}")
    T, hkv = 333, 3
    gc, oc = _codecs(O, levels, C, seed=101 + levels, hkv=hkv)
    x = synth.kv_tensor(kind, T, hkv, seed=7, device=DEV)
    perm = torch.randperm(400, generator=torch.Generator().manual_seed(3))[:T]
    slots = perm.to(DEV)
    _assert_encode_equal(*_encode_both(O, gc, oc, x, slots, 400), f"{levels}/{C}/{kind}")


def _adversarial_batch():
    rows = []
    z = np.zeros(128, np.float32)
    rows.append(z.copy())                                  # zero vector
    rows.append(np.full(128, 1e-30, np.float32))            # norm underflows fp16
    rows.append(np.full(128, 1e30, np.float32))             # squares overflow fp32
    r = z.copy(); r[5] = np.inf; rows.append(r)              # inf
    r = np.ones(128, np.float32); r[7] = np.nan; rows.append(r)  # nan
    r = z.copy(); r[0] = 3.3895314e38; rows.append(r)        # largest bf16
    r = z.copy(); r[:3] = [9.2e-41, -4.6e-41, 1e-39]; rows.append(r)  # bf16 subnormals
    r = z.copy(); r[:3] = [2048, 64, 1]; rows.append(r)      # |x| = 2049: fp16 tie -> 2048
    r = z.copy(); r[:4] = [2048, 64, 1, 1]; rows.append(r)   # just above the tie -> 2050
    r = z.copy(); r[:3] = [1.0, 2.0 ** -5, 2.0 ** -11]; rows.append(r)  # tie at 1 + 2^-11
    r = z.copy(); r[0] = -0.0; r[1] = 1.0; rows.append(r)    # negative zero
    r = z.copy(); r[3] = 1.0; rows.append(r)                 # one-hot: |y_i| all equal
    rows.append(np.where(np.arange(128) % 2 == 0, 1.0, -1.0).astype(np.float32))
    rows.append((np.arange(128) - 64).astype(np.float32))   # exact integer sums
    rows.append(np.full(128, 65504.0 / 11.3, np.float32))    # norm near fp16 max
    rng = np.random.default_rng(0)
    for _ in range(17):
        v = rng.standard_normal(128).astype(np.float32)
        v[rng.integers(0, 128, 6)] *= 10 ** rng.uniform(-3, 3)
        rows.append(v)
    return np.stack(rows)


@pytest.mark.parametrize("levels,C,step64", [(8, 34, 0), (6, 34, 0), (8, 29, 0), (6, 29, 0),
                                             (8, 34, 64), (6, 34, 64), (4, 30, 64), (16, 60, 25), (10, 40, 34)])
def test_encode_adversarial(oracle_lib, encode_path, levels, C, step64):
    """Degenerate norms, fp16 rounding ties, exact threshold ties (step 1.0
    and one-hot inputs put |y| exactly on a threshold), subnormals."""
    O = oracle_lib
    _say(f"adversarial {levels}/{C}/{step64} {encode_path}")
    rows = _adversarial_batch()
    x = torch.from_numpy(rows).to(torch.bfloat16).reshape(-1, 1, 128).to(DEV)
    gc, oc = _codecs(O, levels, C, seed=5, hkv=1, step64=step64)
    slots = torch.arange(x.shape[0], dtype=torch.int64, device=DEV)
    _assert_encode_equal(*_encode_both(O, gc, oc, x, slots, x.shape[0]), "adversarial")


@pytest.mark.parametrize("span", [0, 1 << 21])
@pytest.mark.parametrize("levels,C,step64", [(8, 34, 0), (6, 34, 0), (6, 29, 0), (16, 60, 25), (4, 30, 64)])
def test_encode_in_group_scan_fallback(oracle_lib, knob, span, levels, C, step64):
    """The lane encoder ranks a drift group's members by integer keys and
    falls back to float scans for members past the keys' span.  Narrowed
    spans force the fallback (span 0: from the first member on; 2^21: for
    |y| above 2^(1/4) times the group's threshold, so it also starts
    mid-way); the bytes must stay the oracle's."""
    knob("encode_wave_max", "0")
    knob("encode_key_span", str(span))
    O = oracle_lib
    _say(f"in-group fallback span {span} {levels}/{C}/{step64}")
    gc, oc = _codecs(O, levels, C, seed=41 + levels, hkv=2, step64=step64)
    for kind in ("outlier", "student_t5"):
        x = synth.kv_tensor(kind, 600, 2, seed=43, device=DEV)
        slots = torch.arange(600, dtype=torch.int64, device=DEV)
        _assert_encode_equal(*_encode_both(O, gc, oc, x, slots, 600), f"span {span} {levels}/{C}/{kind}")
    rows = _adversarial_batch()
    x = torch.from_numpy(rows).to(torch.bfloat16).reshape(-1, 1, 128).to(DEV)
    ga, oa = _codecs(O, levels, C, seed=5, hkv=1, step64=step64)
    slots = torch.arange(x.shape[0], dtype=torch.int64, device=DEV)
    _assert_encode_equal(*_encode_both(O, ga, oa, x, slots, x.shape[0]), f"span {span} adversarial")


@pytest.mark.parametrize("levels,C,step64", [(8, 34, 0), (6, 34, 0), (8, 29, 0), (6, 29, 0),
                                             (4, 30, 64), (10, 40, 34)])
def test_encode_rate_distortion_order(oracle_lib, encode_path, levels, C, step64):
    """Rate-distortion drift order: containers, norms and stats bit-exact on
    the four distributions and on the adversarial rows (ties, degenerate
    norms, one-hot vectors), through both encode kernels."""
    O = oracle_lib
    _say(f"rd order {levels}/{C}/{step64} {encode_path}")
    gc, oc = _codecs(O, levels, C, seed=33 + levels, hkv=3, step64=step64, order=1)
    for kind in ("iid", "outlier", "student_t5", "iid_scaled"):
        x = synth.kv_tensor(kind, 200, 3, seed=71, device=DEV)
        slots = torch.arange(200, dtype=torch.int64, device=DEV)
        _assert_encode_equal(*_encode_both(O, gc, oc, x, slots, 200), f"rd {levels}/{C} {kind}")
    rows = _adversarial_batch()
    x = torch.from_numpy(rows).to(torch.bfloat16).reshape(-1, 1, 128).to(DEV)
    gc1, oc1 = _codecs(O, levels, C, seed=5, hkv=1, step64=step64, order=1)
    slots = torch.arange(x.shape[0], dtype=torch.int64, device=DEV)
    _assert_encode_equal(*_encode_both(O, gc1, oc1, x, slots, x.shape[0]), f"rd adversarial {levels}/{C}")


def test_encode_strided_input_and_pool_slots(oracle_lib, encode_path):
    O = oracle_lib
    gc, oc = _codecs(O, 8, 34, seed=9, hkv=4)
    big = synth.kv_tensor("outlier", 200, 8, seed=11, device=DEV)
    x = big[:, 1::2]  # stride_h = 256 elements
    assert x.stride(1) == 256
    slots = torch.arange(1000, 1200, dtype=torch.int64, device=DEV)
    cont, norm, st, ocont, onorm, ost = _encode_both(O, gc, oc, x, slots, 1300)
    _assert_encode_equal(cont, norm, st, ocont, onorm, ost, "strided")
    # untouched slots stay zero
    assert int(cont[:, :1000].abs().sum()) == 0


@pytest.mark.parametrize("levels,C,order,T,hkv", [(8, 34, 0, 3072, 4), (6, 29, 0, 3072, 4), (6, 29, 1, 3072, 4),
                                                  (8, 29, 1, 3072, 4), (6, 34, 0, 9000, 2)])
def test_encode_two_pass_many_blocks(oracle_lib, knob, levels, C, order, T, hkv):
    """The two-pass lane encoder over several 8192-vector ranges of its
    second pass (12288 or 18000 vectors, heavy-tailed data so that many need
    the drift search; heads shorter than a range, and longer, so that a
    range starts inside a head and spans two): bytes, norms and stats equal
    to the one-pass kernel's and to the oracle's."""
    O = oracle_lib
    _say(f"two-pass {levels}/{C} order {order} T {T} hkv {hkv}")
    gc, oc = _codecs(O, levels, C, seed=211 + levels, hkv=hkv, order=order)
    x = synth.kv_tensor("student_t5", T, hkv, seed=212, device=DEV)
    slots = torch.randperm(T + 100, generator=torch.Generator().manual_seed(213))[:T].to(DEV)
    knob("encode_wave_max", "0")
    out = {}
    for two in ("1", "0"):
        knob("encode_two_pass", two)
        cont, norm = dq.alloc_pool(gc, T + 100, DEV)
        st = dq.new_stats(DEV)
        dq.encode(gc, x, slots, cont, norm, st)
        torch.cuda.synchronize()
        out[two] = (cont, norm, st)
    assert torch.equal(out["1"][0], out["0"][0]) and torch.equal(out["1"][1], out["0"][1])
    assert dq.stats_dict(out["1"][2]) == dq.stats_dict(out["0"][2])
    assert dq.stats_dict(out["1"][2])["drifted_vectors"] > 0
    ocont, onorm, ost = O.encode(oc, _np_bits(x), slots.cpu().numpy(), num_slots=out["1"][0].shape[1])
    _assert_encode_equal(*out["1"], ocont, onorm, ost, f"two-pass {levels}/{C}")


def test_encode_slots_outside_pool(oracle_lib, encode_path):
    """A vector whose slot is outside the pool (negative or past its end)
    writes nothing; with stats it is still counted, as if it had a slot.
    The in-pool vectors' containers and norms are those of a call without
    the others."""
    O = oracle_lib
    T, hkv = 400, 2
    gc, oc = _codecs(O, 6, 29, seed=15, hkv=hkv)
    x = synth.kv_tensor("student_t5", T, hkv, seed=16, device=DEV)
    cont, norm = dq.alloc_pool(gc, 500, DEV)
    S = cont.shape[1]  # the pool as allocated (rounded up)
    slots = torch.arange(T, dtype=torch.int64) + 50
    slots[::7] = -1
    slots[3::11] = S + 3
    inside = (slots >= 0) & (slots < S)
    st = dq.new_stats(DEV)
    dq.encode(gc, x, slots.to(DEV), cont, norm, st)
    torch.cuda.synchronize()
    # stats: every vector, as encoded into a pool where each has a slot
    full_slots = torch.arange(T, dtype=torch.int64, device=DEV)
    c2, n2 = dq.alloc_pool(gc, T, DEV)
    st2 = dq.new_stats(DEV)
    dq.encode(gc, x, full_slots, c2, n2, st2)
    torch.cuda.synchronize()
    assert dq.stats_dict(st) == dq.stats_dict(st2)
    idx = torch.nonzero(inside).flatten()
    ocont, onorm, ost = O.encode(oc, _np_bits(x[idx.to(DEV)]), slots[idx].numpy(), num_slots=S)
    gcont, gnorm = cont.cpu().numpy(), _np_bits(norm)
    assert (gcont == ocont).all() and (gnorm == onorm).all()


@pytest.mark.parametrize("levels,C", [(8, 34), (6, 29)])
def test_decode_symbols_bit_exact(oracle_lib, levels, C):
    O = oracle_lib
    gc, oc = _codecs(O, levels, C, seed=21, hkv=2)
    x = synth.kv_tensor("outlier", 500, 2, seed=4)
    ocont, _, _ = O.encode(oc, _np_bits(x))
    S = dq.pool_slots(500, C)
    pool = np.zeros((2, S, C), np.uint8)
    pool[:, :500] = ocont
    # corrupted containers: random bytes in slots 500..S-1 and a few overwritten
    rng = np.random.default_rng(1)
    pool[:, 500:] = rng.integers(0, 256, (2, S - 500, C))
    pool[:, 3] = rng.integers(0, 256, (2, C))
    gpool = torch.from_numpy(pool).to(DEV)
    for head in range(2):
        slots = np.arange(S)
        sym, fs, cons = dq.decode_symbols(gc, gpool, head, torch.from_numpy(slots).to(DEV))
        osym, ofs, ocons = O.decode_symbols(oc, pool, head, slots)
        assert (sym.cpu().numpy() == osym).all()
        assert (fs.cpu().numpy() == ofs).all()
        assert (cons.cpu().numpy() == ocons).all()
        valid = [s for s in range(500) if s != 3]
        assert (ofs[valid] == 1 << 23).all()


def _attn_case(O, B, Hq, hkv, lens, kinds=("outlier", "outlier"), C=(34, 34), seed=0, gap=5,
               levels=(8, 6), step64=(0, 0), order=(0, 0)):
    ck, ock = _codecs(O, levels[0], C[0], seed=seed + 1, hkv=hkv, step64=step64[0], order=order[0])
    cv, ocv = _codecs(O, levels[1], C[1], seed=seed + 2, hkv=hkv, step64=step64[1], order=order[1])
    starts, s = [], 0
    for L in lens:
        starts.append(s)
        s += L + gap
    total = s
    K = synth.kv_tensor(kinds[0], total, hkv, seed=seed + 3, device=DEV)
    V = synth.kv_tensor(kinds[1], total, hkv, seed=seed + 4, device=DEV)
    q = synth.q_tensor(B, Hq, seed=seed + 5, device=DEV)
    slots = torch.arange(total, dtype=torch.int64, device=DEV)
    kc, kn = dq.alloc_pool(ck, total, DEV)
    vc, vn = dq.alloc_pool(cv, total, DEV)
    dq.encode(ck, K, slots, kc, kn)
    dq.encode(cv, V, slots, vc, vn)
    ss = torch.tensor(starts, dtype=torch.int64, device=DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return dict(ck=ck, cv=cv, ock=ock, ocv=ocv, q=q, kc=kc, kn=kn, vc=vc, vn=vn, ss=ss, sl=sl,
                starts=np.array(starts), lens=np.array(lens, np.int32))


def _oracle_attn(O, c, rows=None, sm_scale=None):
    idx = np.arange(len(c["lens"])) if rows is None else np.asarray(rows)
    return O.attention(c["ock"], c["ocv"], _np_bits(c["q"])[idx], c["kc"].cpu().numpy(),
                       _np_bits(c["kn"]), c["vc"].cpu().numpy(), _np_bits(c["vn"]),
                       c["starts"][idx], c["lens"][idx], sm_scale=sm_scale)


def _gpu_attn(c, max_len=None, **kw):
    out = dq.attn_decode(c["ck"], c["cv"], c["q"], c["kc"], c["kn"], c["vc"], c["vn"], c["ss"],
                         c["sl"], int(max_len or c["lens"].max()), **kw)
    torch.cuda.synchronize()
    return out


def _assert_close(got, ref, label):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    worst = np.unravel_index(np.argmax(err), err.shape)
    emax = float(err.max())
    _say(f"{label}: max-abs {emax:.3e} rel-L2 {rel:.3e} worst {tuple(int(i) for i in worst)}")
    assert emax <= MAX_ABS and rel <= REL_L2, (label, emax, rel)


@pytest.mark.parametrize("Hq,hkv", [(8, 2), (4, 4), (4, 2), (1, 1)])
def test_attention_ragged_small(oracle_lib, Hq, hkv):
    O = oracle_lib
    lens = [1, 63, 64, 65, 300, 129]
    c = _attn_case(O, len(lens), Hq, hkv, lens, seed=Hq * 10 + hkv)
    _assert_close(_gpu_attn(c).cpu().numpy(), _oracle_attn(O, c), f"ragged Hq={Hq} hkv={hkv}")


def test_attention_many_partials(oracle_lib, knob):
    """A 17000-token sequence in 64-token chunks: 266 partials, so the merge
    takes the two rounds whose (m, l) it holds in registers and a third it
    reads back; a short sequence beside it.  Against the oracle."""
    O = oracle_lib
    knob("split_tokens", "64")
    lens = [17000, 300]
    c = _attn_case(O, 2, 8, 2, lens, seed=13)
    _assert_close(_gpu_attn(c).cpu().numpy(), _oracle_attn(O, c), "266 partials")


def test_attention_split_invariance_and_bf16(oracle_lib, knob):
    """Chunk sizes 64..1024 change only the fp32 order of the sums (P and
    the query are fp16 hi/lo pairs, ~22 bits each), so outputs of different
    splits agree to 1e-4 absolute, well inside the oracle tolerance."""
    O = oracle_lib
    lens = [2000, 777, 1500]
    c = _attn_case(O, 3, 8, 2, lens, kinds=("iid_scaled", "student_t5"), C=(34, 29), seed=3)
    ref = _oracle_attn(O, c, sm_scale=0.11)
    outs = []
    for split in (64, 256, 1024, None):
        knob("split_tokens", split)
        o = _gpu_attn(c, sm_scale=0.11).cpu().numpy()
        _assert_close(o, ref, f"split={split or 'default'}")
        outs.append(o)
    for o in outs[1:]:
        spread = float(np.abs(o - outs[0]).max())
        _say(f"split spread {spread:.3e}")
        assert spread < 1e-4, spread
    ob = _gpu_attn(c, sm_scale=0.11, out_dtype=torch.bfloat16).float().cpu().numpy()
    bf_err = float(np.abs(ob - outs[-1]).max())
    assert bf_err <= float(np.abs(outs[-1]).max()) * 2 ** -8, bf_err


def test_attention_deterministic(oracle_lib):
    O = oracle_lib
    c = _attn_case(O, 2, 8, 2, [3000, 1234], seed=8)
    a = _gpu_attn(c)
    b = _gpu_attn(c)
    assert torch.equal(a, b)


def test_attention_timed_entry_point(oracle_lib):
    """dq_attn_decode_timed writes the same bytes as dq_attn_decode and the
    two events bracket a non-empty interval."""
    O = oracle_lib
    c = _attn_case(O, 2, 8, 2, [3000, 1234], seed=8)
    a = _gpu_attn(c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b = _gpu_attn(c, split_events=(e0, e1))
    assert torch.equal(a, b)
    assert e0.elapsed_time(e1) > 0.0


def test_attention_empty_sequence_gives_zero_row(oracle_lib):
    """A sequence of length 0 (outside the documented range) yields a zero
    output row and leaves every other row as it is with a valid length."""
    O = oracle_lib
    c = _attn_case(O, 3, 8, 2, [700, 90, 1300], seed=21)
    ref = _gpu_attn(c)
    c["sl"] = torch.tensor([700, 0, 1300], dtype=torch.int32, device=DEV)
    got = _gpu_attn(c, max_len=1300)
    assert torch.count_nonzero(got[1]).item() == 0
    assert torch.isfinite(got).all().item()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[2], ref[2])


def _append_both(c, k_new, v_new, max_len):
    """One decode step with append two ways on copies of the pools:
    dq.encode_kv then dq.attn_decode, and dq.attn_decode_append.  Returns
    (pools, stats, out) of each."""
    lens = c["lens"] + 1
    sl = torch.from_numpy(lens.astype(np.int32)).to(DEV)
    slots = torch.from_numpy((c["starts"] + c["lens"]).astype(np.int64)).to(DEV)
    res = []
    for fused in (False, True):
        pools = [t.clone() for t in (c["kc"], c["kn"], c["vc"], c["vn"])]
        st = (dq.new_stats(DEV), dq.new_stats(DEV))
        if fused:
            out = dq.attn_decode_append(c["ck"], c["cv"], c["q"], k_new, v_new, *pools, c["ss"], sl, max_len,
                                        k_stats=st[0], v_stats=st[1])
        else:
            dq.encode_kv(c["ck"], c["cv"], k_new, v_new, slots, *pools, k_stats=st[0], v_stats=st[1])
            out = dq.attn_decode(c["ck"], c["cv"], c["q"], *pools, c["ss"], sl, max_len)
        torch.cuda.synchronize()
        res.append((pools, st, out))
    return res, lens


@pytest.mark.parametrize("Hq,hkv,lens,order,C,split", [
    (8, 2, [0, 1, 63, 64, 65, 300, 1408, 2000], (0, 0), (34, 34), None),
    (4, 4, [0, 127, 128, 129, 1500], (1, 1), (34, 34), 128),
    (4, 2, [4095, 4096, 700], (0, 1), (29, 29), None),
    (1, 1, [640, 5], (1, 0), (34, 29), 192),
])
def test_attention_append(oracle_lib, knob, Hq, hkv, lens, order, C, split):
    """Decode with append in one launch: the new containers, norms and stats
    equal those of dq_encode_kv bit for bit, the output matches encode-then-
    attention up to fp32 order and the fp64 oracle within tolerance.  Old
    lengths 0 (the new token alone) and chunk boundaries at the new token
    (forced splits of 128 and 192 tokens) included."""
    O = oracle_lib
    if split:
        knob("split_tokens", str(split))
    c = _attn_case(O, len(lens), Hq, hkv, lens, C=C, seed=61 + Hq, order=order)
    B = len(lens)
    k_new = synth.kv_tensor("outlier", B, hkv, seed=71 + Hq, device=DEV)
    v_new = synth.kv_tensor("student_t5", B, hkv, seed=72 + Hq, device=DEV)
    max_len = max(lens) + 1
    (pa, sa, oa), (pb, sb, ob) = _append_both(c, k_new, v_new, max_len)[0]
    for x, y, name in zip(pa, pb, ("k_cont", "k_norm", "v_cont", "v_norm")):
        assert torch.equal(x, y), f"append: {name} differs from dq_encode_kv"
    for x, y in zip(sa, sb):
        assert dq.stats_dict(x) == dq.stats_dict(y)
    assert dq.stats_dict(sb[0])["vectors"] == B * hkv
    diff = float((oa - ob).abs().max())
    _say(f"append vs encode-then-attention: max-abs {diff:.3e}")
    assert diff <= 1e-5
    c2 = dict(c, kc=pb[0], kn=pb[1], vc=pb[2], vn=pb[3], lens=np.array(lens, np.int32) + 1)
    _assert_close(ob.cpu().numpy(), _oracle_attn(O, c2), f"append Hq={Hq} hkv={hkv}")
    # the encodes inside the attention launch or in a launch of their own
    # (the call picks by batch size): the same bytes and the same output
    forced = []
    for mode in ("1", "0"):
        knob("append_fuse", mode)
        forced.append(_append_both(c, k_new, v_new, max_len)[0][1])
    knob("append_fuse", None)
    (p1, s1, o1), (p0, s0, o0) = forced
    assert torch.equal(o1, o0) and torch.equal(o1, ob)
    for x, y in zip(list(p1) + list(s1), list(p0) + list(s0)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("Hq,hkv,lens,C,split", [
    (8, 2, [1, 63, 64, 65, 300, 129, 2000], (34, 34), None),
    (4, 4, [5000, 70], (29, 29), 640),
    (1, 1, [128, 1], (34, 29), 64),
])
def test_attention_latency_mode_bit_identical(oracle_lib, knob, Hq, hkv, lens, C, split):
    """Latency mode (each tile's K and V decoded in one pass, PV after the
    tile's softmax) and the pipelined mode do the same arithmetic in the same
    order: forced either way, plain decode and decode with append give the
    same bytes; and the oracle agrees."""
    O = oracle_lib
    if split:
        knob("split_tokens", str(split))
    c = _attn_case(O, len(lens), Hq, hkv, lens, C=C, seed=101 + Hq)
    B = len(lens)
    k_new = synth.kv_tensor("outlier", B, hkv, seed=111, device=DEV)
    v_new = synth.kv_tensor("outlier", B, hkv, seed=112, device=DEV)
    res = {}
    for mode in ("0", "1"):
        knob("latency_mode", mode)
        plain = _gpu_attn(c)
        (_, _, _), (pb, sb, ob) = _append_both(c, k_new, v_new, max(lens) + 1)[0]
        res[mode] = (plain, ob, pb)
    knob("latency_mode", None)
    assert torch.equal(res["0"][0], res["1"][0]), "plain decode differs between modes"
    assert torch.equal(res["0"][1], res["1"][1]), "decode with append differs between modes"
    for x, y in zip(res["0"][2], res["1"][2]):
        assert torch.equal(x, y)
    _assert_close(res["1"][0].cpu().numpy(), _oracle_attn(O, c), f"latency mode Hq={Hq} hkv={hkv}")


@pytest.mark.parametrize("Hq,hkv,lens,split", [
    (32, 8, [6400, 70, 3000, 1], 64),
    (8, 2, [20000, 640, 5, 12000, 129], 64),
    (4, 4, [9000, 9001, 64, 65], 128),
])
def test_attention_work_queue(oracle_lib, knob, Hq, hkv, lens, split):
    """Ragged batches whose items take several rounds of resident waves:
    split-K waves taking items from the device work queue give the same
    bytes as the static deal (each item's arithmetic does not depend on the
    wave that runs it), plain and with append (the queue also hands out the
    encode items when they ride in the launch), and match the oracle."""
    O = oracle_lib
    knob("split_tokens", split)
    c = _attn_case(O, len(lens), Hq, hkv, lens, seed=151 + Hq)
    B = len(lens)
    k_new = synth.kv_tensor("outlier", B, hkv, seed=161, device=DEV)
    v_new = synth.kv_tensor("outlier", B, hkv, seed=162, device=DEV)
    res = {}
    for mode in (0, 1):
        knob("work_queue", mode)
        plain = _gpu_attn(c)
        fused = []
        for fuse in (0, 1):
            knob("append_fuse", fuse)
            (_, _, _), (pb, sb, ob) = _append_both(c, k_new, v_new, max(lens) + 1)[0]
            fused.append((ob, pb))
        res[mode] = (plain, fused)
    assert torch.equal(res[0][0], res[1][0]), "queue and static deal differ"
    for (o0, p0), (o1, p1) in zip(res[0][1], res[1][1]):
        assert torch.equal(o0, o1)
        for x, y in zip(p0, p1):
            assert torch.equal(x, y)
    _assert_close(res[1][0].cpu().numpy(), _oracle_attn(O, c), f"work queue Hq={Hq} hkv={hkv}")


@pytest.mark.parametrize("Hq,hkv,lens,C,step64,split", [
    (8, 2, [1, 63, 64, 65, 300, 129, 2000], (34, 34), (0, 0), None),
    (4, 4, [5000, 70], (29, 29), (0, 0), 640),
    (1, 1, [128, 1], (34, 29), (0, 0), 64),
    (4, 2, [3000, 4097], (38, 29), (66, 0), None),  # the largest container the per-slot tables allow
])
def test_attention_slot_tables_bit_identical(oracle_lib, knob, Hq, hkv, lens, C, step64, split):
    """The per-slot decode tables (one LDS read per step) and the byte table
    plus symbol entries (two dependent reads) hold the same entries: the
    pipelined kernel gives the same bytes either way, plain, with append and
    over a paged pool; and the oracle agrees."""
    O = oracle_lib
    knob("latency_mode", 0)
    if split:
        knob("split_tokens", split)
    c = _attn_case(O, len(lens), Hq, hkv, lens, C=C, step64=step64, seed=171 + Hq, gap=64)
    B = len(lens)
    k_new = synth.kv_tensor("outlier", B, hkv, seed=181, device=DEV)
    v_new = synth.kv_tensor("student_t5", B, hkv, seed=182, device=DEV)
    pools, pages = _paged_copy(c, np.random.default_rng(5))
    pg = torch.from_numpy(pages).to(DEV)
    res = {}
    for mode in (0, 1):
        knob("slot_table", mode)
        plain = _gpu_attn(c)
        (_, _, _), (pb, sb, ob) = _append_both(c, k_new, v_new, max(lens) + 1)[0]
        paged = dq.attn_decode_paged(c["ck"], c["cv"], c["q"], *pools["K"], *pools["V"], pg, c["sl"],
                                     int(c["lens"].max()))
        torch.cuda.synchronize()
        res[mode] = (plain, ob, paged, pb)
    for x, y, name in zip(res[0][:3], res[1][:3], ("plain", "append", "paged")):
        assert torch.equal(x, y), f"{name} differs between table kinds"
    for x, y in zip(res[0][3], res[1][3]):
        assert torch.equal(x, y)
    _assert_close(res[1][0].cpu().numpy(), _oracle_attn(O, c), f"slot tables Hq={Hq} hkv={hkv}")


@pytest.mark.parametrize("Hq,hkv,lens,C,step64,split", [
    (8, 2, [1, 63, 64, 65, 300, 129, 2000], (34, 34), (0, 0), None),
    (4, 4, [5000, 70], (29, 29), (0, 0), 640),
    (1, 1, [128, 1], (34, 29), (0, 0), 64),
    (4, 2, [3000, 4097], (38, 29), (66, 0), None),
])
def test_attention_qk_valu_variant(oracle_lib, knob, Hq, hkv, lens, C, step64, split):
    """The measurement variant with the query-key products as fp32 fused
    multiply-adds on the vector ALU (the rotated query read from global
    memory) instead of MFMAs: within the tolerance of the fp64 oracle, plain
    and over a paged pool, and within fp32 rounding of the MFMA path."""
    O = oracle_lib
    knob("latency_mode", 0)
    knob("slot_table", 1)
    if split:
        knob("split_tokens", split)
    c = _attn_case(O, len(lens), Hq, hkv, lens, C=C, step64=step64, seed=211 + Hq, gap=64)
    pools, pages = _paged_copy(c, np.random.default_rng(9))
    pg = torch.from_numpy(pages).to(DEV)
    res = {}
    for mode in (0, 1):
        knob("qk_valu", mode)
        plain = _gpu_attn(c)
        paged = dq.attn_decode_paged(c["ck"], c["cv"], c["q"], *pools["K"], *pools["V"], pg, c["sl"],
                                     int(c["lens"].max()))
        torch.cuda.synchronize()
        res[mode] = (plain, paged)
    assert torch.equal(res[1][0], res[1][1]), "paged and contiguous differ"
    ref = _oracle_attn(O, c)
    _assert_close(res[1][0].cpu().numpy(), ref, f"qk on valu Hq={Hq} hkv={hkv}")
    assert float((res[1][0] - res[0][0]).abs().max()) <= 1e-4, "VALU and MFMA scores differ beyond fp32 rounding"


def test_decode_step_graph_replay(oracle_lib):
    """A decode step with append captured once in a HIP graph
    (torch.cuda.CUDAGraph over the library's launches, which go to the
    capturing stream) and replayed with new inputs: every replay, with eager
    launches and synchronisations between replays, writes the same output
    and pool bytes as the eager call on the same inputs."""
    O = oracle_lib
    lens = [700, 65, 1300, 1]
    B, Hq, hkv = len(lens), 8, 2
    c = _attn_case(O, B, Hq, hkv, lens, seed=91, gap=8)
    ck, cv = c["ck"], c["cv"]
    max_len = max(lens) + 1
    ws = torch.empty(dq.attn_workspace_bytes(B, Hq, hkv, max_len), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    q = c["q"].clone()
    k_new = synth.kv_tensor("outlier", B, hkv, seed=92, device=DEV)
    v_new = synth.kv_tensor("outlier", B, hkv, seed=93, device=DEV)
    sl = torch.from_numpy(np.array(lens, np.int32) + 1).to(DEV)
    pools = [t.clone() for t in (c["kc"], c["kn"], c["vc"], c["vn"])]

    def step():
        dq.attn_decode_append(ck, cv, q, k_new, v_new, *pools, c["ss"], sl, max_len, out=out, workspace=ws)

    side = torch.cuda.Stream()  # warm-up off the default stream, as torch asks before a capture
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        q.copy_(synth.q_tensor(B, Hq, seed=200 + r, device=DEV))
        k_new.copy_(synth.kv_tensor("outlier", B, hkv, seed=210 + r, device=DEV))
        v_new.copy_(synth.kv_tensor("student_t5", B, hkv, seed=220 + r, device=DEV))
        ref_pools = [t.clone() for t in pools]
        ref = dq.attn_decode_append(ck, cv, q, k_new, v_new, *ref_pools, c["ss"], sl, max_len)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r}: output differs from the eager call"
        for x, y, name in zip(pools, ref_pools, ("k_cont", "k_norm", "v_cont", "v_norm")):
            assert torch.equal(x, y), f"replay {r}: {name} differs from the eager call"
    c2 = dict(c, kc=pools[0], kn=pools[1], vc=pools[2], vn=pools[3], q=q, lens=np.array(lens, np.int32) + 1)
    _assert_close(out.cpu().numpy(), _oracle_attn(O, c2), "graph replay")


def _paged_copy(c, rng, extra_pages=5):
    """The contiguous pools of an attention case re-laid as shuffled 64-token
    pages in a larger pool, with the page table that addresses them."""
    P = dq.PAGE_TOKENS
    lens, starts = c["lens"], c["starts"]
    npages = [(int(L) + P - 1) // P for L in lens]
    total = sum(npages)
    phys = rng.permutation(total + extra_pages)[:total]
    pools = {}
    for tag, cont, norm in (("K", c["kc"], c["kn"]), ("V", c["vc"], c["vn"])):
        S2 = (total + extra_pages) * P
        cont2 = torch.zeros((cont.shape[0], dq.pool_slots(S2), cont.shape[2]), dtype=torch.uint8, device=DEV)
        norm2 = torch.zeros((cont.shape[0], cont2.shape[1]), dtype=torch.float16, device=DEV)
        pools[tag] = (cont2, norm2)
    pages = np.full((len(lens), max(npages) + 2), -7, np.int32)  # unused entries: never read
    logical = 0
    for b, n in enumerate(npages):
        for j in range(n):
            s0 = int(starts[b]) + j * P
            d0 = int(phys[logical]) * P
            for tag, cont, norm in (("K", c["kc"], c["kn"]), ("V", c["vc"], c["vn"])):
                hi = min(s0 + P, cont.shape[1])
                pools[tag][0][:, d0:d0 + hi - s0] = cont[:, s0:hi]
                pools[tag][1][:, d0:d0 + hi - s0] = norm[:, s0:hi]
            pages[b, j] = phys[logical]
            logical += 1
    return pools, pages


def test_attention_paged_pool(oracle_lib):
    """Shuffled 64-token pages addressed through a page table: the same
    result as the contiguous call bit for bit, and within tolerance of the
    oracle's paged attention, for ragged lengths and two group sizes."""
    O = oracle_lib
    rng = np.random.default_rng(17)
    for Hq, hkv in ((8, 2), (4, 4)):
        lens = [1, 63, 64, 65, 300, 129]
        c = _attn_case(O, len(lens), Hq, hkv, lens, seed=40 + Hq, gap=64)
        ref_contig = _gpu_attn(c)
        pools, pages = _paged_copy(c, rng)
        pg = torch.from_numpy(pages).to(DEV)
        out = dq.attn_decode_paged(c["ck"], c["cv"], c["q"], *pools["K"], *pools["V"], pg, c["sl"],
                                   int(c["lens"].max()))
        torch.cuda.synchronize()
        assert torch.equal(out, ref_contig), "paged and contiguous results differ"
        ref = O.attention_paged(c["ock"], c["ocv"], _np_bits(c["q"]), pools["K"][0].cpu().numpy(),
                                _np_bits(pools["K"][1]), pools["V"][0].cpu().numpy(),
                                _np_bits(pools["V"][1]), pages, c["lens"])
        _assert_close(out.cpu().numpy(), ref, f"paged Hq={Hq} hkv={hkv}")


def test_attention_paged_append(oracle_lib):
    """Decode with append over shuffled 64-token pages: each new token lands
    in its page's slot with the bytes of the contiguous append (also when it
    opens a new page), and the output equals the contiguous one bit for
    bit."""
    O = oracle_lib
    rng = np.random.default_rng(23)
    lens = [0, 63, 64, 65, 300, 127]
    B = len(lens)
    c = _attn_case(O, B, 8, 2, lens, seed=44, gap=64)
    k_new = synth.kv_tensor("outlier", B, 2, seed=81, device=DEV)
    v_new = synth.kv_tensor("outlier", B, 2, seed=82, device=DEV)
    max_len = max(lens) + 1
    (_, _, _), (pb, sb, ob) = _append_both(c, k_new, v_new, max_len)[0]
    pools, pages = _paged_copy(dict(c, lens=c["lens"] + 1), rng)
    pg = torch.from_numpy(pages).to(DEV)
    sl = torch.from_numpy((c["lens"] + 1).astype(np.int32)).to(DEV)
    st = (dq.new_stats(DEV), dq.new_stats(DEV))
    outp = dq.attn_decode_paged_append(c["ck"], c["cv"], c["q"], k_new, v_new, *pools["K"], *pools["V"], pg, sl,
                                       max_len, k_stats=st[0], v_stats=st[1])
    torch.cuda.synchronize()
    assert torch.equal(outp, ob), "paged and contiguous append results differ"
    P = dq.PAGE_TOKENS
    for b, L in enumerate(lens):
        sp = int(pages[b, L // P]) * P + L % P
        sc = int(c["starts"][b]) + L
        for (cont, norm), cc, nc in ((pools["K"], pb[0], pb[1]), (pools["V"], pb[2], pb[3])):
            assert torch.equal(cont[:, sp], cc[:, sc]) and torch.equal(norm[:, sp], nc[:, sc])
    for x, y in zip(st, sb):
        assert dq.stats_dict(x) == dq.stats_dict(y)


def test_attention_paged_ids_outside_pool_read_zeros(oracle_lib):
    """A page id past the pool or negative is a caller error: the kernel's
    pool bounds checks turn it into zero containers; the other sequences
    are unaffected."""
    O = oracle_lib
    lens = [130, 70]
    c = _attn_case(O, 2, 8, 2, lens, seed=3, gap=64)
    pools, pages = _paged_copy(c, np.random.default_rng(2), extra_pages=0)
    n_pool_pages = pools["K"][0].shape[1] // dq.PAGE_TOKENS
    bad = pages.copy()
    bad[0, 1] = n_pool_pages + 1
    bad[0, 2] = -1
    pg = torch.from_numpy(bad).to(DEV)
    out = dq.attn_decode_paged(c["ck"], c["cv"], c["q"], *pools["K"], *pools["V"], pg, c["sl"], 130)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    good = _gpu_attn(c)
    assert torch.equal(out[1], good[1])


def test_tiny_1seq_1k_config(oracle_lib):
    """1 sequence, 1 query / 1 kv head, context 1024, per-token scaled
    N(0,1) K/V, 34-byte containers: every container and the output."""
    O = oracle_lib
    w = synth.workloads()["tiny_1seq_1k"]
    ck, ock = _codecs(O, 8, 34, seed=w.seed, hkv=1)
    cv, ocv = _codecs(O, 6, 34, seed=w.seed + 1, hkv=1)
    K = synth.kv_tensor(w.kind, 1024, 1, seed=w.seed + 10, device=DEV)
    V = synth.kv_tensor(w.kind, 1024, 1, seed=w.seed + 11, device=DEV)
    slots = torch.arange(1024, dtype=torch.int64, device=DEV)
    for gc, oc, x in ((ck, ock, K), (cv, ocv, V)):
        _assert_encode_equal(*_encode_both(O, gc, oc, x, slots, 1024), "tiny")
    c = _attn_case(O, 1, 1, 1, [1024], kinds=(w.kind, w.kind), seed=w.seed)
    _assert_close(_gpu_attn(c).cpu().numpy(), _oracle_attn(O, c), "tiny attention")


def test_qwen3_shape_full_encode_and_sampled_attention(oracle_lib):
    """Batch 16 x 8192 context, 32 q / 8 kv heads, outlier channels, 34-byte
    containers: every K and V container bit-exact; attention rows of two
    sequences against the oracle, in the launch configuration the bench uses."""
    O = oracle_lib
    w = synth.workloads()["qwen3_8b_b16_8k"]
    B, Hq, hkv, ctx = w.batch, w.hq, w.hkv, w.ctx[0]
    total = B * ctx
    _say("qwen3-shape: encode")
    ck, ock = _codecs(O, 8, 34, seed=w.seed, hkv=hkv)
    cv, ocv = _codecs(O, 6, 34, seed=w.seed + 1, hkv=hkv)
    K = synth.kv_tensor(w.kind, total, hkv, seed=w.seed + 10, device=DEV)
    V = synth.kv_tensor(w.kind, total, hkv, seed=w.seed + 11, device=DEV)
    slots = torch.arange(total, dtype=torch.int64, device=DEV)
    pools = {}
    for name, gc, oc, x in (("K", ck, ock, K), ("V", cv, ocv, V)):
        cont, norm, st, ocont, onorm, ost = _encode_both(O, gc, oc, x, slots, total)
        _assert_encode_equal(cont, norm, st, ocont, onorm, ost, f"qwen3 {name}")
        s = dq.stats_dict(st)
        _say(f"qwen3 {name}: drift rate {s['drifted_symbols'] / (128 * s['vectors']):.4%}, "
             f"multilevel {s['multilevel_events']}")
        pools[name] = (cont, norm)
    _say("qwen3-shape: attention")
    q = synth.q_tensor(B, Hq, seed=w.seed + 12, device=DEV)
    ss = torch.arange(B, dtype=torch.int64, device=DEV) * ctx
    sl = torch.full((B,), ctx, dtype=torch.int32, device=DEV)
    out = dq.attn_decode(ck, cv, q, *pools["K"], *pools["V"], ss, sl, ctx)
    torch.cuda.synchronize()
    rows = [0, 9]
    ref = O.attention(ock, ocv, _np_bits(q)[rows], pools["K"][0].cpu().numpy(), _np_bits(pools["K"][1]),
                      pools["V"][0].cpu().numpy(), _np_bits(pools["V"][1]),
                      ss.cpu().numpy()[rows], sl.cpu().numpy()[rows])
    _assert_close(out.cpu().numpy()[rows], ref, "qwen3 attention rows 0, 9")


def _workload_case(O, name, cap_extra):
    """Every context token of a workload encoded into pools with `cap_extra`
    free slots after each sequence (as the bench lays them out); every K and
    V container, norm and stat bit-exact against the oracle."""
    w = synth.workloads()[name]
    hkv = w.hkv
    ctx = np.array(w.ctx, np.int64)
    cap = ctx + cap_extra
    starts = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    S = int(cap.sum())
    ck, ock = _codecs(O, w.levels_k, w.container_k, seed=w.seed, hkv=hkv)
    cv, ocv = _codecs(O, w.levels_v, w.container_v, seed=w.seed + 1, hkv=hkv)
    slots = torch.from_numpy(np.concatenate([np.arange(s, s + L) for s, L in zip(starts, ctx)])).to(DEV)
    pools = {}
    for tag, gc, oc, seed in (("K", ck, ock, w.seed + 10), ("V", cv, ocv, w.seed + 11)):
        _say(f"{name}: encode {tag} ({slots.numel()} tokens x {hkv} heads)")
        x = synth.kv_tensor(w.kind, slots.numel(), hkv, seed=seed, device=DEV)
        cont, norm, st, ocont, onorm, ost = _encode_both(O, gc, oc, x, slots, S)
        _assert_encode_equal(cont, norm, st, ocont, onorm, ost, f"{name} {tag}")
        s = dq.stats_dict(st)
        _say(f"{name} {tag}: drift rate {s['drifted_symbols'] / (128 * s['vectors']):.4%}, "
             f"multilevel {s['multilevel_events']}")
        pools[tag] = (cont, norm)
        del x
    return dict(w=w, ck=ck, cv=cv, ock=ock, ocv=ocv, pools=pools, starts=starts, ctx=ctx, S=S)


def _append_and_check(O, c, n_new, seed):
    """Encodes n_new tokens after each sequence's context (the append of a
    decode step or a prefill chunk) and checks the new containers."""
    w = c["w"]
    slots_np = np.concatenate([np.arange(s + L, s + L + n_new) for s, L in zip(c["starts"], c["ctx"])])
    slots = torch.from_numpy(slots_np).to(DEV)
    for tag, gc, oc, off in (("K", c["ck"], c["ock"], 0), ("V", c["cv"], c["ocv"], 1)):
        x = synth.kv_tensor(w.kind, slots.numel(), w.hkv, seed=seed + off, device=DEV)
        cont, norm = c["pools"][tag]
        st = dq.new_stats(DEV)
        dq.encode(gc, x, slots, cont, norm, st)
        torch.cuda.synchronize()
        ocont, onorm, ost = O.encode(oc, _np_bits(x), slots_np, num_slots=cont.shape[1])
        got = cont[:, slots].cpu().numpy()
        assert (got == ocont[:, slots_np]).all(), f"{w.name} appended {tag} containers differ"
        assert (_np_bits(norm[:, slots]) == onorm[:, slots_np]).all()
        assert dq.stats_dict(st) == O_stats(ost)
    return torch.from_numpy(c["ctx"] + n_new)


def _sampled_attention(O, c, lens, max_len, rows, label):
    w = c["w"]
    q = synth.q_tensor(w.batch, w.hq, seed=w.seed + 12, device=DEV)
    ss = torch.from_numpy(c["starts"]).to(DEV)
    sl = lens.to(torch.int32).to(DEV)
    kc, kn = c["pools"]["K"]
    vc, vn = c["pools"]["V"]
    out = dq.attn_decode(c["ck"], c["cv"], q, kc, kn, vc, vn, ss, sl, int(max_len))
    torch.cuda.synchronize()
    ref = O.attention(c["ock"], c["ocv"], _np_bits(q)[rows], kc.cpu().numpy(), _np_bits(kn),
                      vc.cpu().numpy(), _np_bits(vn), c["starts"][rows], lens.numpy().astype(np.int32)[rows])
    _assert_close(out.cpu().numpy()[rows], ref, f"{label} attention rows {rows}")
    return out


def test_llama31_b128_8k_bench_configuration(oracle_lib):
    """Batch 128 x 8192, 32 q / 8 kv heads, 34-byte containers, laid out as
    the bench does (28 free slots per sequence: 12 warm-up and 16 timed
    steps): the full prompt encode
    bit-exact, one decode step's append bit-exact, and attention at the
    bench's max_len (context + 28) on sampled sequences."""
    O = oracle_lib
    c = _workload_case(O, "llama31_8b_b128_8k", cap_extra=28)
    lens = _append_and_check(O, c, 1, seed=c["w"].seed + 20)
    out = _sampled_attention(O, c, lens, int(c["ctx"].max()) + 28, [0, 77, 127], "llama31 b128")
    # the same pools re-laid as shuffled 64-token pages: identical output
    P = dq.PAGE_TOKENS
    cap = int(c["ctx"][0]) + 28
    npg = (cap + P - 1) // P
    B = c["w"].batch
    rng = np.random.default_rng(8)
    phys = torch.from_numpy(rng.permutation(B * npg).astype(np.int64)).to(DEV)
    pages = phys.view(B, npg).to(torch.int32).contiguous()
    src = (torch.from_numpy(c["starts"]).to(DEV)[:, None] + torch.arange(npg, device=DEV)[None, :] * P)
    paged = {}
    for tag in ("K", "V"):
        cont, norm = c["pools"][tag]
        cont2 = torch.zeros((cont.shape[0], B * npg * P, cont.shape[2]), dtype=torch.uint8, device=DEV)
        norm2 = torch.zeros((cont.shape[0], B * npg * P), dtype=torch.float16, device=DEV)
        for j in range(P):
            s_idx = (src + j).clamp(max=cont.shape[1] - 1).flatten()
            d_idx = (phys.view(B, npg) * P + j).flatten()
            cont2[:, d_idx] = cont[:, s_idx]
            norm2[:, d_idx] = norm[:, s_idx]
        paged[tag] = (cont2, norm2)
    q = synth.q_tensor(B, c["w"].hq, seed=c["w"].seed + 12, device=DEV)
    outp = dq.attn_decode_paged(c["ck"], c["cv"], q, *paged["K"], *paged["V"], pages,
                                lens.to(torch.int32).to(DEV), int(c["ctx"].max()) + 28)
    torch.cuda.synchronize()
    assert torch.equal(outp, out), "paged pool differs from the contiguous pool at full size"
    # the next decode step as one launch (append + attention): the new
    # containers, norms and stats bit-exact against the oracle's encode,
    # sampled rows within tolerance of the oracle's attention
    w = c["w"]
    k_new = synth.kv_tensor(w.kind, B, w.hkv, seed=w.seed + 30, device=DEV)
    v_new = synth.kv_tensor(w.kind, B, w.hkv, seed=w.seed + 31, device=DEV)
    lens2 = lens + 1
    slots_np = (c["starts"] + lens.numpy()).astype(np.int64)
    kc, kn = c["pools"]["K"]
    vc, vn = c["pools"]["V"]
    st = (dq.new_stats(DEV), dq.new_stats(DEV))
    out2 = dq.attn_decode_append(c["ck"], c["cv"], q, k_new, v_new, kc, kn, vc, vn,
                                 torch.from_numpy(c["starts"]).to(DEV), lens2.to(torch.int32).to(DEV),
                                 int(c["ctx"].max()) + 28, k_stats=st[0], v_stats=st[1])
    torch.cuda.synchronize()
    for x, oc, (cont, norm), s in ((k_new, c["ock"], (kc, kn), st[0]), (v_new, c["ocv"], (vc, vn), st[1])):
        ocont, onorm, ost = O.encode(oc, _np_bits(x), slots_np, num_slots=cont.shape[1])
        assert (cont[:, slots_np].cpu().numpy() == ocont[:, slots_np]).all(), "fused append containers differ"
        assert (_np_bits(norm[:, slots_np]) == onorm[:, slots_np]).all()
        assert dq.stats_dict(s) == O_stats(ost)
    rows = [3, 64, 126]
    ref = O.attention(c["ock"], c["ocv"], _np_bits(q)[rows], kc.cpu().numpy(), _np_bits(kn), vc.cpu().numpy(),
                      _np_bits(vn), c["starts"][rows], lens2.numpy().astype(np.int32)[rows])
    _assert_close(out2.cpu().numpy()[rows], ref, f"llama31 b128 fused append rows {rows}")


def test_longctx_b4_64k_c29(oracle_lib):
    """Batch 4 x 65536, 29-byte containers (1.94 bits/value), Student-t (5)
    K/V: full encode bit-exact, attention on two sequences."""
    O = oracle_lib
    c = _workload_case(O, "longctx_b4_64k_c29", cap_extra=0)
    _sampled_attention(O, c, torch.from_numpy(c["ctx"]), int(c["ctx"].max()), [1, 3], "longctx c29")


def test_ragged_32seq_4k_128k(oracle_lib):
    """32 sequences with log-uniform contexts in [4096, 131072]: full encode
    bit-exact, the 8192-token chunk appended to every sequence bit-exact,
    attention over the grown lengths on the shortest, a middle and the
    longest sequence."""
    O = oracle_lib
    c = _workload_case(O, "ragged_32seq_4k_128k", cap_extra=8192)
    lens = _append_and_check(O, c, 8192, seed=c["w"].seed + 30)
    order = np.argsort(c["ctx"])
    rows = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    _sampled_attention(O, c, lens, int(lens.max()), rows, "ragged")


def _prefill_case(O, lens, Tq, Hq, hkv, seed, kinds=("outlier", "iid_scaled"), C=(34, 34), levels=(8, 6),
                  step64=(0, 0)):
    c = _attn_case(O, len(lens), Hq, hkv, lens, kinds=kinds, C=C, seed=seed, levels=levels, step64=step64)
    q = synth.q_tensor(len(lens) * Tq, Hq, seed=seed + 9, device=DEV).view(len(lens), Tq, Hq, 128).contiguous()
    return c, q


def _gpu_prefill(c, q, max_len=None, **kw):
    out = dq.attn_prefill(c["ck"], c["cv"], q, c["kc"], c["kn"], c["vc"], c["vn"], c["ss"], c["sl"],
                          int(max_len or c["lens"].max()), **kw)
    torch.cuda.synchronize()
    return out


def _oracle_prefill(O, c, q, sm_scale=None):
    return O.attention_prefill(c["ock"], c["ocv"], _np_bits(q), c["kc"].cpu().numpy(), _np_bits(c["kn"]),
                               c["vc"].cpu().numpy(), _np_bits(c["vn"]), c["starts"], c["lens"],
                               sm_scale=sm_scale)


@pytest.mark.parametrize("Hq,hkv,Tq", [(8, 2, 5), (4, 4, 16), (4, 2, 1), (8, 2, 16), (2, 2, 3)])
def test_prefill_attention_small(oracle_lib, Hq, hkv, Tq):
    """Causal chunked prefill on ragged contexts (including a context equal
    to the chunk), every query row against the oracle."""
    O = oracle_lib
    lens = [max(Tq, 1), 63 + Tq, 300, 129, 64 + Tq]
    c, q = _prefill_case(O, lens, Tq, Hq, hkv, seed=Hq * 7 + hkv + Tq)
    _assert_close(_gpu_prefill(c, q).cpu().numpy(), _oracle_prefill(O, c, q), f"prefill Hq={Hq} hkv={hkv} Tq={Tq}")


@pytest.mark.parametrize("C,step64,Tq", [((44, 40), (30, 40), 21), ((60, 48), (30, 40), 9)])
def test_prefill_attention_per_block_kernel(oracle_lib, C, step64, Tq):
    """Containers too large for the shared-decode kernel's LDS (44 and 60
    bytes) take the per-block kernel: every row against the oracle."""
    O = oracle_lib
    lens = [Tq, 200 + Tq, 70]
    c, q = _prefill_case(O, lens, Tq, 8, 2, seed=31 + C[0], C=C, step64=step64)
    _assert_close(_gpu_prefill(c, q).cpu().numpy(), _oracle_prefill(O, c, q), f"prefill C={C}")


@pytest.mark.parametrize("Tq", [40, 129])
def test_prefill_many_query_blocks(oracle_lib, Tq):
    """More query blocks than one shared-decode item holds (8), a ragged
    last item, and contexts of 1 to 6 rounds: every row against the oracle."""
    O = oracle_lib
    lens = [Tq, Tq + 1, 600, 1500]
    c, q = _prefill_case(O, lens, Tq, 8, 2, seed=41 + Tq)
    _assert_close(_gpu_prefill(c, q).cpu().numpy(), _oracle_prefill(O, c, q), f"prefill Tq={Tq}")


def test_prefill_one_query_equals_decode(oracle_lib):
    O = oracle_lib
    lens = [1, 100, 777]
    c, q = _prefill_case(O, lens, 1, 8, 2, seed=5)
    pre = _gpu_prefill(c, q)[:, 0]
    c["q"] = q[:, 0].contiguous()
    dec = _gpu_attn(c)
    err = float((pre - dec).abs().max())
    assert err <= MAX_ABS / 4, err


def test_prefill_split_invariance(oracle_lib, knob):
    O = oracle_lib
    lens = [2000, 900]
    c, q = _prefill_case(O, lens, 12, 8, 2, seed=11, kinds=("iid_scaled", "student_t5"), C=(34, 29))
    ref = _oracle_prefill(O, c, q, sm_scale=0.1)
    for split in (64, 256, 1024):
        knob("split_tokens", split)
        _assert_close(_gpu_prefill(c, q, sm_scale=0.1).cpu().numpy(), ref, f"prefill split={split}")
    knob("split_tokens", None)
    _assert_close(_gpu_prefill(c, q, sm_scale=0.1).cpu().numpy(), ref, "prefill split=default")


def test_prefill_8k_context_64_token_chunk(oracle_lib):
    """Two sequences of 8192 tokens (Qwen3-8B-shaped heads, outlier
    channels) whose last 64 tokens are the chunk: every row."""
    O = oracle_lib
    lens = [8192, 8192]
    c, q = _prefill_case(O, lens, 64, 32, 8, seed=23)
    _assert_close(_gpu_prefill(c, q).cpu().numpy(), _oracle_prefill(O, c, q), "prefill 8k/64")



@pytest.mark.parametrize("C,levels,step64", [((60, 48), (8, 6), (30, 40)), ((132, 100), (16, 12), (25, 25)),
                                             ((80, 48), (2, 8), (20, 64))])
def test_attention_large_containers(oracle_lib, C, levels, step64):
    """Containers above 47 and 79 bytes take the 5- and 9-piece tile fetch
    and fewer waves per block; 2, 12 and 16 levels."""
    O = oracle_lib
    lens = [1, 64, 65, 300, 1000]
    for Hq, hkv in ((8, 2), (4, 4)):
        c = _attn_case(O, len(lens), Hq, hkv, lens, kinds=("student_t5", "outlier"), C=C, seed=C[0] + Hq,
                       levels=levels, step64=step64)
        _assert_close(_gpu_attn(c).cpu().numpy(), _oracle_attn(O, c), f"decode C={C} L={levels} Hq={Hq}")
    c, q = _prefill_case(O, [70, 300], 9, 8, 2, seed=C[1], C=C, levels=levels, step64=step64)
    _assert_close(_gpu_prefill(c, q).cpu().numpy(), _oracle_prefill(O, c, q), f"prefill C={C} L={levels}")


@pytest.mark.parametrize("levels,C,step64", [(16, 132, 25), (2, 20, 64), (12, 48, 30), (8, 132, 30)])
def test_encode_extreme_codecs(oracle_lib, encode_path, levels, C, step64):
    """Largest container, most and fewest levels: bit-exact containers."""
    O = oracle_lib
    gc, oc = _codecs(O, levels, C, seed=77, hkv=2, step64=step64)
    for kind in ("iid", "outlier"):
        x = synth.kv_tensor(kind, 150, 2, seed=78, device=DEV)
        slots = torch.arange(150, dtype=torch.int64, device=DEV)
        _assert_encode_equal(*_encode_both(O, gc, oc, x, slots, 150), f"extreme {levels}/{C}/{kind}")



@pytest.mark.parametrize("T,order", [(128, 0), (100, 1), (5000, 0)])
def test_encode_kv_matches_separate_calls(oracle_lib, T, order):
    """One K+V call writes the same bytes and stats as two dq_encode calls
    (fused launch for small batches, two launches above the threshold),
    and both equal the oracle."""
    O = oracle_lib
    hkv = 8 if T <= 128 else 4
    ck, ock = _codecs(O, 8, 34, seed=3, hkv=hkv, order=order)
    cv, ocv = _codecs(O, 6, 34, seed=4, hkv=hkv, order=order)
    k = synth.kv_tensor("outlier", T, hkv, seed=5, device=DEV)
    v = synth.kv_tensor("outlier", T, hkv, seed=6, device=DEV)
    slots = torch.randperm(T + 40, generator=torch.Generator().manual_seed(1))[:T].to(DEV)
    pools = [dq.alloc_pool(c, T + 40, DEV) for c in (ck, cv)]
    sts = [dq.new_stats(DEV), dq.new_stats(DEV)]
    dq.encode_kv(ck, cv, k, v, slots, *pools[0], *pools[1], *sts)
    torch.cuda.synchronize()
    for (codec, oc, x), (cont, norm), st in zip(((ck, ock, k), (cv, ocv, v)), pools, sts):
        c2, n2 = dq.alloc_pool(codec, T + 40, DEV)
        s2 = dq.new_stats(DEV)
        dq.encode(codec, x, slots, c2, n2, s2)
        torch.cuda.synchronize()
        assert torch.equal(cont, c2) and torch.equal(norm, n2)
        assert dq.stats_dict(st) == dq.stats_dict(s2)
        ocont, onorm, ost = O.encode(oc, _np_bits(x), slots.cpu().numpy(), num_slots=cont.shape[1])
        _assert_encode_equal(cont, norm, st, ocont, onorm, ost, f"encode_kv T={T}")
