"""GPU parity of the HIP path against the fp64 oracle, at sizes the oracle
finishes in seconds that still span several tiles and a ragged tail, plus the
invariants the pages fix (single visible key, prefix invariance, shared ==
per-layer copies, decode == last prefill row, split independence).

Attention parity is checked against the oracle run on the GPU's own stored
K^/V^/Q^, so projection rounding never enters the attention tolerance; the
projections are checked separately against the fp64 projection."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_parity, assert_projection_bf16, to_dev, to_stored
from workloads import as_f32

pytestmark = pytest.mark.gpu

y = pytest.importorskip("yoco_shared_kv_amd")

ORC = None


def orc():
    global ORC
    if ORC is None:
        ORC = oracle.default()
    return ORC


def rng(seed):
    return np.random.default_rng(seed)


def make_cache_from(k_list, v_list, capacity, dtype):
    """Cache holding the given per-sequence stored slabs (rows beyond each
    length hold a canary pattern)."""
    n_seq = len(k_list)
    hkv, dh = k_list[0].shape[1:]
    tdt = torch.bfloat16 if dtype == W.BF16 else torch.float32
    cache = y.KVCache(n_seq, capacity, hkv, dh, tdt)
    cache.k.fill_(7.0)
    cache.v.fill_(7.0)
    for b, (kb, vb) in enumerate(zip(k_list, v_list)):
        cache.k[b, : kb.shape[0]] = to_dev(kb)
        cache.v[b, : vb.shape[0]] = to_dev(vb)
        cache.len[b] = kb.shape[0]
    return cache


# ---------------------------------------------------------------------------
# Tiny fp32 end-to-end case: project, q-project, prefill, append, decode.
# ---------------------------------------------------------------------------
def test_tiny_fp32_end_to_end():
    c = W.make_tiny()
    n, hq, hkv, dh = c.n_prompt, c.n_q_heads, c.n_kv_heads, c.head_dim
    dev = {k: to_dev(getattr(c, k)) for k in ("m", "x", "w_k", "w_v", "w_q", "gain_kv", "gain_q")}
    cache = y.KVCache(1, n + 1, hkv, dh, torch.float32, zero=True)

    y.kv_project(cache, dev["m"][:n], dev["w_k"], dev["w_v"], dev["gain_kv"], c.eps)
    assert cache.len.tolist() == [n]
    ref_k = orc().project(c.m[:n], c.w_k, c.gain_kv, c.eps).reshape(n, hkv, dh)
    ref_v = orc().project(c.m[:n], c.w_v, c.gain_kv, c.eps).reshape(n, hkv, dh)
    k_st = to_stored(cache.k[0, :n])
    v_st = to_stored(cache.v[0, :n])
    assert_parity(k_st, ref_k, bf16=False, what="K^ projection")
    assert_parity(v_st, ref_v, bf16=False, what="V^ projection")

    q = y.q_project(dev["x"][:n], dev["w_q"], hq, dh, dev["gain_q"], c.eps)
    q_st = to_stored(q)
    assert_parity(q_st, orc().project(c.x[:n], c.w_q, c.gain_q, c.eps).reshape(n, hq, dh), bf16=False,
                  what="Q^ projection")

    o, lse = y.cross_attn_prefill(q, cache, q_start=0, softmax_scale=c.softmax_scale, want_lse=True)
    ro, rlse = orc().prefill(q_st, 0, k_st, v_st, c.softmax_scale, want_lse=True)
    assert_parity(to_stored(o), ro, bf16=False, what="prefill O")
    assert_parity(to_stored(lse), rlse, bf16=False, what="prefill lse")

    # generated token: position 257 (row 256)
    y.kv_append(cache, dev["m"][n:n + 1], dev["w_k"], dev["w_v"], dev["gain_kv"], c.eps)
    assert cache.len.tolist() == [n + 1]
    k_all = to_stored(cache.k[0])
    v_all = to_stored(cache.v[0])
    assert_parity(k_all[n], orc().project(c.m[n:n + 1], c.w_k, c.gain_kv, c.eps).reshape(hkv, dh),
                  bf16=False, what="appended K^ row")
    qn = y.q_project(dev["x"][n:n + 1], dev["w_q"], hq, dh, dev["gain_q"], c.eps)
    od, lsed = y.cross_attn_decode(qn, cache, c.softmax_scale, want_lse=True)
    rd, rlsed = orc().decode(to_stored(qn), n + 1, k_all, v_all, c.softmax_scale, want_lse=True)
    assert_parity(to_stored(od), rd, bf16=False, what="decode O")
    assert_parity(to_stored(lsed), rlsed, bf16=False, what="decode lse")


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------
DECODE_CASES = [
    # (dtype, dh, hq, hkv, lens, rows_per_split)
    (W.BF16, 128, 24, 8, [5000], 0),
    (W.BF16, 128, 24, 8, [5000], 256),
    (W.BF16, 128, 8, 8, [1, 300, 4097], 0),
    (W.BF16, 64, 8, 4, [777, 1], 512),
    (W.BF16, 64, 16, 4, [2049], 0),
    (W.BF16, 128, 12, 2, [1500, 3000], 256),
    (W.BF16, 128, 64, 8, [999], 256),
    (W.F32, 64, 4, 2, [257, 3], 256),
    (W.F32, 128, 6, 1, [1200], 0),
]


def _decode_case(dtype, dh, hq, hkv, lens, seed=0):
    r = rng(seed)
    ks = [W.store(r.standard_normal((L, hkv, dh)).astype(np.float32), dtype) for L in lens]
    vs = [W.store(r.standard_normal((L, hkv, dh)).astype(np.float32), dtype) for L in lens]
    q = W.store(r.standard_normal((len(lens), hq, dh)).astype(np.float32), dtype)
    return ks, vs, q


@pytest.mark.parametrize("dtype,dh,hq,hkv,lens,rows", DECODE_CASES)
def test_decode_parity(dtype, dh, hq, hkv, lens, rows):
    ks, vs, q = _decode_case(dtype, dh, hq, hkv, lens)
    cache = make_cache_from(ks, vs, max(lens) + 5, dtype)
    s = 1 / math.sqrt(dh)
    n_seq = len(lens)
    # Guard bands: the outputs are views into NaN-filled buffers with a row
    # before and after, and the workspace is followed by a 64 KiB pattern;
    # the decode must write only its [n_seq, H_q, d_h] and [n_seq, H_q]
    # outputs and stay inside the workspace size the library reports.
    o_buf = torch.full((n_seq + 2, hq, dh), float("nan"), dtype=torch.float32, device="cuda")
    lse_buf = torch.full((n_seq + 2, hq), float("nan"), dtype=torch.float32, device="cuda")
    ws_bytes = y.decode_workspace_bytes(cache, hq, rows)
    guard = 64 * 1024
    ws_buf = torch.zeros(ws_bytes + guard, dtype=torch.uint8, device="cuda")
    ws_buf[ws_bytes:] = 0xA5
    o, lse = y.cross_attn_decode(to_dev(q), cache, s, workspace=ws_buf[:ws_bytes], rows_per_split=rows,
                                 out=o_buf[1:n_seq + 1], lse_out=lse_buf[1:n_seq + 1], want_lse=True)
    torch.cuda.synchronize()
    assert torch.isnan(o_buf[0]).all() and torch.isnan(o_buf[n_seq + 1]).all(), "decode wrote outside o"
    assert torch.isnan(lse_buf[0]).all() and torch.isnan(lse_buf[n_seq + 1]).all(), "decode wrote outside lse"
    assert bool((ws_buf[ws_bytes:] == 0xA5).all()), "decode wrote past its workspace"
    assert not bool(ws_buf[:64 * 1024].any()), "decode left an arrival counter non-zero"
    o, lse = to_stored(o), to_stored(lse)
    for b, L in enumerate(lens):
        ro, rl = orc().decode(q[b:b + 1], L, ks[b], vs[b], s, want_lse=True)
        assert_parity(o[b], ro[0], bf16=(dtype == W.BF16), what=f"decode seq {b} len {L}")
        assert_parity(lse[b], rl[0], bf16=(dtype == W.BF16), what=f"decode lse seq {b}")


def test_decode_split_size_independence_and_determinism():
    ks, vs, q = _decode_case(W.BF16, 128, 24, 8, [6000, 2500], seed=3)
    cache = make_cache_from(ks, vs, 6000, W.BF16)
    qd = to_dev(q)
    outs = {}
    for rows in (256, 512, 1024, 4096, 0):
        ws = y.decode_workspace(cache, 24, rows)
        a = to_stored(y.cross_attn_decode(qd, cache, workspace=ws, rows_per_split=rows))
        b = to_stored(y.cross_attn_decode(qd, cache, workspace=ws, rows_per_split=rows))
        assert np.array_equal(a, b), f"decode not bitwise reproducible at rows_per_split={rows}"
        outs[rows] = a
    ref = [orc().decode(q[b:b + 1], L, ks[b], vs[b], 1 / math.sqrt(128))[0] for b, L in enumerate([6000, 2500])]
    for rows, o in outs.items():
        for b in range(2):
            assert_parity(o[b], ref[b], bf16=True, what=f"rows_per_split={rows} seq {b}")


def test_decode_shared_cache_equals_per_layer_copies():
    """13 layers over one shared K^/V^ give exactly what 13 layers each over
    their own copy of the same K^/V^ give."""
    ks, vs, q13 = _decode_case(W.BF16, 128, 24, 8, [3000], seed=4)
    layers_q = [to_dev(W.store(rng(100 + l).standard_normal((1, 24, 128)).astype(np.float32), W.BF16))
                for l in range(13)]
    shared = make_cache_from(ks, vs, 3000, W.BF16)
    ws = y.decode_workspace(shared, 24)
    out_shared = [to_stored(y.cross_attn_decode(ql, shared, workspace=ws)) for ql in layers_q]
    for l, ql in enumerate(layers_q):
        copy = make_cache_from(ks, vs, 3000, W.BF16)
        assert np.array_equal(to_stored(y.cross_attn_decode(ql, copy)), out_shared[l])
    # and the layers differ from one another (shared storage, not shared results)
    assert not np.array_equal(out_shared[0], out_shared[1])


def test_decode_row_permutation_invariance():
    ks, vs, q = _decode_case(W.BF16, 128, 24, 8, [2048], seed=5)
    perm = rng(6).permutation(2048)
    a = to_stored(y.cross_attn_decode(to_dev(q), make_cache_from(ks, vs, 2048, W.BF16)))
    b = to_stored(y.cross_attn_decode(to_dev(q), make_cache_from([ks[0][perm]], [vs[0][perm]], 2048, W.BF16)))
    assert_parity(a, b, bf16=True, what="row permutation")


def test_decode_single_row_returns_v0():
    ks, vs, q = _decode_case(W.BF16, 128, 24, 8, [1], seed=7)
    o = to_stored(y.cross_attn_decode(to_dev(q), make_cache_from(ks, vs, 16, W.BF16)))
    want = np.repeat(W.as_f32(vs[0][0]), 3, axis=0)      # head h reads KV head h // 3
    assert np.array_equal(o[0], want)


# ---------------------------------------------------------------------------
# Prefill
# ---------------------------------------------------------------------------
PREFILL_CASES = [
    # (dtype, dh, hq, hkv, n_rows, q_start, t)
    (W.BF16, 128, 6, 2, 300, 0, 300),
    (W.BF16, 128, 24, 8, 520, 0, 520),
    (W.BF16, 64, 4, 4, 700, 200, 500),
    (W.BF16, 128, 3, 1, 1000, 999, 1),
    (W.BF16, 64, 8, 2, 129, 0, 129),
    (W.BF16, 128, 4, 2, 900, 250, 130),
    (W.BF16, 128, 12, 2, 333, 0, 333),      # group of 6
    (W.BF16, 128, 48, 8, 300, 40, 260),     # group of 6 at 8 KV heads
    (W.BF16, 128, 8, 1, 290, 30, 260),      # group of 8
    (W.BF16, 64, 16, 2, 515, 0, 515),       # group of 8, head_dim 64
    (W.F32, 64, 4, 2, 300, 0, 300),
    (W.F32, 128, 2, 2, 200, 50, 100),
]


@pytest.mark.parametrize("dtype,dh,hq,hkv,n,q_start,t", PREFILL_CASES)
def test_prefill_parity(dtype, dh, hq, hkv, n, q_start, t):
    c = W.make_prefill(n=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=dh, dtype=dtype,
                       q_start=q_start, t=t, seed=11)
    cache = make_cache_from([c.k], [c.v], n + 3, dtype)
    canary = float("nan")
    o_buf = torch.full((t + 2, hq, dh), canary, dtype=torch.float32, device="cuda")
    o, lse = y.cross_attn_prefill(to_dev(c.q), cache, q_start=q_start, out=o_buf[:t], want_lse=True)
    assert torch.isnan(o_buf[t:]).all(), "prefill wrote past its output rows"
    ro, rl = orc().prefill(c.q, q_start, c.k, c.v, c.softmax_scale, want_lse=True)
    assert_parity(to_stored(o), ro, bf16=(dtype == W.BF16), what="prefill O")
    assert_parity(to_stored(lse), rl, bf16=(dtype == W.BF16), what="prefill lse")


def test_prefill_bf16_output():
    c = W.make_prefill(n=400, n_q_heads=8, n_kv_heads=2, head_dim=128, seed=12)
    cache = make_cache_from([c.k], [c.v], 400, W.BF16)
    o = y.cross_attn_prefill(to_dev(c.q), cache, out_dtype=torch.bfloat16)
    assert o.dtype == torch.bfloat16
    ro = orc().prefill(c.q, 0, c.k, c.v, c.softmax_scale)
    # bf16 output rounding adds up to half an ulp on top of the fp32 error
    assert_parity(W.as_f32(to_stored(o)), ro, bf16=True, what="prefill O (bf16 store)")


def test_prefill_first_row_is_v0_exactly():
    c = W.make_prefill(n=256, n_q_heads=6, n_kv_heads=2, head_dim=128, seed=13)
    cache = make_cache_from([c.k], [c.v], 256, W.BF16)
    o = to_stored(y.cross_attn_prefill(to_dev(c.q), cache))
    want = np.repeat(W.as_f32(c.v[0]), 3, axis=0)
    assert np.array_equal(o[0], want)


def test_prefill_prefix_invariance_bitwise():
    c = W.make_prefill(n=640, n_q_heads=6, n_kv_heads=2, head_dim=128, seed=14)
    full = make_cache_from([c.k], [c.v], 640, W.BF16)
    o_full = to_stored(y.cross_attn_prefill(to_dev(c.q), full))
    short = make_cache_from([c.k[:300]], [c.v[:300]], 640, W.BF16)
    o_short = to_stored(y.cross_attn_prefill(to_dev(c.q[:300]), short))
    assert np.array_equal(o_short, o_full[:300])


def _overflow_case(n, hot_key, hot_row, hot_head, scale=6.0, seed=16):
    """Prefill input where query (hot_row, hot_head) meets key hot_key with a
    logit of about scale*|q|^2/sqrt(128) ~ 68 (98 in log2 units), far above
    the maximum over its first 32 keys: the kernel's fixed reference must
    give way to its second pass.  The key row is stored in bf16 like the
    rest, and the oracle reads the same stored values."""
    c = W.make_prefill(n=n, n_q_heads=6, n_kv_heads=2, head_dim=128, seed=seed)
    q = W.as_f32(c.q)
    k = W.as_f32(c.k)
    g = hot_head // 3
    k[hot_key, g] = np.float32(scale) * q[hot_row, hot_head]
    c.k = W.store(k, W.BF16)
    return c


def test_prefill_overflow_second_pass():
    c = _overflow_case(n=600, hot_key=300, hot_row=310, hot_head=3)
    s_hot = float(W.as_f32(c.q)[310, 3] @ W.as_f32(c.k)[300, 1]) * c.softmax_scale
    assert s_hot / np.log(2.0) > 64 + 16, "the planted logit must exceed the overflow margin"
    cache = make_cache_from([c.k], [c.v], 600, W.BF16)
    o, lse = y.cross_attn_prefill(to_dev(c.q), cache, want_lse=True)
    ro, rl = orc().prefill(c.q, 0, c.k, c.v, c.softmax_scale, want_lse=True)
    assert_parity(to_stored(o), ro, bf16=True, what="prefill O with an overflowing row")
    assert_parity(to_stored(lse), rl, bf16=True, what="prefill lse with an overflowing row")
    # the hot row attends almost only to the hot key
    assert np.abs(to_stored(o)[310, 3] - W.as_f32(c.v)[300, 1]).max() < 2e-2


def test_prefill_overflow_keeps_other_rows_bitwise():
    # Rows 256..299 share a workgroup with the overflowing row 510 only in
    # the full run; their results must not change.
    c = _overflow_case(n=640, hot_key=500, hot_row=510, hot_head=0)
    full = make_cache_from([c.k], [c.v], 640, W.BF16)
    o_full = to_stored(y.cross_attn_prefill(to_dev(c.q), full))
    short = make_cache_from([c.k[:300]], [c.v[:300]], 640, W.BF16)
    o_short = to_stored(y.cross_attn_prefill(to_dev(c.q[:300]), short))
    assert np.array_equal(o_short, o_full[:300])
    ro = orc().prefill(c.q, 0, c.k, c.v, c.softmax_scale, rows=[509, 510, 511])
    assert_parity(o_full[509:512], ro, bf16=True, what="rows around the overflowing row")


def test_decode_matches_last_prefill_row():
    c = W.make_prefill(n=1000, n_q_heads=24, n_kv_heads=8, head_dim=128, seed=15)
    cache = make_cache_from([c.k], [c.v], 1000, W.BF16)
    o_pre = to_stored(y.cross_attn_prefill(to_dev(c.q), cache))
    o_dec = to_stored(y.cross_attn_decode(to_dev(c.q[-1:]), cache))
    assert_parity(o_dec[0], o_pre[-1], bf16=True, what="decode vs last prefill row")


# ---------------------------------------------------------------------------
# Projections
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,n,d", [(W.BF16, 130, 3072), (W.BF16, 64, 256), (W.F32, 70, 512)])
def test_kv_project_parity(dtype, n, d):
    p = W.make_project(n=n, d_model=d, dtype=dtype, unit_gain=False, seed=21)
    tdt = torch.bfloat16 if dtype == W.BF16 else torch.float32
    cache = y.KVCache(2, n + 40, 8, 128, tdt)
    cache.k.fill_(7.0)
    cache.v.fill_(7.0)
    cache.len[:] = [0, 10]
    gain = torch.from_numpy(p.gain).cuda()
    y.kv_project(cache, to_dev(p.m), to_dev(p.w_k), to_dev(p.w_v), gain, p.eps, seq=1, row_start=20)
    assert cache.len.tolist() == [0, 20 + n]
    k = to_stored(cache.k[1, 20:20 + n]).reshape(n, -1)
    v = to_stored(cache.v[1, 20:20 + n]).reshape(n, -1)
    rk = orc().project(p.m, p.w_k, p.gain, p.eps)
    rv = orc().project(p.m, p.w_v, p.gain, p.eps)
    if dtype == W.BF16:
        ynorm = np.abs(orc().rmsnorm(p.m, p.gain, p.eps))
        assert_projection_bf16(k, rk, ynorm @ np.abs(W.as_f32(p.w_k).astype(np.float64)), d, "K^")
        assert_projection_bf16(v, rv, ynorm @ np.abs(W.as_f32(p.w_v).astype(np.float64)), d, "V^")
    else:
        assert_parity(k, rk, bf16=False, what="K^")
        assert_parity(v, rv, bf16=False, what="V^")
    # guard bands: nothing else in the cache was touched
    assert torch.all(cache.k[0] == 7.0) and torch.all(cache.k[1, :20] == 7.0)
    assert torch.all(cache.v[1, 20 + n:] == 7.0)


@pytest.mark.parametrize("n,d,hkv,dh,unit_gain", [
    (600, 256, 2, 128, True),     # 3 row tiles with a ragged tail, unit gain (NULL)
    (600, 256, 2, 128, False),    # same rows, fp32 gain (hi/lo split)
    (257, 1024, 4, 64, False),    # one full row tile plus one row
    (300, 128, 2, 128, False),    # d_model 128: four reduction slices, one pass of the staging ring
    (40, 384, 2, 128, True),      # d_model 384: three passes; fewer rows than one tile
    (96, 192, 2, 128, False),     # d_model % 128 != 0: the fp32-FMA tiled kernel
])
def test_prompt_projection_paths(n, d, hkv, dh, unit_gain):
    """Prompt-sized bf16 projections run on the matrix cores when d_model is a
    multiple of 128 and the columns a multiple of 256, else on the fp32-FMA
    tiled kernel; both meet the same bound."""
    p = W.make_project(n=n, d_model=d, n_kv_heads=hkv, head_dim=dh, unit_gain=unit_gain, seed=25)
    cache = y.KVCache(2, n + 9, hkv, dh, torch.bfloat16)
    cache.k.fill_(7.0)
    cache.v.fill_(7.0)
    gain = None if unit_gain else torch.from_numpy(p.gain).cuda()
    y.kv_project(cache, to_dev(p.m), to_dev(p.w_k), to_dev(p.w_v), gain, p.eps, seq=1, row_start=5)
    g = None if unit_gain else p.gain
    ynorm = np.abs(orc().rmsnorm(p.m, g, p.eps))
    for got, w, name in ((cache.k, p.w_k, "K^"), (cache.v, p.w_v, "V^")):
        stored = to_stored(got[1, 5:5 + n]).reshape(n, -1)
        ref = orc().project(p.m, w, g, p.eps)
        assert_projection_bf16(stored, ref, ynorm @ np.abs(W.as_f32(w).astype(np.float64)), d, name)
        assert torch.all(got[0] == 7.0) and torch.all(got[1, :5] == 7.0) and torch.all(got[1, 5 + n:] == 7.0)


def test_q_project_prompt_mfma():
    r = rng(26)
    x = W.store(r.standard_normal((300, 512)).astype(np.float32), W.BF16)
    wq = W.store((r.standard_normal((512, 8 * 64)) / math.sqrt(512)).astype(np.float32), W.BF16)
    gain = (0.5 + r.random(512)).astype(np.float32)
    q = y.q_project(to_dev(x), to_dev(wq), 8, 64, gain=torch.from_numpy(gain).cuda(), eps=1e-5)
    abs_terms = np.abs(orc().rmsnorm(x, gain, 1e-5)) @ np.abs(W.as_f32(wq).astype(np.float64))
    assert_projection_bf16(to_stored(q).reshape(300, -1), orc().project(x, wq, gain, 1e-5), abs_terms, 512, "Q^")


def test_append_matches_project_and_advances_lengths():
    p = W.make_project(n=3, d_model=3072, seed=22)
    cache = y.KVCache(3, 50, 8, 128, torch.bfloat16)
    cache.k.fill_(7.0)
    cache.len[:] = [0, 17, 49]
    m = to_dev(p.m)
    y.kv_append(cache, m, to_dev(p.w_k), to_dev(p.w_v))
    assert cache.len.tolist() == [1, 18, 50]
    ref = y.KVCache(1, 3, 8, 128, torch.bfloat16)
    y.kv_project(ref, m, to_dev(p.w_k), to_dev(p.w_v))
    for b, row in enumerate([0, 17, 49]):
        assert torch.equal(cache.k[b, row], ref.k[0, b])
        assert torch.equal(cache.v[b, row], ref.v[0, b])
    assert torch.all(cache.k[1, 18:] == 7.0) and torch.all(cache.k[0, 1:] == 7.0)
    with pytest.raises(y.YocoError):
        y.kv_append(cache, m, to_dev(p.w_k), to_dev(p.w_v))   # sequence 2 is full
    assert cache.len.tolist() == [1, 18, 50]


def test_q_project_bf16_parity():
    r = rng(23)
    x = W.store(r.standard_normal((33, 3072)).astype(np.float32), W.BF16)
    wq = W.store((r.standard_normal((3072, 24 * 128)) / math.sqrt(3072)).astype(np.float32), W.BF16)
    q = y.q_project(to_dev(x), to_dev(wq), 24, 128)
    assert q.shape == (33, 24, 128) and q.dtype == torch.bfloat16
    abs_terms = np.abs(orc().rmsnorm(x)) @ np.abs(W.as_f32(wq).astype(np.float64))
    assert_projection_bf16(to_stored(q).reshape(33, -1), orc().project(x, wq), abs_terms, 3072, "Q^")


@pytest.mark.parametrize("split_rows", [True, False], ids=["split-W", "strips"])
@pytest.mark.parametrize("dtype,n,d", [(W.BF16, 1, 3072), (W.BF16, 5, 3072), (W.BF16, 13, 3072),
                                       (W.BF16, 16, 3072), (W.F32, 1, 256), (W.F32, 8, 256),
                                       (W.F32, 30, 512), (W.BF16, 3, 8192), (W.BF16, 32, 200)])
def test_small_row_projection_parity(dtype, n, d, split_rows):
    """Few-row projections (generation-time append and per-token queries), in
    launches of up to 8 rows: with a workspace on the kernel that splits W's
    rows over the whole chip, without one on the column-strip kernel."""
    p = W.make_project(n=n, d_model=d, dtype=dtype, unit_gain=False, seed=24)
    tdt = torch.bfloat16 if dtype == W.BF16 else torch.float32
    cache = y.KVCache(1, n + 7, 8, 128, tdt)
    cache.k.fill_(7.0)
    cache.v.fill_(7.0)
    y.kv_project(cache, to_dev(p.m), to_dev(p.w_k), to_dev(p.w_v), torch.from_numpy(p.gain).cuda(), p.eps,
                 row_start=3, workspace=None if split_rows else False)
    k = to_stored(cache.k[0, 3:3 + n]).reshape(n, -1)
    v = to_stored(cache.v[0, 3:3 + n]).reshape(n, -1)
    rk = orc().project(p.m, p.w_k, p.gain, p.eps)
    rv = orc().project(p.m, p.w_v, p.gain, p.eps)
    if dtype == W.BF16:
        ynorm = np.abs(orc().rmsnorm(p.m, p.gain, p.eps))
        assert_projection_bf16(k, rk, ynorm @ np.abs(W.as_f32(p.w_k).astype(np.float64)), d, "K^")
        assert_projection_bf16(v, rv, ynorm @ np.abs(W.as_f32(p.w_v).astype(np.float64)), d, "V^")
    else:
        assert_parity(k, rk, bf16=False, what="K^")
        assert_parity(v, rv, bf16=False, what="V^")
    assert torch.all(cache.k[0, :3] == 7.0) and torch.all(cache.k[0, 3 + n:] == 7.0)


def test_q_project_single_token():
    r = rng(25)
    x = W.store(r.standard_normal((1, 3072)).astype(np.float32), W.BF16)
    wq = W.store((r.standard_normal((3072, 24 * 128)) / math.sqrt(3072)).astype(np.float32), W.BF16)
    gain = (1 + 0.1 * r.standard_normal(3072)).astype(np.float32)
    q = y.q_project(to_dev(x), to_dev(wq), 24, 128, torch.from_numpy(gain).cuda(), out_dtype=torch.float32)
    assert_parity(to_stored(q).reshape(1, -1), orc().project(x, wq, gain), bf16=False, what="Q^ (fp32 out)")


def test_decode_and_append_at_the_sequence_limit():
    """YOCO_MAX_SEQ (256) sequences of mixed lengths 1..600: one appended row
    per sequence, then a decode step of every sequence against the oracle."""
    print("decode + append, 256 sequences", flush=True)
    n_seq, hkv, dh, hq, d = 256, 2, 64, 6, 128
    r = rng(77)
    lens = r.integers(1, 600, n_seq)
    lens[0], lens[1] = 1, 0  # a one-row slab and an empty one that the append fills
    ks = [W.store(r.standard_normal((max(L, 1), hkv, dh)).astype(np.float32), W.BF16) for L in lens]
    vs = [W.store(r.standard_normal((max(L, 1), hkv, dh)).astype(np.float32), W.BF16) for L in lens]
    cache = make_cache_from(ks, vs, 640, W.BF16)
    cache.len[:] = lens
    m_new = W.store(r.standard_normal((n_seq, d)).astype(np.float32), W.BF16)
    w_k = W.store((r.standard_normal((d, hkv * dh)) / math.sqrt(d)).astype(np.float32), W.BF16)
    w_v = W.store((r.standard_normal((d, hkv * dh)) / math.sqrt(d)).astype(np.float32), W.BF16)
    y.kv_append(cache, to_dev(m_new), to_dev(w_k), to_dev(w_v))
    assert cache.len.tolist() == (lens + 1).tolist()
    q = W.store(r.standard_normal((n_seq, hq, dh)).astype(np.float32), W.BF16)
    o = to_stored(y.cross_attn_decode(to_dev(q), cache, 1 / math.sqrt(dh)))
    k_all = to_stored(cache.k)
    v_all = to_stored(cache.v)
    new_k = orc().project(m_new, w_k, None, 1e-6).reshape(n_seq, hkv, dh)
    for b in range(n_seq):
        L = int(lens[b]) + 1
        kb, vb = k_all[b, :L], v_all[b, :L]
        assert_projection_bf16(kb[L - 1].reshape(1, -1), new_k[b].reshape(1, -1),
                               np.abs(orc().rmsnorm(m_new[b:b + 1])) @ np.abs(as_f32(w_k).astype(np.float64)),
                               d, what=f"appended K^ row of sequence {b}")
        ro = orc().decode(q[b:b + 1], L, kb, vb, 1 / math.sqrt(dh))
        assert_parity(o[b], ro[0], bf16=True, what=f"decode seq {b} len {L}")
