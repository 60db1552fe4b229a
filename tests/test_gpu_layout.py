"""Padded cache rows (row_stride > n_kv_heads * head_dim) against dense rows.

The row stride only moves rows in memory, so every entry point must give
bitwise the same results on a padded cache as on a dense one, and must never
write (or let a result depend on) the padding.  The padding is filled with
NaN before anything runs: a kernel that read it would turn its output NaN,
one that wrote it would overwrite the NaN."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

y = pytest.importorskip("yoco_shared_kv_amd")


def _caches(n_seq, cap, hkv, dh, dtype):
    dense = y.KVCache(n_seq, cap, hkv, dh, dtype, zero=True, padded=False)
    padded = y.KVCache(n_seq, cap, hkv, dh, dtype, zero=True, padded=True)
    assert padded.row_stride > hkv * dh and dense.row_stride == hkv * dh
    for c in (padded,):
        c._k_rows[..., hkv * dh:] = float("nan")
        c._v_rows[..., hkv * dh:] = float("nan")
    return dense, padded


def _padding_untouched(c):
    dense = c.n_kv_heads * c.head_dim
    return bool(torch.isnan(c._k_rows[..., dense:]).all() and torch.isnan(c._v_rows[..., dense:]).all())


@pytest.mark.parametrize("dtype,n,d", [(torch.bfloat16, 1000, 512), (torch.float32, 300, 256)])
def test_padded_rows_give_identical_results(dtype, n, d):
    print(f"layout: {dtype} n={n} d={d}", flush=True)
    hkv, dh, hq = 8, 128, 24
    wdt = W.BF16 if dtype == torch.bfloat16 else W.F32
    pc = W.make_project(n=n + 1, d_model=d, n_kv_heads=hkv, head_dim=dh, dtype=wdt, unit_gain=False)
    m, wk, wv = to_dev(pc.m), to_dev(pc.w_k), to_dev(pc.w_v)
    gain = torch.from_numpy(pc.gain).cuda()
    dense, padded = _caches(1, n + 5, hkv, dh, dtype)
    outs = {}
    for name, c in (("dense", dense), ("padded", padded)):
        y.kv_project(c, m[:n], wk, wv, gain, pc.eps)
        y.kv_append(c, m[n:n + 1], wk, wv, gain, pc.eps)
        rng = np.random.default_rng(4)
        q = to_dev(W.store(rng.standard_normal((n + 1, hq, dh)).astype(np.float32), wdt))
        o_pre = y.cross_attn_prefill(q, c)
        o_dec = y.cross_attn_decode(q[n:n + 1], c)
        outs[name] = (c.k[0, :n + 1].clone(), c.v[0, :n + 1].clone(), o_pre, o_dec)
        if dtype == torch.bfloat16:
            o_b, lse = y.cross_attn_prefill(q, c, want_lse=True)
            d_o = to_dev(W.store(rng.standard_normal((n + 1, hq, dh)).astype(np.float32), W.BF16))
            grads = y.cross_attn_prefill_bwd(q, o_b, d_o, lse, c)
            outs[name] += tuple(grads)
    torch.cuda.synchronize()
    assert _padding_untouched(padded), "a kernel wrote into the row padding"
    for a, b in zip(outs["dense"], outs["padded"]):
        assert torch.isfinite(b).all()
        assert torch.equal(a, b)


def test_padded_rows_multi_sequence_decode_and_append():
    """Several sequences of different lengths: the slab stride is
    capacity * row_stride."""
    print("layout: 3 sequences", flush=True)
    hkv, dh, hq, d = 8, 128, 24, 256
    pc = W.make_project(n=3, d_model=d, n_kv_heads=hkv, head_dim=dh, dtype=W.BF16, unit_gain=False)
    m, wk, wv = to_dev(pc.m), to_dev(pc.w_k), to_dev(pc.w_v)
    dense, padded = _caches(3, 700, hkv, dh, torch.bfloat16)
    rng = np.random.default_rng(9)
    lens = [650, 1, 299]
    for b, L in enumerate(lens):
        kv = to_dev(W.store(rng.standard_normal((2, L, hkv, dh)).astype(np.float32), W.BF16))
        for c in (dense, padded):
            c.k[b, :L] = kv[0]
            c.v[b, :L] = kv[1]
            c.len[b] = L
    q = to_dev(W.store(rng.standard_normal((3, hq, dh)).astype(np.float32), W.BF16))
    res = []
    for c in (dense, padded):
        y.kv_append(c, m, wk, wv)
        res.append((y.cross_attn_decode(q, c), c.k.clone(), c.v.clone()))
    torch.cuda.synchronize()
    assert _padding_untouched(padded)
    for a, b in zip(*res):
        assert torch.equal(a, b)
