"""The cross-decoder's share of prefill with early exit, composed from the
boundary's calls ([Notes] "YOCO：You Only Cache Once 中文精读笔记" s.2.5 and
[Blog] "NeurIPS'24 | YOCO: 长上下文 LLM 为什么不必每层都存一份 KV Cache?"
s.6-7: the prompt's history positions only write K^/V^ into the cache, and
only the last prompt token runs the cross layers):

* chunked projection: K^/V^ of a prompt written chunk by chunk (row_start)
  equals the one-shot projection bitwise;
* chunked prefill (training forward in query chunks, q_start > 0) equals the
  one-shot prefill bitwise;
* the early-exit pipeline (chunked projection of rows 0..N-2, append of row
  N-1, then per cross layer a query projection and one decode at position
  N-1) matches the fp64 oracle and the last row of the full prefill.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_parity, to_dev, to_stored

pytestmark = pytest.mark.gpu

y = pytest.importorskip("yoco_shared_kv_amd")


def _chunks(n, size):
    return [(s, min(s + size, n)) for s in range(0, n, size)]


def test_chunked_kv_project_equals_one_shot():
    p = W.make_project(n=5000, d_model=1024, n_kv_heads=4, head_dim=128, unit_gain=False, seed=31)
    m, w_k, w_v = to_dev(p.m), to_dev(p.w_k), to_dev(p.w_v)
    gain = torch.from_numpy(p.gain).cuda()
    one = y.KVCache(1, 5000, 4, 128, torch.bfloat16, zero=True)
    y.kv_project(one, m, w_k, w_v, gain, p.eps)
    chunked = y.KVCache(1, 5000, 4, 128, torch.bfloat16, zero=True)
    for s, e in _chunks(5000, 1536):                  # 3 full chunks and a ragged one
        y.kv_project(chunked, m[s:e], w_k, w_v, gain, p.eps, row_start=s)
    assert chunked.len.tolist() == [5000]
    assert torch.equal(chunked.k, one.k) and torch.equal(chunked.v, one.v)


@pytest.mark.parametrize("with_gain", [True, False])
def test_wide_and_narrow_projection_tiles_agree_bitwise(with_gain):
    """16300 rows take 256-column tiles (512 tiles); 2048-row chunks take
    128-column tiles (64 tiles, fewer than the CUs), the last chunk ragged.
    The wave tiles differ with and without a gain, but each output element
    sees the same products in the same order, so the caches agree bitwise."""
    n = 16300
    print(f"pipeline: wide vs narrow tiles, gain={with_gain}", flush=True)
    p = W.make_project(n=n, d_model=1024, n_kv_heads=8, head_dim=128, unit_gain=False, seed=33)
    m, w_k, w_v = to_dev(p.m), to_dev(p.w_k), to_dev(p.w_v)
    gain = torch.from_numpy(p.gain).cuda() if with_gain else None
    wide = y.KVCache(1, n, 8, 128, torch.bfloat16, zero=True)
    y.kv_project(wide, m, w_k, w_v, gain, p.eps)
    narrow = y.KVCache(1, n, 8, 128, torch.bfloat16, zero=True)
    for s, e in _chunks(n, 2048):
        y.kv_project(narrow, m[s:e], w_k, w_v, gain, p.eps, row_start=s)
    assert torch.equal(wide.k, narrow.k) and torch.equal(wide.v, narrow.v)


def test_chunked_prefill_equals_one_shot():
    c = W.make_prefill(n=2000, n_q_heads=6, n_kv_heads=2, head_dim=128, seed=32)
    cache = y.KVCache(1, 2000, 2, 128, torch.bfloat16)
    cache.k[0] = to_dev(c.k)
    cache.v[0] = to_dev(c.v)
    cache.len[0] = 2000
    q = to_dev(c.q)
    one, lse_one = y.cross_attn_prefill(q, cache, want_lse=True)
    parts, lses = [], []
    for s, e in _chunks(2000, 700):
        o, lse = y.cross_attn_prefill(q[s:e], cache, q_start=s, want_lse=True)
        parts.append(o)
        lses.append(lse)
    assert torch.equal(torch.cat(parts), one) and torch.equal(torch.cat(lses), lse_one)


def test_early_exit_prefill_pipeline():
    n, d, hq, hkv, dh, layers = 3000, 1024, 8, 2, 128, 4
    r = np.random.default_rng(33)
    # self-decoder output M for the whole prompt, and each cross layer's input
    # for the last prompt token (synthetic: no trained model here)
    pm = W.make_project(n=n, d_model=d, n_kv_heads=hkv, head_dim=dh, unit_gain=False, seed=34)
    x_last = [W.store(r.standard_normal((1, d)).astype(np.float32), W.BF16) for _ in range(layers)]
    w_q = [W.store((r.standard_normal((d, hq * dh)) / math.sqrt(d)).astype(np.float32), W.BF16)
           for _ in range(layers)]
    gain = torch.from_numpy(pm.gain).cuda()
    m, w_k, w_v = to_dev(pm.m), to_dev(pm.w_k), to_dev(pm.w_v)

    cache = y.KVCache(1, n, hkv, dh, torch.bfloat16, zero=True)
    for s, e in _chunks(n - 1, 1024):                 # history positions: cache only
        y.kv_project(cache, m[s:e], w_k, w_v, gain, pm.eps, row_start=s)
    y.kv_append(cache, m[n - 1:n], w_k, w_v, gain, pm.eps)     # the last prompt token
    assert cache.len.tolist() == [n]
    ws = y.decode_workspace(cache, hq)
    outs, qs = [], []
    for l in range(layers):
        q = y.q_project(to_dev(x_last[l]), to_dev(w_q[l]), hq, dh)
        qs.append(to_stored(q))
        outs.append(to_stored(y.cross_attn_decode(q, cache, workspace=ws))[0])

    k_st, v_st = to_stored(cache.k[0]), to_stored(cache.v[0])
    scale = 1.0 / math.sqrt(dh)
    for l in range(layers):
        ref = oracle.decode(qs[l], n, k_st, v_st, scale)[0]
        assert_parity(outs[l], ref, bf16=True, what=f"early-exit layer {l}")
    # the same as the last row of a full prefill whose last query is layer 0's
    q_full = np.concatenate([W.store(r.standard_normal((n - 1, hq, dh)).astype(np.float32), W.BF16), qs[0]])
    o_full = to_stored(y.cross_attn_prefill(to_dev(q_full), cache))
    assert_parity(outs[0], o_full[-1], bf16=True, what="early exit vs full prefill last row")
