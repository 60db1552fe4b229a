"""The decode that allocates nothing (yoco_cross_attn_decode_noalloc, for
callers that cannot allocate) against yoco_cross_attn_decode with a
caller's workspace: the same bits for the same cache, query, scale and split
size, on two calls in a row, the second with smaller inputs (fewer sequences,
shorter caches, another split size), and a third back on the first shape."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

y = pytest.importorskip("yoco_shared_kv_amd")


def _case(n_seq, lens, hkv, hq, dh, seed):
    r = np.random.default_rng(seed)
    cache = y.KVCache(n_seq, max(lens) + 3, hkv, dh, torch.bfloat16)
    for b, L in enumerate(lens):
        cache.k[b, :L] = to_dev(W.store(r.standard_normal((L, hkv, dh)).astype(np.float32), W.BF16))
        cache.v[b, :L] = to_dev(W.store(r.standard_normal((L, hkv, dh)).astype(np.float32), W.BF16))
        cache.len[b] = L
    q = to_dev(W.store(r.standard_normal((n_seq, hq, dh)).astype(np.float32), W.BF16))
    return cache, q


def _both(cache, q, rows_per_split):
    n_seq, hq, dh = q.shape
    scale = 1.0 / math.sqrt(dh)
    ref, ref_lse = y.cross_attn_decode(q, cache, scale, rows_per_split=rows_per_split, want_lse=True)
    out = torch.full((n_seq, hq, dh), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((n_seq, hq), float("nan"), dtype=torch.float32, device="cuda")
    y.cross_attn_decode_noalloc(q, cache, out, scale, rows_per_split=rows_per_split, lse_out=lse)
    torch.cuda.synchronize()
    return ref, ref_lse, out, lse


def test_noalloc_decode_matches_the_workspace_decode_bitwise():
    print("no-alloc decode: 3 sequences x 24/8 heads, then 1 sequence x 8/8 heads, then the first again",
          flush=True)
    big = _case(3, [70000, 5000, 131], 8, 24, 128, seed=91)
    small = _case(1, [2049], 8, 8, 128, seed=92)
    for (cache, q), rows in ((big, 0), (small, 256), (big, 512)):
        ref, ref_lse, out, lse = _both(cache, q, rows)
        assert torch.equal(out, ref), "output differs from the workspace decode"
        assert torch.equal(lse, ref_lse), "lse differs from the workspace decode"
        assert bool(torch.isfinite(out).all())


def test_noalloc_decode_head_dim_64_and_fp32_cache():
    r = np.random.default_rng(93)
    cache = y.KVCache(2, 900, 2, 64, torch.float32)
    for b, L in enumerate([900, 17]):
        cache.k[b, :L] = torch.from_numpy(r.standard_normal((L, 2, 64)).astype(np.float32)).cuda()
        cache.v[b, :L] = torch.from_numpy(r.standard_normal((L, 2, 64)).astype(np.float32)).cuda()
        cache.len[b] = L
    q = torch.from_numpy(r.standard_normal((2, 8, 64)).astype(np.float32)).cuda()
    ref, ref_lse, out, lse = _both(cache, q, 256)
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
