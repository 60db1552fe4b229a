"""RMSNorm gain folded into the projection weights ([Notes] "YOCO：You Only
Cache Once 中文精读笔记" s.2.1 Eq. 2-3: LN(x) W = (x / r) (diag(g) W)).

* The fold itself against its definition, bit for bit: each weight is the
  fp32 product g[c] * w[c][j] rounded once to bf16 (round to nearest even),
  on the vector path (rows a multiple of 8 wide), the one-element path,
  fp32 and bf16 weights, and in place.
* Projections given folded weights and no gain against the fp64 oracle run
  with the ORIGINAL gain and weights (the method's result; the bf16 rounding
  of g*w is the only difference, so the bf16 tolerance applies), and against
  the oracle run with the folded weights and unit gain (the tight one-ulp
  bound of every bf16 projection: the kernels add nothing of their own).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_parity, assert_projection_bf16, metrics, to_dev, to_stored

pytestmark = pytest.mark.gpu

y = pytest.importorskip("yoco_shared_kv_amd")

ORC = None


def orc():
    global ORC
    if ORC is None:
        ORC = oracle.default()
    return ORC


def _fold_bits(w_stored: np.ndarray, gain: np.ndarray) -> np.ndarray:
    """RNE_bf16(fp32(w) * g) as bf16 bits (IEEE fp32 product; finite or inf)."""
    prod = (W.as_f32(w_stored).astype(np.float32) * gain.astype(np.float32)[:, None]).astype(np.float32)
    u = prod.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _gain(d: int, seed: int) -> np.ndarray:
    g = (1.0 + 0.1 * np.random.default_rng(seed).standard_normal(d)).astype(np.float32)
    # a zero channel, a sign flip, a product in the fp32 subnormal range, one
    # that overflows to inf
    g[0], g[1], g[2] = 0.0, -1.5, 1e-39
    if d > 3:
        g[3] = 3e38
    return g


@pytest.mark.parametrize("d,ncols,dtype", [
    (3072, 1024, W.BF16),   # the 3B K^/V^ weights: vector path
    (512, 256, W.F32),      # fp32 weights
    (96, 100, W.BF16),      # rows not a multiple of 8: one element per lane
    (7, 13, W.F32),
])
def test_fold_matches_its_definition(d, ncols, dtype):
    r = np.random.default_rng(41)
    w = W.store((r.standard_normal((d, ncols)) * 3.0).astype(np.float32), dtype)
    g = _gain(d, 42)
    got = y.fold_norm_gain(to_dev(w), torch.from_numpy(g).cuda())
    assert got.dtype == torch.bfloat16 and tuple(got.shape) == (d, ncols)
    want = _fold_bits(w, g)
    bits = to_stored(got)
    assert np.array_equal(bits, want), f"{int(np.sum(bits != want))} of {want.size} folded weights differ"


def test_fold_in_place_equals_out_of_place():
    r = np.random.default_rng(43)
    w = to_dev(W.store(r.standard_normal((256, 512)).astype(np.float32), W.BF16))
    g = torch.from_numpy(_gain(256, 44)).cuda()
    out = y.fold_norm_gain(w, g)
    w2 = w.clone()
    ret = y.fold_norm_gain(w2, g, out=w2)
    assert ret.data_ptr() == w2.data_ptr()
    assert torch.equal(w2.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("n,d,hkv,dh", [
    (600, 384, 2, 128),     # matrix cores: three row tiles with a ragged tail
    (4096, 3072, 8, 128),   # one early-exit chunk at the 3B widths
    (1, 3072, 8, 128),      # the one-row path (split over W's rows)
])
def test_folded_projection_matches_the_gained_oracle(n, d, hkv, dh):
    p = W.make_project(n=n, d_model=d, n_kv_heads=hkv, head_dim=dh, unit_gain=False, seed=45)
    g = torch.from_numpy(p.gain).cuda()
    wk_f = y.fold_norm_gain(to_dev(p.w_k), g)
    wv_f = y.fold_norm_gain(to_dev(p.w_v), g)
    cache = y.KVCache(1, n + 3, hkv, dh, torch.bfloat16)
    cache.k.fill_(7.0)
    cache.v.fill_(7.0)
    y.kv_project(cache, to_dev(p.m), wk_f, wv_f, None, p.eps, row_start=2)
    rows = np.arange(n) if n <= 600 else np.unique(np.r_[0, 1, n - 1, np.random.default_rng(46).choice(n, 200)])
    ynorm = np.abs(orc().rmsnorm(p.m[rows], None, p.eps))
    for got, w, wf, name in ((cache.k, p.w_k, wk_f, "K^"), (cache.v, p.w_v, wv_f, "V^")):
        stored = to_stored(got[0, torch.as_tensor(2 + rows, device=got.device)]).reshape(rows.size, -1)
        # the method's result: the oracle with the original gain and weights
        max_abs, rel = assert_parity(W.as_f32(stored), orc().project(p.m[rows], w, p.gain, p.eps), bf16=True,
                                     what=f"{name} folded vs gained oracle")
        print(f"{name} n={n}: folded weights vs the gained fp64 oracle: max-abs {max_abs:.2e}, rel-L2 {rel:.2e}")
        # what the kernels compute: the unit-gain projection of the folded weights
        wf_bits = to_stored(wf)
        ref = orc().project(p.m[rows], wf_bits, None, p.eps)
        assert_projection_bf16(stored, ref, ynorm @ np.abs(W.as_f32(wf_bits).astype(np.float64)), d,
                               f"{name} folded, unit gain")
        assert torch.all(got[0, :2] == 7.0) and torch.all(got[0, 2 + n:] == 7.0)


def test_folded_query_projection_one_row_and_prompt():
    r = np.random.default_rng(47)
    d, hq, dh = 3072, 24, 128
    wq = W.store((r.standard_normal((d, hq * dh)) / math.sqrt(d)).astype(np.float32), W.BF16)
    g = (0.5 + r.random(d)).astype(np.float32)
    wq_f = y.fold_norm_gain(to_dev(wq), torch.from_numpy(g).cuda())
    for n in (1, 300):
        x = W.store(r.standard_normal((n, d)).astype(np.float32), W.BF16)
        q = to_stored(y.q_project(to_dev(x), wq_f, hq, dh, eps=1e-5)).reshape(n, -1)
        max_abs, rel = metrics(W.as_f32(q), orc().project(x, wq, g, 1e-5))
        assert max_abs <= 2e-2 and rel <= 5e-3, f"Q^ n={n}: max-abs {max_abs:.2e}, rel-L2 {rel:.2e}"
