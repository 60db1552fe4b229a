"""Rotary position embedding on the projections against the fp64 oracle
(rope of the fp64 projection): K^ rotated at its cache row, V^ untouched, Q
at pos0 + r or at per-row positions, on every projection kernel (matrix
cores, fp32-FMA tiles, few-row matrix-vector), up to positions near 2^20
with the 1M-stage base (80M).

Bound for a rotated bf16 value: it mixes the two members of its pair, each
with the fp32 accumulation error of the projection, so the accumulation term
of element j sums both members' sum|y W|; the single-precision sine and
cosine (and the rotation's own roundings) add 2^-18 of that sum."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_parity, assert_projection_bf16, to_dev, to_stored

pytestmark = pytest.mark.gpu

y = pytest.importorskip("yoco_shared_kv_amd")

ROPE_SLACK = 2.0 ** -18


def _pair_terms(terms, head_dim):
    n = terms.shape[0]
    t = terms.reshape(n, -1, head_dim // 2, 2)
    return np.broadcast_to(t.sum(-1, keepdims=True), t.shape).reshape(n, -1)


def _check_rotated(stored, m, w, gain, eps, pos, theta, head_dim, d, what):
    g = gain
    ref = oracle.rope(oracle.project(m, w, g, eps), pos, theta, head_dim)
    terms = np.abs(oracle.rmsnorm(m, g, eps)) @ np.abs(W.as_f32(w).astype(np.float64))
    assert_projection_bf16(stored, ref, _pair_terms(terms, head_dim), d, what, rel_slack=ROPE_SLACK)


@pytest.mark.parametrize("n,d,hkv,dh,row_start,theta", [
    (600, 256, 2, 128, 1000, 640e3),      # matrix cores, 3 row tiles
    (300, 512, 4, 64, 7, 5e6),            # matrix cores, head_dim 64
    (96, 192, 2, 128, 33, 640e3),         # fp32-FMA tiles (d_model % 128 != 0)
    (5, 3072, 8, 128, 131_000, 5e6),      # few-row matrix-vector kernel
    (300, 256, 1, 128, 1_000_000, 80e6),  # positions near 2^20
])
def test_kv_project_rope(n, d, hkv, dh, row_start, theta):
    p = W.make_project(n=n, d_model=d, n_kv_heads=hkv, head_dim=dh, unit_gain=False, seed=41)
    cache = y.KVCache(1, row_start + n + 3, hkv, dh, torch.bfloat16)
    cache.k[0, row_start - 3:].fill_(7.0)
    cache.v[0, row_start - 3:].fill_(7.0)
    gain = torch.from_numpy(p.gain).cuda()
    y.kv_project(cache, to_dev(p.m), to_dev(p.w_k), to_dev(p.w_v), gain, p.eps, row_start=row_start,
                 rope_theta=theta)
    assert cache.len.tolist() == [row_start + n]
    k = to_stored(cache.k[0, row_start:row_start + n]).reshape(n, -1)
    v = to_stored(cache.v[0, row_start:row_start + n]).reshape(n, -1)
    _check_rotated(k, p.m, p.w_k, p.gain, p.eps, row_start + np.arange(n), theta, dh, d, "rotated K^")
    terms = np.abs(oracle.rmsnorm(p.m, p.gain, p.eps)) @ np.abs(W.as_f32(p.w_v).astype(np.float64))
    assert_projection_bf16(v, oracle.project(p.m, p.w_v, p.gain, p.eps), terms, d, "V^ (not rotated)")
    assert torch.all(cache.k[0, row_start - 3:row_start] == 7.0) and torch.all(cache.v[0, row_start + n:] == 7.0)


def test_kv_append_rope_positions_are_lengths():
    p = W.make_project(n=3, d_model=3072, seed=42)
    cache = y.KVCache(3, 50, 8, 128, torch.bfloat16)
    cache.len[:] = [0, 17, 49]
    y.kv_append(cache, to_dev(p.m), to_dev(p.w_k), to_dev(p.w_v), rope_theta=640e3)
    assert cache.len.tolist() == [1, 18, 50]
    k = np.stack([to_stored(cache.k[b, row]).reshape(-1) for b, row in enumerate([0, 17, 49])])
    _check_rotated(k, p.m, p.w_k, None, p.eps, np.array([0, 17, 49]), 640e3, 128, 3072, "appended K^")
    # position 0 is the identity: sequence 0's row equals the plain projection
    plain = y.KVCache(1, 3, 8, 128, torch.bfloat16)
    y.kv_project(plain, to_dev(p.m), to_dev(p.w_k), to_dev(p.w_v))
    assert torch.equal(cache.k[0, 0], plain.k[0, 0]) and torch.equal(cache.v[1, 17], plain.v[0, 1])


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_q_project_rope_prefill_positions(out_dtype):
    r = np.random.default_rng(43)
    n, d, hq, dh, pos0, theta = 300, 512, 8, 64, 70_000, 5e6
    x = W.store(r.standard_normal((n, d)).astype(np.float32), W.BF16)
    wq = W.store((r.standard_normal((d, hq * dh)) / math.sqrt(d)).astype(np.float32), W.BF16)
    q = y.q_project(to_dev(x), to_dev(wq), hq, dh, out_dtype=out_dtype, rope_theta=theta, pos0=pos0)
    ref = oracle.rope(oracle.project(x, wq), pos0 + np.arange(n), theta, dh)
    if out_dtype == torch.bfloat16:
        _check_rotated(to_stored(q).reshape(n, -1), x, wq, None, 1e-6, pos0 + np.arange(n), theta, dh, d,
                       "rotated Q^ (bf16)")
    else:
        assert_parity(to_stored(q).reshape(n, -1), ref, bf16=False, what="rotated Q^ (fp32)")


def test_q_project_rope_position_table():
    r = np.random.default_rng(44)
    positions = np.array([131071, 0, (1 << 20) - 1], dtype=np.int64)
    x = W.store(r.standard_normal((3, 3072)).astype(np.float32), W.BF16)
    wq = W.store((r.standard_normal((3072, 24 * 128)) / math.sqrt(3072)).astype(np.float32), W.BF16)
    q = y.q_project(to_dev(x), to_dev(wq), 24, 128, rope_theta=80e6, positions=positions)
    _check_rotated(to_stored(q).reshape(3, -1), x, wq, None, 1e-6, positions, 80e6, 128, 3072,
                   "rotated decode queries")
    q32 = y.q_project(to_dev(x), to_dev(wq), 24, 128, out_dtype=torch.float32, rope_theta=80e6, positions=positions)
    assert_parity(to_stored(q32).reshape(3, -1), oracle.rope(oracle.project(x, wq), positions, 80e6, 128),
                  bf16=False, what="rotated decode queries (fp32)")


def test_rope_decode_end_to_end():
    """A generation step with RoPE: K^ rotated at its rows (prompt projection
    plus one append), the query rotated at len - 1, then decode, against the
    oracle on the stored values."""
    p = W.make_project(n=1500, d_model=1024, n_kv_heads=2, head_dim=128, unit_gain=False, seed=45)
    cache = y.KVCache(1, 1500, 2, 128, torch.bfloat16)
    gain = torch.from_numpy(p.gain).cuda()
    y.kv_project(cache, to_dev(p.m[:1499]), to_dev(p.w_k), to_dev(p.w_v), gain, p.eps, rope_theta=640e3)
    y.kv_append(cache, to_dev(p.m[1499:]), to_dev(p.w_k), to_dev(p.w_v), gain, p.eps, rope_theta=640e3)
    r = np.random.default_rng(46)
    x = W.store(r.standard_normal((1, 1024)).astype(np.float32), W.BF16)
    wq = W.store((r.standard_normal((1024, 6 * 128)) / 32.0).astype(np.float32), W.BF16)
    q = y.q_project(to_dev(x), to_dev(wq), 6, 128, rope_theta=640e3, positions=[1499])
    o = to_stored(y.cross_attn_decode(q, cache))
    ref = oracle.decode(to_stored(q), 1500, to_stored(cache.k[0]), to_stored(cache.v[0]), 1 / math.sqrt(128))
    assert_parity(o, ref, bf16=True, what="decode with rotated K^ and Q")
