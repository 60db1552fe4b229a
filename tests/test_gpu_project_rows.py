"""Few-row projections on the kernel that splits W's reduction rows over the
chip (taken whenever a projection of 1..32 rows gets a workspace), against
the fp64 oracle:

* the 3B generation shapes: one appended row (K^ and V^, 8 x 128 from
  d_model 3072) and one query row (24 x 128), bf16 and fp32 outputs, with a
  gain, within one bf16 ulp plus the fp32 accumulation bound (fp32: 1e-5);
* 16 sequences appended at once (two launches of 8 rows): each row has the
  same bits as the one-row projection of the same input (the merge order
  depends on neither the launch's row count nor its other rows);
* repeat calls give the same bits; the arrival counters are zero after every
  call, and nothing past the reported workspace size or outside the output
  rows is written.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_parity, assert_projection_bf16, to_dev, to_stored

pytestmark = pytest.mark.gpu

y = pytest.importorskip("yoco_shared_kv_amd")

COUNTER_BYTES = 16384


def _guarded_workspace(nbytes, guard=64 * 1024):
    buf = torch.zeros(nbytes + guard, dtype=torch.uint8, device="cuda")
    buf[nbytes:] = 0xA5
    return buf


def _check_workspace(buf, nbytes):
    torch.cuda.synchronize()
    assert not bool(buf[:COUNTER_BYTES].any()), "an arrival counter was left non-zero"
    assert bool((buf[nbytes:] == 0xA5).all()), "the projection wrote past its workspace"


@pytest.mark.parametrize("gain", [True, False])
def test_append_one_row_3b(gain):
    p = W.make_project(n=1, d_model=3072, unit_gain=not gain, seed=81)
    print(f"rows path: append one row, 3072 -> 2 x 1024, gain={gain}", flush=True)
    nbytes = y.project_workspace_bytes(1, 3072, 1024, 2)
    assert nbytes > COUNTER_BYTES
    ws = _guarded_workspace(nbytes)
    cache = y.KVCache(1, 40, 8, 128, torch.bfloat16)
    cache.k.fill_(7.0)
    cache.v.fill_(7.0)
    cache.len[0] = 17
    g = torch.from_numpy(p.gain).cuda() if gain else None
    y.kv_append(cache, to_dev(p.m), to_dev(p.w_k), to_dev(p.w_v), g, p.eps, workspace=ws[:nbytes])
    _check_workspace(ws, nbytes)
    assert cache.len.tolist() == [18]
    gr = p.gain if gain else None
    ynorm = np.abs(oracle.rmsnorm(p.m, gr, p.eps))
    for got, w, name in ((cache.k, p.w_k, "K^"), (cache.v, p.w_v, "V^")):
        stored = to_stored(got[0, 17:18]).reshape(1, -1)
        ref = oracle.project(p.m, w, gr, p.eps)
        assert_projection_bf16(stored, ref, ynorm @ np.abs(W.as_f32(w).astype(np.float64)), 3072, name)
        assert torch.all(got[0, :17] == 7.0) and torch.all(got[0, 18:] == 7.0)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_query_one_row_3b(out_dtype):
    r = np.random.default_rng(82)
    x = W.store(r.standard_normal((1, 3072)).astype(np.float32), W.BF16)
    wq = W.store((r.standard_normal((3072, 24 * 128)) / math.sqrt(3072)).astype(np.float32), W.BF16)
    gain = (1 + 0.1 * r.standard_normal(3072)).astype(np.float32)
    nbytes = y.project_workspace_bytes(1, 3072, 3072, 1)
    ws = _guarded_workspace(nbytes)
    out = torch.full((3, 24, 128), float("nan"), dtype=out_dtype, device="cuda")
    q = y.q_project(to_dev(x), to_dev(wq), 24, 128, torch.from_numpy(gain).cuda(), out=out[1:2],
                    workspace=ws[:nbytes])
    _check_workspace(ws, nbytes)
    assert torch.isnan(out[0].float()).all() and torch.isnan(out[2].float()).all(), "wrote outside its output row"
    ref = oracle.project(x, wq, gain)
    if out_dtype == torch.float32:
        assert_parity(to_stored(q).reshape(1, -1), ref, bf16=False, what="Q^ (fp32 out)")
    else:
        terms = np.abs(oracle.rmsnorm(x, gain)) @ np.abs(W.as_f32(wq).astype(np.float64))
        assert_projection_bf16(to_stored(q).reshape(1, -1), ref, terms, 3072, "Q^")


def test_append_sixteen_sequences_matches_one_row_projections_bitwise():
    n_seq = 16
    p = W.make_project(n=n_seq, d_model=3072, unit_gain=False, seed=83)
    lens = np.random.default_rng(84).integers(0, 60, n_seq)
    cache = y.KVCache(n_seq, 64, 8, 128, torch.bfloat16)
    cache.k.fill_(7.0)
    cache.v.fill_(7.0)
    cache.len[:] = lens
    m, wk, wv, g = to_dev(p.m), to_dev(p.w_k), to_dev(p.w_v), torch.from_numpy(p.gain).cuda()
    y.kv_append(cache, m, wk, wv, g, p.eps)
    assert cache.len.tolist() == (lens + 1).tolist()
    one = y.KVCache(1, 1, 8, 128, torch.bfloat16)
    for b in range(n_seq):
        one.len[0] = 0
        y.kv_project(one, m[b:b + 1], wk, wv, g, p.eps)
        assert torch.equal(cache.k[b, lens[b]], one.k[0, 0]), f"K^ row of sequence {b}"
        assert torch.equal(cache.v[b, lens[b]], one.v[0, 0]), f"V^ row of sequence {b}"
    gr = p.gain
    ynorm = np.abs(oracle.rmsnorm(p.m, gr, p.eps))
    got = to_stored(cache.k[torch.arange(n_seq), torch.from_numpy(lens)]).reshape(n_seq, -1)
    assert_projection_bf16(got, oracle.project(p.m, p.w_k, gr, p.eps),
                           ynorm @ np.abs(W.as_f32(p.w_k).astype(np.float64)), 3072, "K^ (16 sequences)")


def test_repeat_calls_are_bitwise_equal():
    r = np.random.default_rng(85)
    x = W.store(r.standard_normal((5, 3072)).astype(np.float32), W.BF16)
    wq = W.store((r.standard_normal((3072, 24 * 128)) / math.sqrt(3072)).astype(np.float32), W.BF16)
    a = y.q_project(to_dev(x), to_dev(wq), 24, 128, out_dtype=torch.float32)
    b = y.q_project(to_dev(x), to_dev(wq), 24, 128, out_dtype=torch.float32)
    assert torch.equal(a, b)
    strips = y.q_project(to_dev(x), to_dev(wq), 24, 128, out_dtype=torch.float32, workspace=False)
    ref = oracle.project(x, wq)
    assert_parity(to_stored(a).reshape(5, -1), ref, bf16=False, what="Q^ split over W rows")
    assert_parity(to_stored(strips).reshape(5, -1), ref, bf16=False, what="Q^ column strips")


def test_too_small_workspace_is_refused_and_nothing_runs():
    r = np.random.default_rng(86)
    x = W.store(r.standard_normal((1, 256)).astype(np.float32), W.BF16)
    wq = W.store(r.standard_normal((256, 256)).astype(np.float32), W.BF16)
    nbytes = y.project_workspace_bytes(1, 256, 256, 1)
    out = torch.full((1, 4, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(y.YocoError) as e:
        y.q_project(to_dev(x), to_dev(wq), 4, 64, out=out,
                    workspace=torch.zeros(nbytes - 16, dtype=torch.uint8, device="cuda"))
    assert e.value.name == "YOCO_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
