"""Backward of the fused RMSNorm + projections (yoco_kv_project_bwd,
yoco_q_project_bwd) against the fp64 oracle, on the same stored inputs.

Tolerances (derived from the arithmetic; the pages fix none for gradients):
* matrix-core path (bf16 input and weights, d_model and the output width
  multiples of 256): y = x g / r and fp32 upstream gradients are rounded to
  bf16 (2^-9 relative) before the two products, which accumulate in fp32, so
  each gradient tensor must have a relative L2 error <= 5e-3 and no element
  off by more than 1% of the tensor's largest magnitude (the bound of the
  attention backward);
* fp32 path (fp32 inputs, or shapes the tiles do not cover): every product
  in fp32 from the stored values, so relative L2 <= 1e-5 and no element off
  by more than 1e-5 of the tensor's largest magnitude.

Full size (32768 rows, d_model 3072 -> 2 x 1024, the 3B widths): d_m on
sampled rows (each row's d_m depends on that row only), d_W on sampled
columns (each column depends on that column of dz only), and d_gain
through additivity over row blocks plus the oracle on one block.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

y = pytest.importorskip("yoco_shared_kv_amd")


def assert_grad(got, ref, what, rel_l2, max_rel):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    top = float(np.abs(ref).max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"  {what}: rel-L2 {rel:.2e}, max-abs {err.max():.2e} of max {top:.2e}", flush=True)
    assert rel <= rel_l2 and err.max() <= max_rel * top, \
        f"{what}: rel-L2 {rel:.2e} (limit {rel_l2}), max-abs {err.max():.2e} (limit {max_rel * top:.2e})"


TOL_MFMA = dict(rel_l2=5e-3, max_rel=1e-2)
TOL_F32 = dict(rel_l2=1e-5, max_rel=1e-5)


def _case(n, d, hkv, dh, dtype, dz_dtype, gain, seed):
    pc = W.make_project(n=n, d_model=d, n_kv_heads=hkv, head_dim=dh, dtype=dtype, seed=seed,
                        unit_gain=not gain)
    dz_k, dz_v = W.make_proj_grad(n, hkv * dh, 2, dtype=dz_dtype, seed=seed)
    return pc, dz_k, dz_v


def _gpu_kv(pc, dz_k, dz_v, gain, init=None, d_gain=True):
    g = torch.from_numpy(pc.gain).cuda() if gain else None
    m, wk, wv = to_dev(pc.m), to_dev(pc.w_k), to_dev(pc.w_v)
    dzk, dzv = to_dev(dz_k), to_dev(dz_v)
    dwk = dwv = dg = None
    if init is not None:
        dwk, dwv, dg = (torch.from_numpy(a.copy()).cuda() for a in init)
    out = y.kv_project_bwd(m, wk, wv, dzk, dzv, pc.n_kv_heads, pc.head_dim, gain=g, eps=pc.eps, d_w_k=dwk,
                           d_w_v=dwv, d_gain=dg, want_gain=d_gain)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().numpy() for t in out]


@pytest.mark.parametrize("n,d,hkv,dh,dtype,dz_dtype,gain,tol", [
    (256, 256, 2, 64, W.F32, W.F32, False, TOL_F32),     # the tiny fp32 end-to-end shapes
    (256, 256, 2, 64, W.F32, W.F32, True, TOL_F32),
    (257, 256, 2, 64, W.BF16, W.F32, True, TOL_F32),     # bf16 stored, width 128: fp32 products
    (300, 512, 2, 128, W.BF16, W.F32, True, TOL_MFMA),   # matrix cores, ragged row tile
    (300, 512, 2, 128, W.BF16, W.BF16, False, TOL_MFMA),
    (700, 256, 4, 64, W.BF16, W.F32, True, TOL_MFMA),    # two row splits of the d_W product
    (1, 256, 2, 128, W.BF16, W.F32, True, TOL_MFMA),     # one row
    (130, 768, 2, 128, W.BF16, W.F32, True, TOL_MFMA),   # the row kernels' last column groups half past d
    (64, 3584, 2, 128, W.BF16, W.F32, True, TOL_MFMA),   # d > 3072: the general row kernel after the MFMA products
    (100, 320, 2, 64, W.F32, W.F32, True, TOL_F32),      # d % 256 != 0: the general row kernel, 4-column groups
    (90, 130, 1, 64, W.F32, W.F32, True, TOL_F32),       # odd width: single columns
])
def test_kv_project_bwd_matches_oracle(n, d, hkv, dh, dtype, dz_dtype, gain, tol):
    print(f"kv_project_bwd n={n} d={d} hkv={hkv} dh={dh} {dtype} dz {dz_dtype} gain={gain}", flush=True)
    pc, dz_k, dz_v = _case(n, d, hkv, dh, dtype, dz_dtype, gain, seed=7)
    rng = np.random.default_rng(3)
    init = [rng.standard_normal(pc.w_k.shape).astype(np.float32),
            rng.standard_normal(pc.w_v.shape).astype(np.float32),
            rng.standard_normal(d).astype(np.float32)]
    d_m, d_wk, d_wv, d_g = _gpu_kv(pc, dz_k, dz_v, gain, init=init)
    ref = oracle.project_bwd(pc.m, pc.w_k, pc.w_v, dz_k, dz_v, gain=pc.gain if gain else None, eps=pc.eps)
    ref_g = ref[3] if gain else _unit_gain_dgain(pc, dz_k, dz_v)
    assert_grad(d_m, ref[0], "d_m", **tol)
    assert_grad(d_wk - init[0], ref[1], "d_w_k (added)", **tol)
    assert_grad(d_wv - init[1], ref[2], "d_w_v (added)", **tol)
    assert_grad(d_g - init[2], ref_g, "d_gain (added)", **tol)


def _unit_gain_dgain(pc, dz_k, dz_v):
    """d_gain of a unit-gain forward: the oracle with an explicit gain of ones
    (the gradient does not depend on the gain's value through dy)."""
    ones = np.ones(pc.m.shape[1], dtype=np.float32)
    return oracle.project_bwd(pc.m, pc.w_k, pc.w_v, dz_k, dz_v, gain=ones, eps=pc.eps)[3]


@pytest.mark.parametrize("n,d,hq,dh,dtype,tol", [
    (200, 256, 4, 128, W.BF16, TOL_MFMA),   # matrix cores, width 512
    (129, 256, 4, 64, W.F32, TOL_F32),      # the tiny query shapes, fp32
])
def test_q_project_bwd_matches_oracle(n, d, hq, dh, dtype, tol):
    print(f"q_project_bwd n={n} d={d} hq={hq} dh={dh} {dtype}", flush=True)
    rng = np.random.default_rng(11)
    x = W.store(rng.standard_normal((n, d)).astype(np.float32), dtype)
    w_q = W.store((rng.standard_normal((d, hq * dh)) / np.sqrt(d)).astype(np.float32), dtype)
    gain = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    (dz,) = W.make_proj_grad(n, hq * dh, 1, dtype=W.F32, seed=5)
    d_x, d_wq, d_g = y.q_project_bwd(to_dev(x), to_dev(w_q), to_dev(dz), hq, dh, gain=torch.from_numpy(gain).cuda(),
                                     want_gain=True)
    torch.cuda.synchronize()
    zeros_w = np.zeros_like(w_q)
    zeros_z = np.zeros_like(dz)
    ref = oracle.project_bwd(x, w_q, zeros_w, dz, zeros_z, gain=gain, eps=1e-6)
    assert_grad(d_x.cpu().numpy(), ref[0], "d_x", **tol)
    assert_grad(d_wq.cpu().numpy(), ref[1], "d_w_q", **tol)
    assert_grad(d_g.cpu().numpy(), ref[3], "d_gain", **tol)


def test_kv_project_bwd_row_blocks_add_up_and_repeat_bitwise():
    """Calls over row blocks with shared d_W / d_gain buffers equal one call
    over all rows; the same call twice gives identical bits."""
    print("kv_project_bwd row blocks", flush=True)
    pc, dz_k, dz_v = _case(600, 512, 2, 128, W.BF16, W.F32, True, seed=9)
    g = torch.from_numpy(pc.gain).cuda()
    m, wk, wv, dzk, dzv = (to_dev(a) for a in (pc.m, pc.w_k, pc.w_v, dz_k, dz_v))
    whole = y.kv_project_bwd(m, wk, wv, dzk, dzv, 2, 128, gain=g, want_gain=True)
    again = y.kv_project_bwd(m, wk, wv, dzk, dzv, 2, 128, gain=g, want_gain=True)
    torch.cuda.synchronize()
    for a, b in zip(whole, again):
        assert torch.equal(a, b)
    dwk = torch.zeros_like(whole[1])
    dwv = torch.zeros_like(whole[2])
    dg = torch.zeros_like(whole[3])
    parts = []
    for r0, r1 in ((0, 250), (250, 600)):
        out = y.kv_project_bwd(m[r0:r1], wk, wv, dzk[r0:r1], dzv[r0:r1], 2, 128, gain=g, d_w_k=dwk, d_w_v=dwv,
                               d_gain=dg)
        parts.append(out[0])
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts), whole[0])   # d_m rows depend on their own row only
    for got, ref, what in ((dwk, whole[1], "d_w_k"), (dwv, whole[2], "d_w_v"), (dg, whole[3], "d_gain")):
        assert_grad(got.cpu().numpy(), ref.cpu().numpy(), what, rel_l2=1e-6, max_rel=1e-5)


def test_kv_project_bwd_full_size_sampled():
    """32768 rows at the 3B widths (bf16, fp32 gain, fp32 upstream gradients):
    the launch configuration the benchmark times."""
    cfg = W.PROJECT_3B
    n, d, hkv, dh = cfg["n"], cfg["d_model"], cfg["n_kv_heads"], cfg["head_dim"]
    print(f"kv_project_bwd full size n={n} d={d}", flush=True)
    pc, dz_k, dz_v = _case(n, d, hkv, dh, W.BF16, W.F32, True, seed=0)
    g = torch.from_numpy(pc.gain).cuda()
    m, wk, wv, dzk, dzv = (to_dev(a) for a in (pc.m, pc.w_k, pc.w_v, dz_k, dz_v))
    d_m, d_wk, d_wv, d_g = y.kv_project_bwd(m, wk, wv, dzk, dzv, hkv, dh, gain=g, eps=pc.eps, want_gain=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    # d_m on sampled rows: the oracle on those rows alone.
    rows = np.sort(rng.choice(n, 48, replace=False))
    rows = np.concatenate([[0, n - 1], rows])
    ref = oracle.project_bwd(pc.m[rows], pc.w_k, pc.w_v, dz_k[rows], dz_v[rows], gain=pc.gain, eps=pc.eps)
    assert_grad(d_m[rows].cpu().numpy(), ref[0], "d_m (sampled rows)", **TOL_MFMA)
    # d_W on sampled columns: the oracle with those columns of W and dz.
    cols = np.sort(rng.choice(hkv * dh, 8, replace=False))
    ref = oracle.project_bwd(pc.m, pc.w_k[:, cols], pc.w_v[:, cols], dz_k[:, cols], dz_v[:, cols],
                             gain=pc.gain, eps=pc.eps)
    assert_grad(d_wk[:, cols].cpu().numpy(), ref[1], "d_w_k (sampled columns)", **TOL_MFMA)
    assert_grad(d_wv[:, cols].cpu().numpy(), ref[2], "d_w_v (sampled columns)", **TOL_MFMA)
    # d_gain: the sum of eight 4096-row blocks, and the oracle on a 512-row block.
    acc = torch.zeros_like(d_g)
    for r0 in range(0, n, 4096):
        y.kv_project_bwd(m[r0:r0 + 4096], wk, wv, dzk[r0:r0 + 4096], dzv[r0:r0 + 4096], hkv, dh, gain=g,
                         eps=pc.eps, d_gain=acc)
    blk = y.kv_project_bwd(m[:512], wk, wv, dzk[:512], dzv[:512], hkv, dh, gain=g, eps=pc.eps, want_gain=True)[3]
    torch.cuda.synchronize()
    assert_grad(acc.cpu().numpy(), d_g.cpu().numpy(), "d_gain (blocks add up)", rel_l2=1e-5, max_rel=1e-4)
    ref = oracle.project_bwd(pc.m[:512], pc.w_k, pc.w_v, dz_k[:512], dz_v[:512], gain=pc.gain, eps=pc.eps)
    assert_grad(blk.cpu().numpy(), ref[3], "d_gain (512-row block)", **TOL_MFMA)
