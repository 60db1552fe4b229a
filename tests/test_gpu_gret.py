"""Gated retention (yoco_gret_prefill, yoco_gret_decode) against the fp64
oracle's parallel form (Eq. 4, continued from a start state) and recurrent
step (Eq. 5), on the same stored q, k, v and fp32 gate logits.

Tolerances (derived from the arithmetic; the outputs are not normalised, so
bounds are relative to the output's scale):
* chunkwise path (bf16, head dim 128): the q.k scores times their decay and
  the carried state are rounded to bf16 (2^-9 relative) before the second
  products, which accumulate in fp32; relative L2 <= 5e-3 and no element off
  by more than 2e-2 of the largest output magnitude (the bf16 bounds of the
  attention outputs, taken relative to scale);
* recurrent path (fp32 arithmetic on the stored values): relative L2 <= 1e-5
  and no element off by more than 1e-5 of the largest magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

y = pytest.importorskip("yoco_shared_kv_amd")

TOL_BF16 = dict(rel_l2=5e-3, max_rel=2e-2)
TOL_F32 = dict(rel_l2=1e-5, max_rel=1e-5)


def assert_close(got, ref, what, rel_l2, max_rel):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    top = float(np.abs(ref).max())
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    print(f"  {what}: rel-L2 {rel:.2e}, max-abs {err.max():.2e} of max {top:.2e}", flush=True)
    assert rel <= rel_l2 and err.max() <= max_rel * top, \
        f"{what}: rel-L2 {rel:.2e} (limit {rel_l2}), max-abs {err.max():.2e} (limit {max_rel * top:.2e})"


def _dev(c):
    return to_dev(c.q), to_dev(c.k), to_dev(c.v), torch.from_numpy(c.gate).cuda()


@pytest.mark.parametrize("n,heads,dh,dtype,tau,with_state", [
    (300, 3, 128, W.BF16, 16.0, False),   # chunkwise: 3 chunks, ragged last one
    (300, 3, 128, W.BF16, 16.0, True),    # ... continuing from a start state
    (1000, 2, 128, W.BF16, 1.0, True),    # strong decay: carried factors underflow across chunks
    (2500, 2, 128, W.BF16, 4.0, True),    # 20 chunks: groups of 8, 8 and 4 chunks, ragged last chunk
    (2049, 1, 128, W.BF16, 16.0, False),  # 17 chunks: the last group is one chunk of one position
    (3000, 2, 128, W.BF16, 1.0, False),   # strong decay across groups
    (128, 2, 128, W.BF16, 16.0, False),   # exactly one chunk
    (1024, 2, 128, W.BF16, 16.0, True),   # exactly one group of 8 chunks (32 whole 32-row sub-tiles)
    (1025, 1, 128, W.BF16, 4.0, True),    # one group and a second group of one position
    (4096, 3, 128, W.BF16, 16.0, True),   # four whole groups chained through the scan
    (1100, 2, 128, W.BF16, 16.0, False),  # second group of 76 positions: 3 sub-tiles, the last ragged
    (1, 2, 128, W.BF16, 16.0, True),      # one position
    (257, 2, 64, W.BF16, 16.0, True),     # head dim 64: recurrent path on bf16 values
    (200, 2, 128, W.F32, 16.0, True),     # fp32: recurrent path
    (96, 3, 64, W.F32, 4.0, False),
])
def test_gret_prefill_matches_oracle(n, heads, dh, dtype, tau, with_state):
    print(f"gret_prefill n={n} heads={heads} dh={dh} {dtype} tau={tau} state={with_state}", flush=True)
    c = W.make_gret(n=n, n_heads=heads, head_dim=dh, dtype=dtype, seed=3, tau=tau)
    s0 = np.random.default_rng(8).standard_normal((heads, dh, dh)).astype(np.float32) if with_state else None
    q, k, v, g = _dev(c)
    o, s1 = y.gret_prefill(q, k, v, g, tau, state_in=None if s0 is None else torch.from_numpy(s0).cuda(),
                           want_state=True)
    torch.cuda.synchronize()
    gamma = oracle.gret_gate(c.gate, tau)
    ref_o, ref_s = oracle.gret(c.q, c.k, c.v, gamma, s_in=s0, want_state=True)
    tol = TOL_BF16 if (dtype == W.BF16 and dh == 128) else TOL_F32
    assert_close(o.cpu().numpy(), ref_o, "o", **tol)
    assert_close(s1.cpu().numpy(), ref_s, "state after the block", **tol)


def test_gret_decode_matches_oracle_step():
    print("gret_decode 3 sequences x 24 heads", flush=True)
    rng = np.random.default_rng(12)
    for dtype, dh in ((W.BF16, 128), (W.F32, 64)):
        c = W.make_gret(n=3, n_heads=24, head_dim=dh, dtype=dtype, seed=4)  # one token per sequence
        st = rng.standard_normal((3, 24, dh, dh)).astype(np.float32)
        state = torch.from_numpy(st).cuda()
        q, k, v, g = _dev(c)
        o = y.gret_decode(q, k, v, g, c.tau, state)
        torch.cuda.synchronize()
        ref_o, ref_s = oracle.gret_step(c.q, c.k, c.v, oracle.gret_gate(c.gate, c.tau), st.astype(np.float64))
        assert_close(o.cpu().numpy(), ref_o, f"decode o ({dtype}, D={dh})", **TOL_F32)
        assert_close(state.cpu().numpy(), ref_s, f"decode state ({dtype}, D={dh})", **TOL_F32)


def test_gret_prefill_then_decode_continues_the_sequence():
    """A chunkwise prefill of 300 positions hands its state to five decode
    steps; the outputs equal the oracle's parallel form over 305 positions."""
    print("gret prefill 300 + 5 decode steps", flush=True)
    c = W.make_gret(n=305, n_heads=3, head_dim=128, dtype=W.BF16, seed=5)
    q, k, v, g = _dev(c)
    o, state = y.gret_prefill(q[:300], k[:300], v[:300], g[:300], c.tau, want_state=True)
    state = state[None].contiguous()
    outs = [o]
    for t in range(300, 305):
        outs.append(y.gret_decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], c.tau, state))
    torch.cuda.synchronize()
    got = torch.cat(outs).cpu().numpy()
    ref = oracle.gret(c.q, c.k, c.v, oracle.gret_gate(c.gate, c.tau))
    assert_close(got, ref, "prefill + decode outputs", **TOL_BF16)


def test_gret_prefill_blocks_chain():
    """Two blocks, the second started from the first's state, equal one block."""
    print("gret prefill 200 + 150 vs 350", flush=True)
    c = W.make_gret(n=350, n_heads=2, head_dim=128, dtype=W.BF16, seed=6)
    q, k, v, g = _dev(c)
    whole, s_whole = y.gret_prefill(q, k, v, g, c.tau, want_state=True)
    o1, s1 = y.gret_prefill(q[:200], k[:200], v[:200], g[:200], c.tau, want_state=True)
    o2, s2 = y.gret_prefill(q[200:], k[200:], v[200:], g[200:], c.tau, state_in=s1, want_state=True)
    torch.cuda.synchronize()
    assert_close(torch.cat([o1, o2]).cpu().numpy(), whole.cpu().numpy(), "two blocks vs one", **TOL_BF16)
    assert_close(s2.cpu().numpy(), s_whole.cpu().numpy(), "final state", **TOL_BF16)
    again = y.gret_prefill(q, k, v, g, c.tau)
    torch.cuda.synchronize()
    assert torch.equal(again, whole)  # bitwise reproducible


def test_gret_prefill_full_size_sampled():
    """32768 positions, 24 heads of 128 (the 3B self-decoder shapes), bf16:
    a row of every 128-position chunk and the final state against the oracle."""
    cfg = W.GRET_32K
    print(f"gret_prefill full size {cfg}", flush=True)
    c = W.make_gret(**cfg, dtype=W.BF16, seed=0)
    q, k, v, g = _dev(c)
    o, s = y.gret_prefill(q, k, v, g, c.tau, want_state=True)
    torch.cuda.synchronize()
    n = cfg["n"]
    # One seeded row in every 128-position chunk (every chunk step of every
    # group's output pass, all heads) plus chunk and group edges.
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, 127, 128, 1023, 1024, n - 1]] +
                                    [[c0 * 128 + int(rng.integers(128))] for c0 in range(n // 128)])).astype(np.int64)
    gamma = oracle.gret_gate(c.gate, c.tau)
    ref_o, ref_s = oracle.gret(c.q, c.k, c.v, gamma, rows=rows, want_state=True)
    assert_close(o.cpu().numpy()[rows], ref_o, "sampled rows", **TOL_BF16)
    assert_close(s.cpu().numpy(), ref_s, "final state", **TOL_BF16)
