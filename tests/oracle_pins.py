"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Every pin takes an ``oracle.Oracle`` instance and raises ``AssertionError``
when the instance disagrees.  ``test_oracle.py`` runs them against the real
oracle; ``test_oracle_mutations.py`` runs them against copies of ``oracle.c``
with a plausible mistake planted, and requires each copy to fail at least one.

None of these re-types the oracle's formula.  They use closed forms
(constant and one-hot rows, one or two visible keys, identical keys),
invariants the pages fix (causality, GQA == MHA with repeated heads, prefix
invariance, shared == per-layer copies), invariances of softmax (shift of the
keys, affine V, row permutation) and independent library routines
(``torch.nn.functional.rms_norm`` and ``scaled_dot_product_attention`` in
fp64 on the CPU, numpy fp64 matmul).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from workloads import BF16, F32, as_f32, store


def _rng(seed):
    return np.random.default_rng(1000 + seed)


def _grid(rng, shape, step=1.0 / 64, lim=4.0):
    """fp32 values on a coarse grid, so that sums of a few of them are exact."""
    return (np.round(rng.uniform(-lim, lim, size=shape) / step) * step).astype(np.float32)


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise AssertionError(f"{what}: non-finite oracle output")
    if not np.allclose(a, b, rtol=rtol, atol=atol):
        err = np.max(np.abs(a - b))
        raise AssertionError(f"{what}: max abs err {err:.3e}")


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------
def pin_rmsnorm_constant_row(orc):
    """x = c*1 gives y = c*g / sqrt(c^2 + eps) (mean of squares is c^2)."""
    rng = _rng(1)
    d = 16
    g = (1.0 + 0.5 * rng.standard_normal(d)).astype(np.float32)
    eps = 0.25
    for c in (0.5, -3.0, 2.0):
        x = np.full((1, d), c, dtype=np.float32)
        y = orc.rmsnorm(x, g, eps)
        want = c * g.astype(np.float64) / math.sqrt(c * c + eps)
        _close(y[0], want, 1e-13, 0, f"rmsnorm constant row c={c}")


def pin_rmsnorm_one_hot(orc):
    """x = a*e_k gives y_k = a*g_k / sqrt(a^2/d + eps) and zeros elsewhere."""
    d, k, a, eps = 32, 5, 3.0, 0.5
    g = np.linspace(0.5, 2.0, d).astype(np.float32)
    x = np.zeros((1, d), dtype=np.float32)
    x[0, k] = a
    y = orc.rmsnorm(x, g, eps)
    want = np.zeros(d)
    want[k] = a * float(g[k]) / math.sqrt(a * a / d + eps)
    _close(y[0], want, 1e-13, 0, "rmsnorm one-hot")


def pin_rmsnorm_library(orc):
    """Agrees with torch.nn.functional.rms_norm in fp64 (fp32 and bf16 storage)."""
    rng = _rng(2)
    for dtype in (F32, BF16):
        x = store(rng.standard_normal((7, 96)).astype(np.float32) * 3, dtype)
        g = (1 + 0.2 * rng.standard_normal(96)).astype(np.float32)
        eps = 1e-3
        got = orc.rmsnorm(x, g, eps)
        xt = torch.from_numpy(as_f32(x).astype(np.float64))
        want = torch.nn.functional.rms_norm(xt, (96,), torch.from_numpy(g.astype(np.float64)), eps)
        _close(got, want.numpy(), 1e-12, 1e-14, f"rmsnorm vs torch ({dtype})")


# ---------------------------------------------------------------------------
# Projections (RMSNorm then @ W)
# ---------------------------------------------------------------------------
def pin_project_identity(orc):
    """With W = I the projection is the normalised input."""
    rng = _rng(3)
    x = rng.standard_normal((5, 24)).astype(np.float32)
    g = (1 + 0.3 * rng.standard_normal(24)).astype(np.float32)
    out = orc.project(x, np.eye(24, dtype=np.float32), g, 1e-6)
    _close(out, orc.rmsnorm(x, g, 1e-6), 1e-14, 0, "project with identity W")


def pin_project_column_selector(orc):
    """Column j of W = e_{c_j} picks normalised feature c_j (orientation of W)."""
    rng = _rng(4)
    d, ncols = 40, 12
    x = rng.standard_normal((6, d)).astype(np.float32)
    cols = rng.choice(d, ncols, replace=False)
    w = np.zeros((d, ncols), dtype=np.float32)
    w[cols, np.arange(ncols)] = 1.0
    out = orc.project(x, w, None, 1e-6)
    xt = torch.from_numpy(x.astype(np.float64))
    y = torch.nn.functional.rms_norm(xt, (d,), None, 1e-6).numpy()
    _close(out, y[:, cols], 1e-13, 0, "project column selector")


def pin_project_library(orc):
    """Agrees with torch rms_norm followed by numpy fp64 matmul (non-square W)."""
    rng = _rng(5)
    for dtype in (F32, BF16):
        d, ncols = 48, 20
        x = store(rng.standard_normal((9, d)).astype(np.float32), dtype)
        w = store((rng.standard_normal((d, ncols)) / math.sqrt(d)).astype(np.float32), dtype)
        g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
        got = orc.project(x, w, g, 1e-6)
        xt = torch.from_numpy(as_f32(x).astype(np.float64))
        y = torch.nn.functional.rms_norm(xt, (d,), torch.from_numpy(g.astype(np.float64)), 1e-6)
        want = y.numpy() @ as_f32(w).astype(np.float64)
        _close(got, want, 1e-12, 1e-14, f"project vs torch+numpy ({dtype})")


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def _torch_reference(q, q_pos, k, v, scale):
    """fp64 SDPA with an explicit causal mask built from absolute positions and
    repeat-interleaved K/V heads (query head h reads KV head h // G)."""
    qf = torch.from_numpy(as_f32(q).astype(np.float64))       # [n_q, hq, dh]
    kf = torch.from_numpy(as_f32(k).astype(np.float64))       # [rows, hkv, dh]
    vf = torch.from_numpy(as_f32(v).astype(np.float64))
    hq, hkv = qf.shape[1], kf.shape[1]
    kr = kf.repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2).contiguous()
    vr = vf.repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2).contiguous()
    qh = qf.permute(1, 0, 2).contiguous()
    rows = kf.shape[0]
    mask = torch.arange(rows)[None, :] <= torch.as_tensor(np.asarray(q_pos))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qh, kr, vr, attn_mask=mask, scale=scale)
    logits = (qh @ kr.transpose(1, 2)) * scale
    logits = logits.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


def pin_attn_single_visible_key(orc):
    """Position 0 sees only row 0: the output is V_0 exactly and lse is the
    one logit."""
    rng = _rng(6)
    q = rng.standard_normal((1, 4, 16)).astype(np.float32)
    k = rng.standard_normal((5, 2, 16)).astype(np.float32)
    v = rng.standard_normal((5, 2, 16)).astype(np.float32)
    o, lse = orc.attention(q, [0], k, v, 0.3, want_lse=True)
    for h in range(4):
        g = h // 2
        if not np.array_equal(o[0, h], v[0, g].astype(np.float64)):
            raise AssertionError("single visible key must return V_0 exactly")
        want = 0.3 * float(np.dot(q[0, h].astype(np.float64), k[0, g].astype(np.float64)))
        _close(lse[0, h], want, 1e-13, 1e-15, "lse with one visible key")


def pin_attn_identical_keys(orc):
    """All keys equal: uniform weights, output = mean of visible V rows,
    lse = logit + ln(t+1)."""
    rng = _rng(7)
    rows, dh = 9, 8
    k = np.tile(rng.standard_normal((1, 1, dh)).astype(np.float32), (rows, 1, 1))
    v = rng.standard_normal((rows, 1, dh)).astype(np.float32)
    q = rng.standard_normal((rows, 1, dh)).astype(np.float32)
    pos = np.arange(rows)
    o, lse = orc.attention(q, pos, k, v, 0.7, want_lse=True)
    for t in range(rows):
        want = v[: t + 1, 0].astype(np.float64).mean(axis=0)
        _close(o[t, 0], want, 1e-13, 1e-15, f"identical keys, position {t}")
        x = 0.7 * float(np.dot(q[t, 0].astype(np.float64), k[0, 0].astype(np.float64)))
        _close(lse[t, 0], x + math.log(t + 1), 1e-13, 1e-15, "lse with identical keys")


def pin_attn_two_keys_closed_form(orc):
    """Two visible keys: weights are a logistic pair in s*(q.k0 - q.k1)."""
    q = np.array([[[1.0, 2.0, -1.0, 0.5]]], dtype=np.float32)
    k = np.array([[[0.5, 1.0, 0.0, 2.0]], [[-1.0, 0.25, 1.5, 1.0]]], dtype=np.float32)
    v = np.array([[[1.0, -2.0, 3.0, 0.0]], [[4.0, 0.5, -1.0, 2.0]]], dtype=np.float32)
    s = 0.37
    x0 = s * (0.5 + 2.0 + 0.0 + 1.0)          # s * q.k0 = s * 3.5
    x1 = s * (-1.0 + 0.5 - 1.5 + 0.5)         # s * q.k1 = s * -1.5
    w0 = 1.0 / (1.0 + math.exp(x1 - x0))
    want = w0 * v[0, 0].astype(np.float64) + (1 - w0) * v[1, 0].astype(np.float64)
    o, lse = orc.attention(q, [1], k, v, s, want_lse=True)
    _close(o[0, 0], want, 1e-14, 1e-15, "two-key closed form")
    _close(lse[0, 0], x0 + math.log1p(math.exp(x1 - x0)), 1e-14, 1e-15, "two-key lse")


def pin_attn_gqa_head_mapping(orc):
    """H_q=6, H_kv=3: query head h reads KV head h // 2.  V of KV head g is the
    constant g+1, so each output is that constant."""
    rng = _rng(8)
    rows, dh = 7, 8
    q = rng.standard_normal((rows, 6, dh)).astype(np.float32)
    k = rng.standard_normal((rows, 3, dh)).astype(np.float32)
    v = np.zeros((rows, 3, dh), dtype=np.float32)
    for g in range(3):
        v[:, g, :] = g + 1
    o = orc.attention(q, np.arange(rows), k, v, 0.5)
    for h in range(6):
        _close(o[:, h, :], np.full((rows, dh), h // 2 + 1.0), 1e-13, 1e-13, f"GQA head {h}")


def pin_attn_gqa_equals_mha(orc):
    """Repeating each KV head G times and running MHA gives the GQA result."""
    rng = _rng(9)
    rows, hq, hkv, dh = 11, 6, 2, 16
    q = rng.standard_normal((rows, hq, dh)).astype(np.float32)
    k = rng.standard_normal((rows, hkv, dh)).astype(np.float32)
    v = rng.standard_normal((rows, hkv, dh)).astype(np.float32)
    pos = np.arange(rows)
    gqa = orc.attention(q, pos, k, v, 0.25)
    mha = orc.attention(q, pos, np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1), 0.25)
    if not np.array_equal(gqa, mha):
        raise AssertionError("GQA must equal MHA over repeated KV heads")


def pin_attn_prefix_invariance(orc):
    """The output at position t does not change when rows after t exist."""
    rng = _rng(10)
    rows, dh = 20, 8
    q = rng.standard_normal((rows, 2, dh)).astype(np.float32)
    k = rng.standard_normal((rows, 1, dh)).astype(np.float32)
    v = rng.standard_normal((rows, 1, dh)).astype(np.float32)
    full = orc.attention(q, np.arange(rows), k, v, 0.4)
    for t in (0, 3, 12, rows - 1):
        part = orc.attention(q[t:t + 1], [t], k[: t + 1], v[: t + 1], 0.4)
        if not np.array_equal(part[0], full[t]):
            raise AssertionError(f"prefix invariance fails at position {t}")


def pin_attn_causal_boundary(orc):
    """Position p depends on row p (inclusive mask) and not on row p+1."""
    rng = _rng(11)
    rows, dh, p = 10, 8, 5
    q = rng.standard_normal((1, 1, dh)).astype(np.float32)
    k = rng.standard_normal((rows, 1, dh)).astype(np.float32)
    v = rng.standard_normal((rows, 1, dh)).astype(np.float32)
    base = orc.attention(q, [p], k, v, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[p + 1] += 3.0
    v2[p + 1] += 3.0
    if not np.array_equal(orc.attention(q, [p], k2, v2, 0.5), base):
        raise AssertionError("row p+1 must be invisible at position p")
    v3 = v.copy()
    v3[p] += 3.0
    if np.allclose(orc.attention(q, [p], k, v3, 0.5), base, rtol=0, atol=1e-9):
        raise AssertionError("row p must be visible at position p")


def pin_attn_shift_invariance(orc):
    """Adding one vector u to every key of a head shifts all logits by s*q.u,
    which softmax ignores.  Keys and u sit on a 1/64 grid so k+u is stored
    exactly.  The large shift pushes logits past 1000, where exp overflows in
    fp64 without the max subtraction."""
    rng = _rng(12)
    rows, dh = 16, 8
    q = _grid(rng, (rows, 1, dh), lim=2.0)
    q[:, 0, 0] = 2.0
    k = _grid(rng, (rows, 1, dh))
    v = _grid(rng, (rows, 1, dh))
    base = orc.attention(q, np.arange(rows), k, v, 1.0)
    for shift in (3.0, 1200.0):
        u = np.zeros((1, 1, dh), dtype=np.float32)
        u[0, 0, 0] = shift
        got = orc.attention(q, np.arange(rows), k + u, v, 1.0)
        _close(got, base, 1e-11, 1e-12, f"shift invariance (shift {shift})")


def pin_attn_v_affine(orc):
    """V -> a*V + b gives O -> a*O + b; a constant V gives that constant."""
    rng = _rng(13)
    rows, dh = 12, 8
    q = rng.standard_normal((rows, 2, dh)).astype(np.float32)
    k = rng.standard_normal((rows, 2, dh)).astype(np.float32)
    v = _grid(rng, (rows, 2, dh))
    b = _grid(rng, (1, 2, dh))
    base = orc.attention(q, np.arange(rows), k, v, 0.3)
    got = orc.attention(q, np.arange(rows), k, 2.0 * v + b, 0.3)
    _close(got, 2.0 * base + b.astype(np.float64), 1e-12, 1e-12, "V affine")


def pin_attn_row_permutation(orc):
    """Decode over all rows is invariant to permuting the cache rows (K and V
    together)."""
    rng = _rng(14)
    rows, dh = 33, 16
    q = rng.standard_normal((3, 4, dh)).astype(np.float32)
    k = rng.standard_normal((rows, 2, dh)).astype(np.float32)
    v = rng.standard_normal((rows, 2, dh)).astype(np.float32)
    perm = rng.permutation(rows)
    a = orc.decode(q, rows, k, v, 0.25)
    b = orc.decode(q, rows, k[perm], v[perm], 0.25)
    _close(a, b, 1e-12, 1e-14, "row permutation")


def pin_attn_library(orc):
    """Agrees with torch SDPA in fp64 (explicit position mask, repeated KV
    heads) for prefill blocks with q_start > 0 and for decode, fp32 and bf16."""
    rng = _rng(15)
    for dtype, (rows, q_start, hq, hkv, dh) in (
            (F32, (37, 0, 4, 2, 16)), (BF16, (45, 13, 6, 2, 32)), (BF16, (29, 28, 3, 1, 8))):
        t = rows - q_start
        q = store(rng.standard_normal((t, hq, dh)).astype(np.float32), dtype)
        k = store(rng.standard_normal((rows, hkv, dh)).astype(np.float32) * 2, dtype)
        v = store(rng.standard_normal((rows, hkv, dh)).astype(np.float32), dtype)
        s = 1 / math.sqrt(dh)
        pos = q_start + np.arange(t)
        o, lse = orc.prefill(q, q_start, k, v, s, want_lse=True)
        ro, rlse = _torch_reference(q, pos, k, v, s)
        _close(o, ro, 1e-11, 1e-13, f"attention vs torch SDPA ({dtype}, q_start={q_start})")
        _close(lse, rlse, 1e-12, 1e-13, f"lse vs torch logsumexp ({dtype})")


def pin_decode_is_last_prefill_row(orc):
    """Decode at length n equals prefill row n-1 (the last prompt position
    runs the cross layer, as the reading notes' section 2.5 describes)."""
    rng = _rng(16)
    rows, dh = 19, 16
    q = rng.standard_normal((rows, 4, dh)).astype(np.float32)
    k = rng.standard_normal((rows, 2, dh)).astype(np.float32)
    v = rng.standard_normal((rows, 2, dh)).astype(np.float32)
    pre = orc.prefill(q, 0, k, v, 0.25)
    dec = orc.decode(q[rows - 1:rows], rows, k, v, 0.25)
    if not np.array_equal(pre[rows - 1], dec[0]):
        raise AssertionError("decode must equal the last prefill row")


# ---------------------------------------------------------------------------
# Rotary position embedding (the blog's section 7: K^ and each layer's Q are
# rotated by position, V is not; base theta per stage from the notes' Table 7)
# ---------------------------------------------------------------------------
def pin_rope_position_zero_is_identity(orc):
    """At position 0 every angle is 0: the rotation leaves x unchanged."""
    x = _rng(20).standard_normal((2, 3, 16))
    for inter in (True, False):
        if not np.array_equal(orc.rope(x, [0, 0], 1e4, 16, inter), x):
            raise AssertionError("RoPE at position 0 must be the identity")


def pin_rope_single_pair_closed_form(orc):
    """One pair (d_h = 2, frequency theta^0 = 1): (1, 0) at position p turns
    to (cos p, sin p) and (0, 1) to (-sin p, cos p)."""
    pos = np.array([1, 2, 7, 100], dtype=np.int64)
    e0 = np.tile(np.array([[1.0, 0.0]]), (4, 1))
    e1 = np.tile(np.array([[0.0, 1.0]]), (4, 1))
    r0 = orc.rope(e0, pos, 640e3, 2)
    r1 = orc.rope(e1, pos, 640e3, 2)
    _close(r0, np.stack([np.cos(pos), np.sin(pos)], 1), 0, 1e-15, "RoPE of (1, 0)")
    _close(r1, np.stack([-np.sin(pos), np.cos(pos)], 1), 0, 1e-15, "RoPE of (0, 1)")


def _torch_rope_interleaved(x, pos, theta, dh):
    """Complex multiplication in torch: consecutive pairs as complex numbers
    times exp(j * pos * theta^(-2i/d_h))."""
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    n, h, _ = xt.shape
    z = torch.view_as_complex(xt.reshape(n, h, dh // 2, 2))
    freq = torch.tensor(theta, dtype=torch.float64) ** (-torch.arange(0, dh, 2, dtype=torch.float64) / dh)
    ang = torch.from_numpy(np.asarray(pos, dtype=np.float64))[:, None] * freq[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.view_as_real(z * rot).reshape(n, h, dh).numpy()


def pin_rope_library_complex(orc):
    """Against torch complex arithmetic, including positions near 2^20 with
    the 1M-stage base (80M), where a single-precision angle would be off."""
    rng = _rng(21)
    for theta, pos in ((640e3, [0, 1, 5, 4096]), (80e6, [1 << 20, (1 << 20) - 1, 999_983, 3])):
        x = rng.standard_normal((4, 3, 64))
        _close(orc.rope(x, pos, theta, 64), _torch_rope_interleaved(x, pos, theta, 64), 1e-12, 1e-12,
               f"RoPE vs torch complex (theta {theta:g})")


def pin_rope_preserves_norms(orc):
    """A rotation keeps the length of every pair (so of every head)."""
    x = _rng(22).standard_normal((5, 2, 32))
    pos = [3, 17, 4095, 65536, 131071]
    for inter in (True, False):
        y = orc.rope(x, pos, 5e6, 32, inter)
        _close(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), 1e-14, 0, "RoPE norm")


def pin_rope_composition(orc):
    """Turning by a then by b is turning by a + b."""
    x = _rng(23).standard_normal((3, 2, 16))
    a = np.array([5, 1000, 77], dtype=np.int64)
    b = np.array([9, 31, 65536], dtype=np.int64)
    for inter in (True, False):
        two = orc.rope(orc.rope(x, a, 640e3, 16, inter), b, 640e3, 16, inter)
        _close(two, orc.rope(x, a + b, 640e3, 16, inter), 1e-11, 1e-11, "RoPE composition")


def pin_rope_scores_depend_on_offset(orc):
    """<R(m) q, R(n) k> depends only on m - n: shifting both positions leaves
    the score unchanged (what lets attention read relative position)."""
    rng = _rng(24)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    base = np.sum(orc.rope(q, [100], 5e6, 64) * orc.rope(k, [37], 5e6, 64))
    for shift in (1, 1000, 500_000):
        s = np.sum(orc.rope(q, [100 + shift], 5e6, 64) * orc.rope(k, [37 + shift], 5e6, 64))
        _close(s, base, 1e-9, 1e-9, f"RoPE score after shift {shift}")
    moved = np.sum(orc.rope(q, [101], 5e6, 64) * orc.rope(k, [37], 5e6, 64))
    if abs(moved - base) < 1e-6:
        raise AssertionError("the score must change with the offset")


def pin_rope_half_is_permuted_interleaved(orc):
    """Pairs (i, i + d_h/2) are pairs (2i, 2i+1) after the permutation that
    interleaves the two halves of a head."""
    x = _rng(25).standard_normal((2, 2, 16))
    perm = np.empty(16, dtype=np.int64)
    perm[0::2] = np.arange(8)
    perm[1::2] = np.arange(8) + 8          # interleaved slot 2i <- i, 2i+1 <- i+8
    half = orc.rope(x, [11, 5000], 1e4, 16, interleaved=False)
    inter = orc.rope(x[..., perm], [11, 5000], 1e4, 16, interleaved=True)
    _close(half[..., perm], inter, 1e-14, 1e-14, "rotate-half vs interleaved")



# ---------------------------------------------------------------------------
# Backward (gradients of the attention and of the shared projection)
# ---------------------------------------------------------------------------
def _fd_grad(f, x, h):
    """Central differences of the scalar f at x (fp64, every element)."""
    g = np.empty_like(x)
    flat, gf = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        fp = f()
        flat[i] = old - h
        fm = f()
        flat[i] = old
        gf[i] = (fp - fm) / (2 * h)
    return g


def pin_attn_bwd_finite_differences(orc):
    """dq, dk, dv are the derivatives of L = sum(dO * O) (O from the pinned
    forward): central differences on fp64 inputs, query rows at repeated and
    out-of-order positions."""
    rng = _rng(30)
    pos = np.array([2, 4, 4, 0, 3])
    q = rng.standard_normal((5, 4, 6))
    k = rng.standard_normal((5, 2, 6))
    v = rng.standard_normal((5, 2, 6))
    dout = rng.standard_normal((5, 4, 6))
    scale = 0.45
    loss = lambda: float(np.sum(dout * orc.attention(q, pos, k, v, scale)))
    dq, dk, dv = orc.attention_bwd(q, pos, k, v, dout, scale)
    for name, got, arr in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _close(got, _fd_grad(loss, arr, 1e-6), 1e-6, 1e-8, f"attention {name} vs finite differences")


def _torch_attn_grads(q, pos, k, v, dout, scale):
    """fp64 autograd of masked softmax attention with repeat-interleaved K/V."""
    qt = torch.tensor(as_f32(q).astype(np.float64), requires_grad=True)
    kt = torch.tensor(as_f32(k).astype(np.float64), requires_grad=True)
    vt = torch.tensor(as_f32(v).astype(np.float64), requires_grad=True)
    hq, hkv = q.shape[1], k.shape[1]
    kr = kt.repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
    vr = vt.repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
    qh = qt.permute(1, 0, 2)
    mask = torch.arange(k.shape[0])[None, :] <= torch.as_tensor(np.asarray(pos))[:, None]
    logits = torch.matmul(qh, kr.transpose(1, 2).contiguous()) * scale
    o = torch.matmul(torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=-1), vr).permute(1, 0, 2)
    (o * torch.from_numpy(as_f32(dout).astype(np.float64))).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_attn_bwd_library(orc):
    """Against torch autograd (fp64) for a prefill block at q_start = 10 over
    40 cache rows, GQA 6/2, bf16 and fp32 storage."""
    rng = _rng(31)
    for dtype in (F32, BF16):
        q = store(rng.standard_normal((30, 6, 16)).astype(np.float32), dtype)
        k = store(rng.standard_normal((40, 2, 16)).astype(np.float32), dtype)
        v = store(rng.standard_normal((40, 2, 16)).astype(np.float32), dtype)
        dout = store(rng.standard_normal((30, 6, 16)).astype(np.float32), dtype)
        pos = 10 + np.arange(30)
        got = orc.attention_bwd(q, pos, k, v, dout, 0.25)
        want = _torch_attn_grads(q, pos, k, v, dout, 0.25)
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            _close(a, b, 1e-10, 1e-12, f"attention {name} vs torch autograd ({dtype})")


def pin_attn_bwd_sums(orc):
    """Softmax weights sum to one and their gradients sum to zero: over all
    cache rows, sum_j dk_j = 0 and sum_j dv_j = sum of dO over the query rows
    and the query heads of each KV head."""
    rng = _rng(32)
    q = rng.standard_normal((24, 6, 8))
    k = rng.standard_normal((24, 3, 8))
    v = rng.standard_normal((24, 3, 8))
    dout = rng.standard_normal((24, 6, 8))
    _, dk, dv = orc.attention_bwd(q, np.arange(24), k, v, dout, 0.5)
    _close(dk.sum(axis=0), np.zeros((3, 8)), 0, 1e-12, "sum of dk over cache rows")
    _close(dv.sum(axis=0), dout.reshape(24, 3, 2, 8).sum(axis=(0, 2)), 1e-12, 1e-12, "sum of dv over cache rows")


def pin_attn_bwd_single_key(orc):
    """A query at position 0 sees only row 0 (p = 1): dq = 0, its dv_0 is dO
    and its dk_0 is 0, exactly."""
    rng = _rng(33)
    q = rng.standard_normal((1, 2, 8))
    k = rng.standard_normal((3, 1, 8))
    v = rng.standard_normal((3, 1, 8))
    dout = rng.standard_normal((1, 2, 8))
    dq, dk, dv = orc.attention_bwd(q, [0], k, v, dout, 0.7)
    if np.any(dq != 0) or np.any(dk != 0) or np.any(dv[1:] != 0):
        raise AssertionError("one visible key: dq, dk and the other rows' dv must be zero")
    if not np.array_equal(dv[0, 0], dout[0, 0] + dout[0, 1]):
        raise AssertionError("one visible key: dv_0 must be the sum of dO over the group")


def pin_attn_bwd_accumulates(orc):
    """dk, dv add up: two calls over disjoint query rows (or two layers)
    equal one call over all of them."""
    rng = _rng(34)
    q = rng.standard_normal((12, 4, 8))
    k = rng.standard_normal((12, 2, 8))
    v = rng.standard_normal((12, 2, 8))
    dout = rng.standard_normal((12, 4, 8))
    pos = np.arange(12)
    _, dk1, dv1 = orc.attention_bwd(q, pos, k, v, dout, 0.3)
    _, dk2, dv2 = orc.attention_bwd(q[:5], pos[:5], k, v, dout[:5], 0.3)
    orc.attention_bwd(q[5:], pos[5:], k, v, dout[5:], 0.3, dk2, dv2)
    _close(dk2, dk1, 1e-12, 1e-13, "dk over two calls")
    _close(dv2, dv1, 1e-12, 1e-13, "dv over two calls")


def pin_project_bwd_finite_differences(orc):
    """dx, dgain, dw_k, dw_v are the derivatives of L = sum(dz_k * K^) +
    sum(dz_v * V^) (K^, V^ from the pinned forward projection); L is linear
    in the gain and the weights, so a grid step gives exact differences
    there."""
    rng = _rng(35)
    x = rng.standard_normal((3, 8))
    w_k = rng.standard_normal((8, 4))
    w_v = rng.standard_normal((8, 4))
    gain = (1.0 + np.round(rng.uniform(-0.5, 0.5, 8) * 64) / 64).astype(np.float32)
    dz_k = rng.standard_normal((3, 4))
    dz_v = rng.standard_normal((3, 4))
    eps = 1e-2
    loss = lambda: float(np.sum(dz_k * orc.project(x, w_k, gain, eps)) + np.sum(dz_v * orc.project(x, w_v, gain, eps)))
    dx, dw_k, dw_v, dgain = orc.project_bwd(x, w_k, w_v, dz_k, dz_v, gain, eps)
    _close(dx, _fd_grad(loss, x, 1e-6), 1e-6, 1e-8, "project dx vs finite differences")
    _close(dw_k, _fd_grad(loss, w_k, 1e-3), 1e-9, 1e-10, "project dw_k vs finite differences")
    _close(dw_v, _fd_grad(loss, w_v, 1e-3), 1e-9, 1e-10, "project dw_v vs finite differences")
    g = gain
    fd = np.empty(8)
    for c in range(8):
        old = g[c]
        g[c] = old + np.float32(2.0 ** -6)
        lp = loss()
        g[c] = old - np.float32(2.0 ** -6)
        lm = loss()
        g[c] = old
        fd[c] = (lp - lm) / 2.0 ** -5
    _close(dgain, fd, 1e-9, 1e-10, "project dgain vs finite differences")


def pin_project_bwd_scale_invariance(orc):
    """With eps = 0, RMSNorm(a x) = RMSNorm(x) for a > 0, so the gradient
    with respect to a row is orthogonal to the row."""
    rng = _rng(36)
    x = rng.standard_normal((4, 16))
    w = rng.standard_normal((16, 8))
    gain = (1.0 + 0.25 * rng.standard_normal(16)).astype(np.float32)
    dx, _, _, _ = orc.project_bwd(x, w, w, rng.standard_normal((4, 8)), rng.standard_normal((4, 8)), gain, 0.0)
    _close(np.sum(dx * x, axis=1), np.zeros(4), 0, 1e-12, "x . dx with eps = 0")


def pin_project_bwd_library(orc):
    """Against torch autograd (fp64) of rms_norm followed by two matmuls, with
    bf16 storage of x and the weights."""
    rng = _rng(37)
    n, d, nc = 10, 32, 12
    x = store(rng.standard_normal((n, d)).astype(np.float32), BF16)
    w_k = store((rng.standard_normal((d, nc)) / 4).astype(np.float32), BF16)
    w_v = store((rng.standard_normal((d, nc)) / 4).astype(np.float32), BF16)
    gain = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    dz_k = rng.standard_normal((n, nc)).astype(np.float32)
    dz_v = rng.standard_normal((n, nc)).astype(np.float32)
    got = orc.project_bwd(x, w_k, w_v, dz_k, dz_v, gain, 1e-6)
    xt = torch.tensor(as_f32(x).astype(np.float64), requires_grad=True)
    gt = torch.tensor(gain.astype(np.float64), requires_grad=True)
    wk = torch.tensor(as_f32(w_k).astype(np.float64), requires_grad=True)
    wv = torch.tensor(as_f32(w_v).astype(np.float64), requires_grad=True)
    y = torch.nn.functional.rms_norm(xt, (d,), gt, 1e-6)
    loss = (torch.matmul(y, wk) * torch.from_numpy(dz_k.astype(np.float64))).sum() + \
        (torch.matmul(y, wv) * torch.from_numpy(dz_v.astype(np.float64))).sum()
    loss.backward()
    for name, a, b in zip(("dx", "dw_k", "dw_v", "dgain"), got, (xt.grad, wk.grad, wv.grad, gt.grad)):
        _close(a, b.numpy(), 1e-10, 1e-12, f"project {name} vs torch autograd")

# ---------------------------------------------------------------------------
# Gated retention (the self-decoder's token mixer)
# ---------------------------------------------------------------------------
GRET_GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "gret_worked_example.txt")


def _gret_golden():
    vals = {}
    for line in open(GRET_GOLDEN):
        if line.strip() and not line.startswith("#"):
            name, *nums = line.split()
            vals[name] = np.array([float(x) for x in nums], dtype=np.float64)
    return vals


def pin_gret_worked_example(orc):
    """The blog's 2x2 example (section 4): state [[2,0],[0,2]], gate 0.5,
    k = [1,0], v = [3,4] -> state [[4,4],[0,1]]; q = [1,0] reads [4,4].  Both
    the recurrent step and the parallel form started from that state."""
    g = _gret_golden()
    q = g["q"].reshape(1, 1, 2)
    k = g["k"].reshape(1, 1, 2)
    v = g["v"].reshape(1, 1, 2)
    gamma = g["gamma"].reshape(1, 1)
    s0 = g["state_before"].reshape(1, 1, 2, 2)
    o, s1 = orc.gret_step(q, k, v, gamma, s0)
    _close(s1.reshape(4), g["state_after"], 0, 0, "gret step: state")
    _close(o.reshape(2), g["o"], 0, 0, "gret step: output")
    o, s1 = orc.gret(q, k, v, gamma, s_in=s0[0], want_state=True)
    _close(s1.reshape(4), g["state_after"], 0, 0, "gret parallel: state")
    _close(o.reshape(2), g["o"], 0, 0, "gret parallel: output")


def pin_gret_two_token_state(orc):
    """The reading notes' example (section 2.2): from S_0 = 0, two tokens give
    S_2 = gamma_2 k_1^T v_1 + k_2^T v_2 -- the first token is decayed by the
    second step's gate, the current token not at all."""
    rng = _rng(40)
    q = _grid(rng, (2, 1, 3)).astype(np.float64)
    k = _grid(rng, (2, 1, 3)).astype(np.float64)
    v = _grid(rng, (2, 1, 4)).astype(np.float64)
    gamma = np.array([[0.75], [0.375]])
    _, s = orc.gret(q, k, v, gamma, want_state=True)
    want = gamma[1, 0] * np.outer(k[0, 0], v[0, 0]) + np.outer(k[1, 0], v[1, 0])
    _close(s[0], want, 1e-15, 1e-15, "gret two-token state")


def pin_gret_parallel_equals_recurrent(orc):
    """Eq. 4 (parallel) and Eq. 5 (recurrent) give the same outputs and final
    state, with and without a starting state."""
    rng = _rng(41)
    n, h, dk, dv = 23, 3, 5, 4
    q = rng.standard_normal((n, h, dk))
    k = rng.standard_normal((n, h, dk))
    v = rng.standard_normal((n, h, dv))
    gamma = rng.uniform(0.2, 1.0, (n, h))
    for s0 in (None, rng.standard_normal((h, dk, dv))):
        o, s = orc.gret(q, k, v, gamma, s_in=s0, want_state=True)
        st = np.zeros((1, h, dk, dv)) if s0 is None else s0[None].copy()
        for t in range(n):
            ot, st = orc.gret_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], gamma[t:t + 1], st)
            _close(o[t], ot[0], 1e-12, 1e-12, f"gret parallel vs recurrent, row {t}")
        _close(s, st[0], 1e-12, 1e-12, "gret parallel vs recurrent, final state")


def pin_gret_unit_gate_is_causal_linear_attention(orc):
    """With every gate 1 the decay matrix is the causal mask: O = tril(QK^T) V
    (numpy fp64), and the state is K^T V."""
    rng = _rng(42)
    n, h, dk, dv = 17, 2, 6, 5
    q = rng.standard_normal((n, h, dk))
    k = rng.standard_normal((n, h, dk))
    v = rng.standard_normal((n, h, dv))
    o, s = orc.gret(q, k, v, np.ones((n, h)), want_state=True)
    for hh in range(h):
        want = np.tril(q[:, hh] @ k[:, hh].T) @ v[:, hh]
        _close(o[:, hh], want, 1e-12, 1e-12, "gret unit gate outputs")
        _close(s[hh], k[:, hh].T @ v[:, hh], 1e-12, 1e-12, "gret unit gate state")


def pin_gret_zero_gate_keeps_current_token(orc):
    """With every gate 0 nothing survives a step: O_t = (q_t . k_t) v_t and the
    state is the last token's outer product."""
    rng = _rng(43)
    n, h, dk, dv = 9, 2, 4, 3
    q = rng.standard_normal((n, h, dk))
    k = rng.standard_normal((n, h, dk))
    v = rng.standard_normal((n, h, dv))
    s0 = rng.standard_normal((h, dk, dv))
    o, s = orc.gret(q, k, v, np.zeros((n, h)), s_in=s0, want_state=True)
    want = np.einsum("nhc,nhc->nh", q, k)[:, :, None] * v
    _close(o, want, 1e-13, 1e-13, "gret zero gate outputs")
    _close(s, np.einsum("hc,he->hce", k[-1], v[-1]), 1e-13, 1e-13, "gret zero gate state")


def pin_gret_block_split(orc):
    """Running a sequence as two blocks, the second starting from the first's
    final state, equals one block (rows and final state); rows can be sampled."""
    rng = _rng(44)
    n, h, dk, dv = 40, 2, 8, 8
    q = store(rng.standard_normal((n, h, dk)).astype(np.float32), BF16)
    k = store(rng.standard_normal((n, h, dk)).astype(np.float32), BF16)
    v = store(rng.standard_normal((n, h, dv)).astype(np.float32), BF16)
    gamma = rng.uniform(0.5, 1.0, (n, h))
    o, s = orc.gret(q, k, v, gamma, want_state=True)
    cut = 13
    o1, s1 = orc.gret(q[:cut], k[:cut], v[:cut], gamma[:cut], want_state=True)
    o2, s2 = orc.gret(q[cut:], k[cut:], v[cut:], gamma[cut:], s_in=s1, want_state=True)
    _close(np.concatenate([o1, o2]), o, 1e-12, 1e-12, "gret split outputs")
    _close(s2, s, 1e-12, 1e-12, "gret split state")
    rows = np.array([0, 5, 39, 12], dtype=np.int64)
    _close(orc.gret(q, k, v, gamma, rows=rows), o[rows], 0, 0, "gret sampled rows")


def pin_gret_gate_library(orc):
    """gamma = sigmoid(g)^(1/tau) against scipy's logistic function."""
    from scipy.special import expit
    g = np.array([-30.0, -4.0, -0.5, 0.0, 0.25, 3.0, 20.0], dtype=np.float32)
    for tau in (1.0, 16.0, 2.5):
        _close(orc.gret_gate(g, tau), expit(g.astype(np.float64)) ** (1.0 / tau), 1e-14, 0, f"gret gate tau={tau}")
    _close(orc.gret_gate(np.zeros(1, np.float32), 1.0), [0.5], 0, 0, "gret gate sigmoid(0)")


ALL_PINS = [
    pin_rmsnorm_constant_row,
    pin_rmsnorm_one_hot,
    pin_rmsnorm_library,
    pin_project_identity,
    pin_project_column_selector,
    pin_project_library,
    pin_attn_single_visible_key,
    pin_attn_identical_keys,
    pin_attn_two_keys_closed_form,
    pin_attn_gqa_head_mapping,
    pin_attn_gqa_equals_mha,
    pin_attn_prefix_invariance,
    pin_attn_causal_boundary,
    pin_attn_shift_invariance,
    pin_attn_v_affine,
    pin_attn_row_permutation,
    pin_attn_library,
    pin_decode_is_last_prefill_row,
    pin_rope_position_zero_is_identity,
    pin_rope_single_pair_closed_form,
    pin_rope_library_complex,
    pin_rope_preserves_norms,
    pin_rope_composition,
    pin_rope_scores_depend_on_offset,
    pin_rope_half_is_permuted_interleaved,
    pin_attn_bwd_finite_differences,
    pin_attn_bwd_library,
    pin_attn_bwd_sums,
    pin_attn_bwd_single_key,
    pin_attn_bwd_accumulates,
    pin_project_bwd_finite_differences,
    pin_project_bwd_scale_invariance,
    pin_project_bwd_library,
    pin_gret_worked_example, pin_gret_two_token_state, pin_gret_parallel_equals_recurrent,
    pin_gret_unit_gate_is_causal_linear_attention, pin_gret_zero_gate_keeps_current_token,
    pin_gret_block_split, pin_gret_gate_library,
]
