"""Seeded synthetic inputs for the shared-KV cross-decoder path.

This module only draws and stores numbers.  It holds none of the method's
arithmetic (no normalisation, projection or attention): both the fp64 oracle
and the HIP library consume exactly the values it returns.

Conventions
-----------
* Generator: PCG64 (numpy), seed 0 unless stated.  Each tensor is a numbered
  *stream*; its elements (row-major) are drawn in chunks of 2**22, chunk i of
  stream s from ``PCG64(SeedSequence(seed, spawn_key=(s, i)))`` with
  ``standard_normal(dtype=float32)``.  Chunks are filled on several threads;
  the values do not depend on the thread count.  Small integer draws (ragged
  lengths, needle rows, peaked rows) use their own numbered streams.
* Values are drawn in float32 and then stored in the workload's dtype.  For
  bf16 the stored value is the round-to-nearest-even bf16 of the float32 draw,
  kept as raw ``uint16`` bits; the oracle reads those bits, never the draw.
* Shapes follow the YOCO-3B cross-decoder ("NeurIPS'24 | YOCO" blog, section 7
  shape table): shared K/V ``[rows, 8, 128]``, per-layer queries
  ``[tokens, 24, 128]``, 13 cross layers.

Each ``make_*`` function documents its draw order; changing that order changes
every stored value, so it is part of the contract.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

_CHUNK = 1 << 22
_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))


def _pool_map(fn, n):
    if n <= 1:
        for i in range(n):
            fn(i)
        return
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(_THREADS, n)) as ex:
        list(ex.map(fn, range(n)))

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    The inputs here are finite normal draws, so no NaN handling is needed; an
    infinite or NaN input raises.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value in a synthetic input")
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1).view(np.uint32), out.reshape(-1)

    for s in range(0, flat_in.size, _CHUNK):
        # finite values are <= 0xFF7FFFFF, so adding at most 0x8000 stays in uint32
        u = flat_in[s:s + _CHUNK].copy()
        lsb = (u >> 16) & 1
        u += 0x7FFF
        u += lsb
        u >>= 16
        flat_out[s:s + _CHUNK] = u
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32 (for host-side checks)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 draws in ``dtype``: float32 stays, bf16 becomes uint16 bits."""
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def as_f32(x: np.ndarray) -> np.ndarray:
    """Stored values (float32 or bf16 bits) widened to float32."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=np.float32)


def _normal(seed: int, stream: int, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) float32 draws of one numbered stream (see module notes)."""
    x = np.empty(shape, dtype=np.float32)
    flat = x.reshape(-1)

    def fill(i):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, i))))
        g.standard_normal(out=flat[i * _CHUNK:(i + 1) * _CHUNK], dtype=np.float32)
        if std != 1.0:
            flat[i * _CHUNK:(i + 1) * _CHUNK] *= np.float32(std)

    _pool_map(fill, (flat.size + _CHUNK - 1) // _CHUNK)
    return x


def _int_rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream,))))


# ---------------------------------------------------------------------------
# Workload 1: the tiny fp32 end-to-end case.
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class TinyCase:
    """One cross layer, 256 prompt tokens plus one generated token, fp32.

    d_model=256, H_q=4, H_kv=2 (GQA group 2), d_h=64.  M, X ~ N(0,1);
    W_K, W_V, W_Q ~ N(0, 1/d_model); RMSNorm gain 1, eps 1e-6.
    Streams: 1 M[257,256], 2 X[257,256], 3 W_K[256,128], 4 W_V[256,128],
    5 W_Q[256,256].
    Row 256 of M and X is the generated token (position 257 counted from 1).
    """
    m: np.ndarray
    x: np.ndarray
    w_k: np.ndarray
    w_v: np.ndarray
    w_q: np.ndarray
    gain_kv: np.ndarray
    gain_q: np.ndarray
    n_prompt: int = 256
    d_model: int = 256
    n_q_heads: int = 4
    n_kv_heads: int = 2
    head_dim: int = 64
    eps: float = 1e-6
    dtype: str = F32

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def make_tiny(seed: int = 0) -> TinyCase:
    d, hq, hkv, dh, n = 256, 4, 2, 64, 256
    m = _normal(seed, 1, (n + 1, d))
    x = _normal(seed, 2, (n + 1, d))
    std = 1.0 / math.sqrt(d)
    w_k = _normal(seed, 3, (d, hkv * dh), std)
    w_v = _normal(seed, 4, (d, hkv * dh), std)
    w_q = _normal(seed, 5, (d, hq * dh), std)
    ones = np.ones(d, dtype=np.float32)
    return TinyCase(m=m, x=x, w_k=w_k, w_v=w_v, w_q=w_q, gain_kv=ones, gain_q=ones.copy())


# ---------------------------------------------------------------------------
# Decode workloads: one shared cache, 13 cross layers each with its own query.
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class DecodeCase:
    """Shared K/V slabs plus 13 layers of single-token queries per sequence.

    k, v: per-sequence arrays ``[len_b, H_kv, d_h]`` (stored dtype).
    q:    ``[layers, n_seq, H_q, d_h]`` (stored dtype).
    needle_pos: for the planted-needle case, ``[n_seq, H_kv]`` row indices.
    """
    k: list
    v: list
    q: np.ndarray
    lens: np.ndarray
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    layers: int
    dtype: str
    needle_pos: Optional[np.ndarray] = None

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def n_seq(self) -> int:
        return len(self.k)


def make_decode(n_rows: int = 131072, n_q_heads: int = 24, n_kv_heads: int = 8,
                head_dim: int = 128, layers: int = 13, dtype: str = BF16,
                seed: int = 0) -> DecodeCase:
    """Single-sequence decode: K, V ``[n_rows, H_kv, d_h]`` and Q
    ``[layers, 1, H_q, d_h]``, all N(0,1).  Streams: 1 K, 2 V, 3 Q.

    The default sizes are the 128 Ki-token decode workload (cache
    2*131072*8*128*2 B = 512 MiB in bf16).
    """
    k = store(_normal(seed, 1, (n_rows, n_kv_heads, head_dim)), dtype)
    v = store(_normal(seed, 2, (n_rows, n_kv_heads, head_dim)), dtype)
    q = store(_normal(seed, 3, (layers, 1, n_q_heads, head_dim)), dtype)
    return DecodeCase(k=[k], v=[v], q=q, lens=np.array([n_rows], dtype=np.int64),
                      n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
                      layers=layers, dtype=dtype)


RAGGED_LO, RAGGED_HI = 8192, 131072


def ragged_lengths(n_seq: int = 16, lo: int = RAGGED_LO, hi: int = RAGGED_HI,
                   seed: int = 0) -> np.ndarray:
    """Per-sequence cache lengths, integers uniform on [lo, hi] inclusive.
    This is the first draw of the ragged workload's generator."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, n_seq, endpoint=True).astype(np.int64)


def make_ragged_decode(n_seq: int = 16, lo: int = RAGGED_LO, hi: int = RAGGED_HI,
                       n_q_heads: int = 24, n_kv_heads: int = 8, head_dim: int = 128,
                       layers: int = 13, dtype: str = BF16, seed: int = 0) -> DecodeCase:
    """Ragged batched decode.  Lengths: ``ragged_lengths`` (the first draw of
    ``default_rng(seed)``).  Streams: 1 Q ``[layers, n_seq, H_q, d_h]``;
    100 + 2b K_b ``[L_b, H_kv, d_h]``; 101 + 2b V_b.  All values N(0,1)."""
    lens = ragged_lengths(n_seq, lo, hi, seed)
    q = store(_normal(seed, 1, (layers, n_seq, n_q_heads, head_dim)), dtype)
    ks, vs = [], []
    for b in range(n_seq):
        ks.append(store(_normal(seed, 100 + 2 * b, (int(lens[b]), n_kv_heads, head_dim)), dtype))
        vs.append(store(_normal(seed, 101 + 2 * b, (int(lens[b]), n_kv_heads, head_dim)), dtype))
    return DecodeCase(k=ks, v=vs, q=q, lens=lens, n_q_heads=n_q_heads,
                      n_kv_heads=n_kv_heads, head_dim=head_dim, layers=layers, dtype=dtype)


NEEDLE_SIGMAS = 12.0


def make_needle_decode(n_rows: int = 1 << 20, n_q_heads: int = 24, n_kv_heads: int = 8,
                       head_dim: int = 128, layers: int = 13, dtype: str = BF16,
                       seed: int = 0, sigmas: float = NEEDLE_SIGMAS) -> DecodeCase:
    """Long-context decode with one planted needle key per KV head.

    Streams: 1 K, 2 V ``[n_rows, H_kv, d_h]``, 3 Q ``[layers, 1, H_q, d_h]``
    (all N(0,1)); stream 4 draws, for g = 0..H_kv-1 in turn, the needle row
    p_g = integers(0, n_rows).

    The needle for KV head g replaces K[p_g, g] by the minimum-norm vector k
    with q.k = sigmas * ||q|| for every stored query q of that group (all
    layers, all G heads; layers*G <= d_h so the system is solvable).  Since
    q.k' for k' ~ N(0, I) has standard deviation ||q||, this plants a key that
    sits ``sigmas`` standard deviations above the background for every one of
    those queries.  The solve runs in float64 on the stored queries; the result
    is stored like every other value.
    """
    kf = _normal(seed, 1, (n_rows, n_kv_heads, head_dim))
    vf = _normal(seed, 2, (n_rows, n_kv_heads, head_dim))
    q = store(_normal(seed, 3, (layers, 1, n_q_heads, head_dim)), dtype)
    rng = _int_rng(seed, 4)
    qf = as_f32(q).astype(np.float64)
    g_size = n_q_heads // n_kv_heads
    pos = np.zeros((1, n_kv_heads), dtype=np.int64)
    for g in range(n_kv_heads):
        p = int(rng.integers(0, n_rows))
        pos[0, g] = p
        a = qf[:, 0, g * g_size:(g + 1) * g_size, :].reshape(-1, head_dim)
        rhs = sigmas * np.linalg.norm(a, axis=1)
        needle, *_ = np.linalg.lstsq(a, rhs, rcond=None)
        kf[p, g, :] = needle.astype(np.float32)
    k = store(kf, dtype)
    del kf
    v = store(vf, dtype)
    del vf
    return DecodeCase(k=[k], v=[v], q=q, lens=np.array([n_rows], dtype=np.int64),
                      n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
                      layers=layers, dtype=dtype, needle_pos=pos)


# ---------------------------------------------------------------------------
# Prefill workload: one layer's queries against the shared cache, causal.
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class PrefillCase:
    """q ``[t, H_q, d_h]``, k/v ``[n_rows, H_kv, d_h]``; query row i sits at
    absolute position q_start + i."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_start: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    peaked_rows: Optional[np.ndarray] = None

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def t(self) -> int:
        return self.q.shape[0]


PEAK_FRACTION = 0.01
PEAK_SCALE = 8.0


def make_prefill(n: int = 32768, n_q_heads: int = 24, n_kv_heads: int = 8,
                 head_dim: int = 128, dtype: str = BF16, seed: int = 0,
                 peak_fraction: float = PEAK_FRACTION, peak_scale: float = PEAK_SCALE,
                 q_start: int = 0, t: Optional[int] = None) -> PrefillCase:
    """Causal full-sequence cross-attention input.

    Streams: 1 Q ``[t, H_q, d_h]``, 2 K ``[n, H_kv, d_h]``, 3 V (all N(0,1));
    stream 4 draws floor(peak_fraction*n) distinct rows
    ``choice(n, ., replace=False)`` whose
    keys (all KV heads) are multiplied by ``peak_scale`` to make peaked softmax
    rows.  A power-of-two scale is exact in bf16, so scaling before or after
    rounding stores the same value.  ``t`` defaults to ``n - q_start``.
    """
    if t is None:
        t = n - q_start
    qf = _normal(seed, 1, (t, n_q_heads, head_dim))
    kf = _normal(seed, 2, (n, n_kv_heads, head_dim))
    vf = _normal(seed, 3, (n, n_kv_heads, head_dim))
    n_peak = int(math.floor(peak_fraction * n))
    rng = _int_rng(seed, 4)
    peaked = np.sort(rng.choice(n, n_peak, replace=False)) if n_peak > 0 else np.zeros(0, np.int64)
    kf[peaked] *= np.float32(peak_scale)
    return PrefillCase(q=store(qf, dtype), k=store(kf, dtype), v=store(vf, dtype),
                       q_start=q_start, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                       head_dim=head_dim, dtype=dtype, peaked_rows=peaked)


def make_grad(t: int, n_q_heads: int = 24, head_dim: int = 128, dtype: str = BF16, seed: int = 0,
              layers: int = 1) -> list:
    """Upstream gradients dO of the attention output for ``layers`` cross
    layers: stream 10 + l, ``[t, H_q, d_h]`` N(0,1) each (a stand-in for the
    gradient a loss would send back; no trained model here)."""
    return [store(_normal(seed, 10 + l, (t, n_q_heads, head_dim)), dtype) for l in range(layers)]


def make_proj_grad(n: int, n_cols: int, n_out: int = 2, dtype: str = F32, seed: int = 0) -> list:
    """Upstream gradients dz_p ``[n, n_cols]`` of the projection outputs
    (p < n_out; K^ then V^, or Q^): stream 20 + p, N(0,1) each (a stand-in for
    what the cross layers' backward sends to the shared projection)."""
    return [store(_normal(seed, 20 + p, (n, n_cols)), dtype) for p in range(n_out)]


# ---------------------------------------------------------------------------
# Projection workload at 3B-like widths.
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class ProjectCase:
    m: np.ndarray       # [n, d_model]
    w_k: np.ndarray     # [d_model, H_kv*d_h]
    w_v: np.ndarray
    gain: np.ndarray    # [d_model] float32
    n_kv_heads: int
    head_dim: int
    eps: float
    dtype: str


def make_project(n: int = 32768, d_model: int = 3072, n_kv_heads: int = 8,
                 head_dim: int = 128, dtype: str = BF16, seed: int = 0,
                 eps: float = 1e-6, unit_gain: bool = True) -> ProjectCase:
    """M ``[n, d_model]`` ~ N(0,1); W_K, W_V ``[d_model, H_kv*d_h]`` ~
    N(0, 1/d_model).  Streams: 1 M, 2 W_K, 3 W_V, 4 (if not unit_gain) the
    RMSNorm gain ~ 1 + 0.1 N(0,1)."""
    m = store(_normal(seed, 1, (n, d_model)), dtype)
    std = 1.0 / math.sqrt(d_model)
    w_k = store(_normal(seed, 2, (d_model, n_kv_heads * head_dim), std), dtype)
    w_v = store(_normal(seed, 3, (d_model, n_kv_heads * head_dim), std), dtype)
    if unit_gain:
        gain = np.ones(d_model, dtype=np.float32)
    else:
        gain = (1.0 + 0.1 * _normal(seed, 4, (d_model,))).astype(np.float32)
    return ProjectCase(m=m, w_k=w_k, w_v=w_v, gain=gain, n_kv_heads=n_kv_heads,
                       head_dim=head_dim, eps=eps, dtype=dtype)


# Sizes of the named workloads, used by tests and the benchmark.
DECODE_128K = dict(n_rows=131072, n_q_heads=24, n_kv_heads=8, head_dim=128, layers=13)
PREFILL_32K = dict(n=32768, n_q_heads=24, n_kv_heads=8, head_dim=128)
RAGGED_16 = dict(n_seq=16, lo=RAGGED_LO, hi=RAGGED_HI, n_q_heads=24, n_kv_heads=8,
                 head_dim=128, layers=13)
NEEDLE_1M = dict(n_rows=1 << 20, n_q_heads=24, n_kv_heads=8, head_dim=128, layers=13)
PROJECT_3B = dict(n=32768, d_model=3072, n_kv_heads=8, head_dim=128)


# ---------------------------------------------------------------------------
# Gated retention (self-decoder token mixer) at the 3B shapes: 24 heads of
# 128 ([Blog] s.7: each self layer keeps a [24, 128, 128] state).
# ---------------------------------------------------------------------------
GRET_TAU = 16.0  # the pages give tau no value; 16 is the reading taken


@dataclasses.dataclass
class GretCase:
    q: np.ndarray       # [n, H, D]
    k: np.ndarray       # [n, H, D], scaled by D^-1/2 before storing
    v: np.ndarray       # [n, H, D]
    gate: np.ndarray    # [n, H] float32 logits
    tau: float
    dtype: str


def make_gret(n: int = 32768, n_heads: int = 24, head_dim: int = 128, dtype: str = BF16, seed: int = 0,
              tau: float = GRET_TAU, gate_mean: float = 0.0) -> GretCase:
    """q, v ~ N(0,1); k ~ N(0,1) / sqrt(D); gate logits ~ N(gate_mean, 1).
    Streams 30 q, 31 k, 32 v, 33 gate."""
    q = store(_normal(seed, 30, (n, n_heads, head_dim)), dtype)
    k = store(_normal(seed, 31, (n, n_heads, head_dim), 1.0 / math.sqrt(head_dim)), dtype)
    v = store(_normal(seed, 32, (n, n_heads, head_dim)), dtype)
    gate = (gate_mean + _normal(seed, 33, (n, n_heads))).astype(np.float32)
    return GretCase(q=q, k=k, v=v, gate=gate, tau=tau, dtype=dtype)


GRET_32K = dict(n=32768, n_heads=24, head_dim=128)
