"""fp64 CPU oracle for YOCO's cross-decoder hot path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never imports, links or
calls it, and it shares no code with that library.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over independent
query rows and heads).  This module only marshals numpy arrays to it:

* ``rmsnorm``     -- RMSNorm in fp64.
* ``project``     -- RMSNorm then ``@ W`` (the shared K^/V^ projection of the
                     YOCO reading notes, section 2.1, Eq. 2, and the per-layer
                     query projection of Eq. 3).
* ``attention``   -- causal GQA softmax attention of one query block over one
                     shared K/V slab (Eq. 3; the blog's section 2 formula).
* ``prefill`` / ``decode`` -- position bookkeeping around ``attention``.
* ``rope``        -- rotary position embedding of K^ / Q^ heads (the blog's
                     section 7: K^ and each layer's Q are rotated, V is not).
* ``attention_bwd`` -- gradients of ``attention`` with respect to the query,
                     K^ and V^ (K^/V^ gradients added, so layers sum).
* ``project_bwd`` -- gradients of the shared projection with respect to M,
                     the norm gain, W_K and W_V.
* ``gret_gate`` / ``gret`` / ``gret_step`` -- gated retention, the
                     self-decoder's token mixer (YOCO reading notes, section
                     2.2): the gate, the parallel form (Eq. 4, continuing from
                     a given state) and one step of the recurrent form (Eq. 5).

Inputs are the stored values: float32 arrays, bf16 kept as ``uint16`` bits,
or float64 (for finite-difference checks).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "oracle.c")
_LIB = os.path.join(_DIR, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``oracle.c`` (or a copy of it) with gcc: fp64, no fast-math,
    no contraction of multiply-add, OpenMP for the independent task loops."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs are float32, float64 or bf16 bits (uint16), got {a.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_f64(a: np.ndarray) -> np.ndarray:
    """Stored values (float32, or bf16 bits as uint16) widened exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


class Oracle:
    """Marshalling around one compiled copy of ``oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_num_threads.restype = i32
        lib.oracle_set_num_threads.argtypes = [i32]
        lib.oracle_rmsnorm.argtypes = [vp, i32, i64, i64, vp, dbl, vp]
        lib.oracle_matmul.argtypes = [vp, i64, i64, vp, i32, i64, vp]
        lib.oracle_project.argtypes = [vp, i32, i64, i64, vp, dbl, vp, i32, i64, vp]
        lib.oracle_project.restype = i32
        lib.oracle_attention.argtypes = [vp, i32, i64, vp, i32, vp, vp, i32, i64, i32, i32,
                                         dbl, vp, vp]
        lib.oracle_attention.restype = i32
        lib.oracle_rope.argtypes = [vp, i64, i32, i32, vp, dbl, i32]
        lib.oracle_attention_bwd.argtypes = [vp, i32, i64, vp, i32, vp, vp, i32, i64, i32, i32,
                                             vp, i32, dbl, vp, vp, vp]
        lib.oracle_attention_bwd.restype = i32
        lib.oracle_project_bwd.argtypes = [vp, i32, i64, i64, vp, dbl, vp, vp, i32, i64, vp, vp, i32,
                                           vp, vp, vp, vp]
        lib.oracle_project_bwd.restype = i32
        lib.oracle_gret_gate.argtypes = [vp, i64, dbl, vp]
        lib.oracle_gret.argtypes = [vp, vp, vp, i32, vp, i64, i32, i32, i32, vp, vp, i64, vp, vp]
        lib.oracle_gret.restype = i32
        lib.oracle_gret_step.argtypes = [vp, vp, vp, i32, vp, i64, i32, i32, i32, vp, vp]
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    def rmsnorm(self, x: np.ndarray, gain=None, eps: float = 1e-6) -> np.ndarray:
        """RMSNorm of the rows of ``x`` ([n, d]), fp64 result."""
        x = np.ascontiguousarray(x)
        n, d = x.shape
        y = np.empty((n, d), dtype=np.float64)
        g = None if gain is None else np.ascontiguousarray(gain, dtype=np.float32)
        self.lib.oracle_rmsnorm(_ptr(x), _code(x), n, d, None if g is None else _ptr(g),
                                eps, _ptr(y))
        return y

    def matmul(self, y: np.ndarray, w: np.ndarray) -> np.ndarray:
        """``y @ w``: y fp64 [n, d], w stored [d, ncols]; fp64 result."""
        y = np.ascontiguousarray(y, dtype=np.float64)
        w = np.ascontiguousarray(w)
        n, d = y.shape
        if w.shape[0] != d:
            raise ValueError("w must be [d, ncols]")
        out = np.empty((n, w.shape[1]), dtype=np.float64)
        self.lib.oracle_matmul(_ptr(y), n, d, _ptr(w), _code(w), w.shape[1], _ptr(out))
        return out

    def project(self, x: np.ndarray, w: np.ndarray, gain=None, eps: float = 1e-6) -> np.ndarray:
        """``RMSNorm(x) @ w`` in fp64: x [n, d], w [d, ncols] -> [n, ncols]."""
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w)
        n, d = x.shape
        if w.shape[0] != d:
            raise ValueError("w must be [d_model, ncols]")
        out = np.empty((n, w.shape[1]), dtype=np.float64)
        g = None if gain is None else np.ascontiguousarray(gain, dtype=np.float32)
        rc = self.lib.oracle_project(_ptr(x), _code(x), n, d, None if g is None else _ptr(g),
                                     eps, _ptr(w), _code(w), w.shape[1], _ptr(out))
        if rc != 0:
            raise MemoryError("oracle_project could not allocate scratch")
        return out

    def rope(self, x: np.ndarray, pos, theta: float, head_dim: int, interleaved: bool = True) -> np.ndarray:
        """Rotary position embedding of every head: x [n, H*d_h] or
        [n, H, d_h] (fp64 or stored values), row r at absolute position
        pos[r].  Returns an fp64 copy of the same shape."""
        shape = np.shape(x)
        n = shape[0]
        xd = np.array(x if np.asarray(x).dtype == np.float64 else _as_f64(x), dtype=np.float64).reshape(n, -1)
        if xd.shape[1] % head_dim or head_dim % 2:
            raise ValueError("row width must be a multiple of an even head_dim")
        heads = xd.shape[1] // head_dim
        pos = np.ascontiguousarray(np.broadcast_to(np.asarray(pos, dtype=np.int64), (n,)))
        xd = np.ascontiguousarray(xd)
        self.lib.oracle_rope(_ptr(xd), n, heads, head_dim, _ptr(pos), float(theta), 1 if interleaved else 0)
        return xd.reshape(shape)

    def attention(self, q: np.ndarray, pos, k: np.ndarray, v: np.ndarray, scale: float,
                  want_lse: bool = False):
        """Causal GQA attention.

        q: [n_q, H_q, d_h] stored values; pos: [n_q] absolute positions (query
        i reads rows 0..pos[i]); k, v: [rows, H_kv, d_h] stored values of one
        sequence.  Returns o [n_q, H_q, d_h] fp64 (and lse [n_q, H_q]).
        """
        q = np.ascontiguousarray(q)
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        if k.dtype != v.dtype:
            raise TypeError("k and v must share a storage type")
        n_q, hq, dh = q.shape
        rows, hkv, dhk = k.shape
        if v.shape != k.shape or dhk != dh:
            raise ValueError("shape mismatch between q, k and v")
        pos = np.ascontiguousarray(pos, dtype=np.int64).reshape(-1)
        if pos.shape[0] != n_q:
            raise ValueError("one position per query row")
        o = np.empty((n_q, hq, dh), dtype=np.float64)
        lse = np.empty((n_q, hq), dtype=np.float64) if want_lse else None
        rc = self.lib.oracle_attention(_ptr(q), _code(q), n_q, _ptr(pos), hq, _ptr(k), _ptr(v),
                                       _code(k), rows, hkv, dh, float(scale), _ptr(o),
                                       None if lse is None else _ptr(lse))
        if rc == -1:
            raise ValueError("bad attention arguments (H_q % H_kv, or a position outside the slab)")
        if rc != 0:
            raise MemoryError("oracle_attention could not allocate scratch")
        return (o, lse) if want_lse else o

    def attention_bwd(self, q: np.ndarray, pos, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                      scale: float, dk=None, dv=None):
        """Gradients of ``attention(q, pos, k, v, scale)`` for the upstream
        gradient ``dout`` ([n_q, H_q, d_h]).  Returns (dq, dk, dv) in fp64;
        dk, dv ([rows, H_kv, d_h]) are added to the given fp64 arrays (zeros
        if None), so that several layers, or disjoint query rows, sum."""
        q = np.ascontiguousarray(q)
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        dout = np.ascontiguousarray(dout)
        if k.dtype != v.dtype:
            raise TypeError("k and v must share a storage type")
        n_q, hq, dh = q.shape
        rows, hkv, dhk = k.shape
        if v.shape != k.shape or dhk != dh or dout.shape != q.shape:
            raise ValueError("shape mismatch between q, dout, k and v")
        pos = np.ascontiguousarray(pos, dtype=np.int64).reshape(-1)
        if pos.shape[0] != n_q:
            raise ValueError("one position per query row")
        dq = np.empty((n_q, hq, dh), dtype=np.float64)
        dk = np.zeros(k.shape, dtype=np.float64) if dk is None else dk
        dv = np.zeros(v.shape, dtype=np.float64) if dv is None else dv
        for a in (dk, dv):
            if a.dtype != np.float64 or a.shape != k.shape or not a.flags.c_contiguous:
                raise ValueError("dk, dv must be C-contiguous float64 [rows, H_kv, d_h]")
        rc = self.lib.oracle_attention_bwd(_ptr(q), _code(q), n_q, _ptr(pos), hq, _ptr(k), _ptr(v),
                                           _code(k), rows, hkv, dh, _ptr(dout), _code(dout),
                                           float(scale), _ptr(dq), _ptr(dk), _ptr(dv))
        if rc == -1:
            raise ValueError("bad attention arguments (H_q % H_kv, or a position outside the slab)")
        if rc != 0:
            raise MemoryError("oracle_attention_bwd could not allocate scratch")
        return dq, dk, dv

    def project_bwd(self, x: np.ndarray, w_k: np.ndarray, w_v: np.ndarray, dz_k: np.ndarray,
                    dz_v: np.ndarray, gain=None, eps: float = 1e-6):
        """Gradients of ``K^ = RMSNorm(x) W_K, V^ = RMSNorm(x) W_V`` for the
        upstream gradients dz_k, dz_v ([n, ncols], one storage type).
        Returns (dx [n, d], dw_k, dw_v [d, ncols], dgain [d] or None), fp64."""
        x = np.ascontiguousarray(x)
        w_k = np.ascontiguousarray(w_k)
        w_v = np.ascontiguousarray(w_v)
        dz_k = np.ascontiguousarray(dz_k)
        dz_v = np.ascontiguousarray(dz_v)
        n, d = x.shape
        if w_k.shape != w_v.shape or w_k.dtype != w_v.dtype or w_k.shape[0] != d:
            raise ValueError("w_k, w_v must be matching [d_model, ncols] arrays")
        ncols = w_k.shape[1]
        if dz_k.shape != (n, ncols) or dz_v.shape != (n, ncols) or dz_k.dtype != dz_v.dtype:
            raise ValueError("dz_k, dz_v must be matching [n, ncols] arrays")
        g = None if gain is None else np.ascontiguousarray(gain, dtype=np.float32)
        dx = np.empty((n, d), dtype=np.float64)
        dw_k = np.empty((d, ncols), dtype=np.float64)
        dw_v = np.empty((d, ncols), dtype=np.float64)
        dgain = None if g is None else np.empty(d, dtype=np.float64)
        rc = self.lib.oracle_project_bwd(_ptr(x), _code(x), n, d, None if g is None else _ptr(g), eps,
                                         _ptr(w_k), _ptr(w_v), _code(w_k), ncols, _ptr(dz_k), _ptr(dz_v),
                                         _code(dz_k), _ptr(dx), _ptr(dw_k), _ptr(dw_v),
                                         None if dgain is None else _ptr(dgain))
        if rc != 0:
            raise MemoryError("oracle_project_bwd could not allocate scratch")
        return dx, dw_k, dw_v, dgain

    def prefill(self, q: np.ndarray, q_start: int, k: np.ndarray, v: np.ndarray,
                scale: float, rows=None, want_lse: bool = False):
        """Causal prefill: query row i sits at position q_start + i.  ``rows``
        optionally selects which query rows to evaluate (sampled parity)."""
        if rows is None:
            rows = np.arange(q.shape[0], dtype=np.int64)
        rows = np.asarray(rows, dtype=np.int64)
        return self.attention(q[rows], q_start + rows, k, v, scale, want_lse)

    def decode(self, q: np.ndarray, length: int, k: np.ndarray, v: np.ndarray,
               scale: float, want_lse: bool = False):
        """Decode: every query row (e.g. one per cross layer) sits at position
        length - 1 and reads cache rows 0..length-1."""
        pos = np.full(q.shape[0], length - 1, dtype=np.int64)
        return self.attention(q, pos, k[:length], v[:length], scale, want_lse)

    def gret_gate(self, g: np.ndarray, tau: float) -> np.ndarray:
        """gamma = sigmoid(g)^(1/tau) in fp64 (g: float32 gate logits)."""
        g = np.ascontiguousarray(g, dtype=np.float32)
        out = np.empty(g.shape, dtype=np.float64)
        self.lib.oracle_gret_gate(_ptr(g), g.size, float(tau), _ptr(out))
        return out

    def gret(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, gamma: np.ndarray, s_in=None,
             rows=None, want_state: bool = False):
        """Gated retention, parallel form, over a block: q, k ``[n, H, dk]``,
        v ``[n, H, dv]`` (one storage type), gamma ``[n, H]`` fp64, s_in
        ``[H, dk, dv]`` (the state before the block) or None.  Returns o
        ``[n_rows, H, dv]`` (and the state after the block)."""
        q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
        n, heads, dk = q.shape
        dv = v.shape[2]
        if k.shape != q.shape or v.shape[:2] != (n, heads) or q.dtype != k.dtype or k.dtype != v.dtype:
            raise ValueError("q, k must be [n, H, dk] and v [n, H, dv] of one dtype")
        gamma = np.ascontiguousarray(gamma, dtype=np.float64)
        if gamma.shape != (n, heads):
            raise ValueError("gamma must be [n, H]")
        sp = None
        if s_in is not None:
            s_in = np.ascontiguousarray(s_in, dtype=np.float64)
            if s_in.shape != (heads, dk, dv):
                raise ValueError("s_in must be [H, dk, dv]")
            sp = _ptr(s_in)
        r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = n if r is None else r.size
        o = np.empty((n_rows, heads, dv), dtype=np.float64)
        s_out = np.empty((heads, dk, dv), dtype=np.float64) if want_state else None
        rc = self.lib.oracle_gret(_ptr(q), _ptr(k), _ptr(v), _code(q), _ptr(gamma), n, heads, dk, dv, sp,
                                  None if r is None else _ptr(r), n_rows, _ptr(o),
                                  None if s_out is None else _ptr(s_out))
        if rc != 0:
            raise ValueError("a row outside the block")
        return (o, s_out) if want_state else o

    def gret_step(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, gamma: np.ndarray, state: np.ndarray):
        """One recurrent step for each sequence: q, k ``[B, H, dk]``, v
        ``[B, H, dv]``, gamma ``[B, H]``, state ``[B, H, dk, dv]`` fp64.
        Returns (o ``[B, H, dv]``, the updated state)."""
        q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
        b, heads, dk = q.shape
        dv = v.shape[2]
        st = np.array(state, dtype=np.float64, copy=True, order="C")
        if st.shape != (b, heads, dk, dv):
            raise ValueError("state must be [B, H, dk, dv]")
        gamma = np.ascontiguousarray(gamma, dtype=np.float64)
        o = np.empty((b, heads, dv), dtype=np.float64)
        self.lib.oracle_gret_step(_ptr(q), _ptr(k), _ptr(v), _code(q), _ptr(gamma), b, heads, dk, dv,
                                  _ptr(st), _ptr(o))
        return o, st


def default() -> Oracle:
    """The oracle built from ``oracle.c`` beside this file (built if stale)."""
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            _lib = Oracle(_LIB)
        return _lib


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def rmsnorm(x, gain=None, eps: float = 1e-6):
    return default().rmsnorm(x, gain, eps)


def matmul(y, w):
    return default().matmul(y, w)


def project(x, w, gain=None, eps: float = 1e-6):
    return default().project(x, w, gain, eps)


def rope(x, pos, theta, head_dim, interleaved=True):
    return default().rope(x, pos, theta, head_dim, interleaved)


def attention(q, pos, k, v, scale, want_lse: bool = False):
    return default().attention(q, pos, k, v, scale, want_lse)


def prefill(q, q_start, k, v, scale, rows=None, want_lse: bool = False):
    return default().prefill(q, q_start, k, v, scale, rows, want_lse)


def decode(q, length, k, v, scale, want_lse: bool = False):
    return default().decode(q, length, k, v, scale, want_lse)


def attention_bwd(q, pos, k, v, dout, scale, dk=None, dv=None):
    return default().attention_bwd(q, pos, k, v, dout, scale, dk, dv)


def project_bwd(x, w_k, w_v, dz_k, dz_v, gain=None, eps: float = 1e-6):
    return default().project_bwd(x, w_k, w_v, dz_k, dz_v, gain, eps)


def gret_gate(g, tau):
    return default().gret_gate(g, tau)


def gret(q, k, v, gamma, s_in=None, rows=None, want_state: bool = False):
    return default().gret(q, k, v, gamma, s_in, rows, want_state)


def gret_step(q, k, v, gamma, state):
    return default().gret_step(q, k, v, gamma, state)
