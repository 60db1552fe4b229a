"""MI355X-native shared-KV cross-decoder hot path of YOCO.

Thin Python binding over the C ABI declared in ``include/yoco.h`` (built as
``libyoco.so`` from ``csrc/``).  Every step of the path runs in the HIP
kernels; this module only passes pointers, sizes and the current stream.
PyTorch provides device memory and streams.

The functions mirror the C entry points:

* ``kv_project``      -> ``yoco_kv_project``   (RMSNorm + K^/V^ projection into the cache)
* ``kv_append``       -> ``yoco_kv_append``    (one new row per sequence)
* ``q_project``       -> ``yoco_q_project``    (per-layer RMSNorm + Q^ projection)
* ``cross_attn_prefill`` -> ``yoco_cross_attn_prefill`` (causal block over the cache)
* ``cross_attn_decode``  -> ``yoco_cross_attn_decode``  (one token per sequence, split-N)
* ``cross_attn_prefill_bwd`` -> ``yoco_cross_attn_prefill_bwd`` (training backward of one layer)
* ``kv_project_bwd`` / ``q_project_bwd`` -> ``yoco_kv_project_bwd`` / ``yoco_q_project_bwd``
  (backward of the fused RMSNorm + projections)
* ``gret_prefill`` / ``gret_decode`` -> ``yoco_gret_prefill`` / ``yoco_gret_decode``
  (gated retention, the self-decoder's token mixer: chunkwise block, recurrent step)
"""
from __future__ import annotations

import contextlib
import ctypes
import threading
from typing import Optional

import numpy as np
import torch

from ._native import (YOCO_DECODE_COUNTER_BYTES, YOCO_DT_BF16, YOCO_DT_F32, KVCacheStruct,
                      YocoError, check, lib)

__all__ = [
    "KVCache", "YocoError", "kv_project", "kv_append", "q_project", "cross_attn_prefill",
    "cross_attn_decode", "decode_workspace", "decode_workspace_bytes", "kv_cache_bytes",
    "kv_cache_row_stride", "lib", "project_workspace_bytes", "default_softmax_scale",
    "cross_attn_prefill_bwd", "prefill_bwd_workspace_bytes", "kv_project_bwd", "q_project_bwd",
    "project_bwd_workspace_bytes", "gret_prefill", "gret_decode", "gret_prefill_workspace_bytes",
    "cross_attn_decode_noalloc", "fold_norm_gain",
]

_DT = {torch.float32: YOCO_DT_F32, torch.bfloat16: YOCO_DT_BF16}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("inputs must be device tensors")


def _on(stream):
    """Temporaries of a call are allocated (and zero-filled) on the stream
    its kernels run on, so the fill is ordered before them and the caching
    allocator does not hand the memory to other streams while they run."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _check_shape(name: str, t: Optional[torch.Tensor], shape, dtype=None) -> None:
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_weights(d: int, ncols: int, gain, *ws) -> None:
    for w in ws:
        _check_shape("weight", w, (d, ncols))
    _check_shape("gain", gain, (d,), torch.float32)


# Few-row projection workspaces, one per (device, stream): calls on one
# stream never overlap, and the library leaves the arrival counters zero
# after each call, so a zero-filled buffer can be reused by every later call
# on its stream.
_scratch_lock = threading.Lock()
_scratch: dict = {}


def _stream_scratch(device: torch.device, stream, nbytes: int) -> Optional[torch.Tensor]:
    if nbytes <= 0:
        return None
    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = (device.index if device.index is not None else torch.cuda.current_device(), s.cuda_stream)
    with _scratch_lock:
        buf = _scratch.get(key)
        if buf is None or buf.numel() < nbytes:
            with torch.cuda.stream(s):
                buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            _scratch[key] = buf
        return buf


def _ws_args(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


class KVCache:
    """The one shared K^/V^ cache: k, v ``[n_seq, capacity, H_kv, d_h]`` on the
    device plus host lengths ``len`` (numpy int64, advanced by project/append).
    With ``padded`` (the default) each row is stored at the row stride
    ``yoco_kv_cache_row_stride`` recommends, so k and v are views into larger
    buffers whose rows end in a few unused elements."""

    def __init__(self, n_seq: int, capacity: int, n_kv_heads: int, head_dim: int,
                 dtype: torch.dtype = torch.bfloat16, device="cuda", zero: bool = False, padded: bool = True):
        alloc = torch.zeros if zero else torch.empty
        dense = n_kv_heads * head_dim
        rs = kv_cache_row_stride(n_kv_heads, head_dim, dtype) if padded else dense
        self._k_rows = alloc((n_seq, capacity, rs), dtype=dtype, device=device)
        self._v_rows = alloc((n_seq, capacity, rs), dtype=dtype, device=device)
        self.k = self._k_rows[:, :, :dense].unflatten(2, (n_kv_heads, head_dim))
        self.v = self._v_rows[:, :, :dense].unflatten(2, (n_kv_heads, head_dim))
        self.len = np.zeros(n_seq, dtype=np.int64)
        self.n_seq, self.capacity = n_seq, capacity
        self.n_kv_heads, self.head_dim, self.dtype = n_kv_heads, head_dim, dtype
        self.row_stride = rs
        self._struct = None
        self._key = None
        self._len_ref = None

    @classmethod
    def wrap(cls, k: torch.Tensor, v: torch.Tensor, lens) -> "KVCache":
        """Use existing k/v tensors ``[n_seq, capacity, H_kv, d_h]`` (dense, or
        rows padded: any stride along capacity, the rest packed)."""
        obj = cls.__new__(cls)
        if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4 or k.stride() != v.stride():
            raise ValueError("k and v must be matching [n_seq, capacity, H_kv, d_h] tensors")
        n_seq, cap, hkv, dh = k.shape
        # (the stride of a dimension of size 1 carries no layout: rows are
        # then dense, and one sequence needs no slab stride)
        rs = k.stride(1) if cap > 1 else (k.stride(0) if n_seq > 1 else hkv * dh)
        if (k.stride(3) != 1 or (hkv > 1 and k.stride(2) != dh) or rs < hkv * dh
                or (n_seq > 1 and k.stride(0) != cap * rs)):
            raise ValueError("k and v rows must be packed [H_kv, d_h] blocks at one row stride")
        obj.k, obj.v = k, v
        obj.n_seq, obj.capacity, obj.n_kv_heads, obj.head_dim = n_seq, cap, hkv, dh
        obj.dtype = k.dtype
        obj.row_stride = rs
        obj.len = np.ascontiguousarray(np.asarray(lens, dtype=np.int64).reshape(obj.n_seq))
        obj._struct = None
        obj._key = None
        obj._len_ref = None
        return obj

    def struct(self) -> KVCacheStruct:
        # The descriptor points at the tensors' storage and into ``len``; it is
        # rebuilt whenever one of them has been replaced.
        # ``len`` is compared by identity, and the descriptor keeps a reference
        # to the array its len_host points into, so a replaced array can never
        # be mistaken for the one the descriptor was built on.
        key = (self.k.data_ptr(), self.v.data_ptr(), self.capacity, self.n_seq)
        if self._struct is not None and self._key == key and self._len_ref is self.len:
            return self._struct
        _on_device(self.k, self.v)
        if self.len.dtype != np.int64 or not self.len.flags.c_contiguous or self.len.shape != (self.n_seq,):
            raise ValueError("len must be a contiguous int64 array of n_seq entries")
        s = KVCacheStruct()
        s.k = self.k.data_ptr()
        s.v = self.v.data_ptr()
        s.len_host = self.len.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        s.seq_capacity = self.capacity
        s.n_seq = self.n_seq
        s.n_kv_heads = self.n_kv_heads
        s.head_dim = self.head_dim
        s.dtype = _dt(self.k)
        s.row_stride = self.row_stride
        self._struct = s
        self._key = key
        self._len_ref = self.len  # keeps the array len_host points into alive
        return s


def kv_cache_bytes(n_seq: int, capacity: int, n_kv_heads: int, head_dim: int,
                   dtype: torch.dtype = torch.bfloat16, row_stride: int = 0) -> int:
    """Bytes of one of k / v (host-only; see ``yoco_kv_cache_bytes``)."""
    out = ctypes.c_size_t(0)
    check(lib().yoco_kv_cache_bytes(n_seq, capacity, n_kv_heads, head_dim, _DT.get(dtype, -1), row_stride,
                                    ctypes.byref(out)))
    return int(out.value)


def kv_cache_row_stride(n_kv_heads: int, head_dim: int, dtype: torch.dtype = torch.bfloat16) -> int:
    """Row stride (elements) the kernels stream fastest (``yoco_kv_cache_row_stride``)."""
    out = ctypes.c_int64(0)
    check(lib().yoco_kv_cache_row_stride(n_kv_heads, head_dim, _DT.get(dtype, -1), ctypes.byref(out)))
    return int(out.value)


def project_workspace_bytes(n: int, d_model: int, n_cols: int, n_out: int,
                            w_dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes of the few-row projection path (``yoco_project_workspace``;
    0 when these shapes do not use it)."""
    out = ctypes.c_size_t(0)
    check(lib().yoco_project_workspace(n, d_model, n_cols, n_out, _DT.get(w_dtype, -1), ctypes.byref(out)))
    return int(out.value)


def default_softmax_scale(head_dim: int) -> float:
    """The pages' softmax scale 1/sqrt(d_h) (``yoco_default_softmax_scale``)."""
    out = ctypes.c_float(0.0)
    check(lib().yoco_default_softmax_scale(head_dim, ctypes.byref(out)))
    return float(out.value)


def _proj_workspace(x: torch.Tensor, n: int, d: int, ncols: int, n_out: int, w: torch.Tensor, workspace, stream):
    """Workspace of a projection call: the caller's tensor; None (the
    default) for this stream's shared one when the call takes the few-row
    path; False for none (few rows then run on the kernel that needs no
    workspace)."""
    if workspace is False:
        return None
    if workspace is not None:
        return workspace
    return _stream_scratch(x.device, stream, project_workspace_bytes(n, d, ncols, n_out, w.dtype))


def kv_project(cache: KVCache, m: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor,
               gain: Optional[torch.Tensor] = None, eps: float = 1e-6, seq: int = 0,
               row_start: int = 0, stream=None, rope_theta: Optional[float] = None,
               workspace: Optional[torch.Tensor] = None) -> None:
    """RMSNorm(M) W_K and RMSNorm(M) W_V into cache rows [row_start, row_start+n);
    with ``rope_theta``, K^ row r is rotated at position row_start + r."""
    if m.dim() != 2:
        raise ValueError("m must be [n, d_model]")
    n, d = m.shape
    ncols = cache.n_kv_heads * cache.head_dim
    if w_k.dtype != w_v.dtype:
        raise TypeError("w_k and w_v must share a dtype")
    _check_weights(d, ncols, gain, w_k, w_v)
    _on_device(m, w_k, w_v, gain)
    s = cache.struct()
    ws, ws_bytes = _ws_args(_proj_workspace(m, n, d, ncols, 2, w_k, workspace, stream))
    args = (_ptr(m), _dt(m), n, d, _ptr(gain), eps, _ptr(w_k), _ptr(w_v), _dt(w_k), ctypes.byref(s), seq, row_start)
    if rope_theta is None:
        check(lib().yoco_kv_project(*args, ws, ws_bytes, _stream(stream)))
    else:
        check(lib().yoco_kv_project_rope(*args, float(rope_theta), ws, ws_bytes, _stream(stream)))


def kv_append(cache: KVCache, m_new: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor,
              gain: Optional[torch.Tensor] = None, eps: float = 1e-6, stream=None,
              rope_theta: Optional[float] = None, workspace: Optional[torch.Tensor] = None) -> None:
    """Project one new row per sequence (m_new ``[n_seq, d_model]``) and append it;
    with ``rope_theta``, the new K^ row of sequence b is rotated at position len[b]."""
    if m_new.dim() != 2 or m_new.shape[0] != cache.n_seq:
        raise ValueError(f"m_new must be [{cache.n_seq}, d_model] (one row per sequence), got {tuple(m_new.shape)}")
    d = m_new.shape[1]
    ncols = cache.n_kv_heads * cache.head_dim
    if w_k.dtype != w_v.dtype:
        raise TypeError("w_k and w_v must share a dtype")
    _check_weights(d, ncols, gain, w_k, w_v)
    _on_device(m_new, w_k, w_v, gain)
    s = cache.struct()
    ws, ws_bytes = _ws_args(_proj_workspace(m_new, cache.n_seq, d, ncols, 2, w_k, workspace, stream))
    args = (_ptr(m_new), _dt(m_new), d, _ptr(gain), eps, _ptr(w_k), _ptr(w_v), _dt(w_k), ctypes.byref(s))
    if rope_theta is None:
        check(lib().yoco_kv_append(*args, ws, ws_bytes, _stream(stream)))
    else:
        check(lib().yoco_kv_append_rope(*args, float(rope_theta), ws, ws_bytes, _stream(stream)))


def q_project(x: torch.Tensor, w_q: torch.Tensor, n_q_heads: int, head_dim: int,
              gain: Optional[torch.Tensor] = None, eps: float = 1e-6,
              out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
              stream=None, rope_theta: Optional[float] = None, positions=None,
              pos0: int = 0, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """RMSNorm_l(X) W_Q^l -> ``[n, H_q, d_h]``; with ``rope_theta``, row r is
    rotated at position ``positions[r]`` (host sequence) or pos0 + r."""
    if x.dim() != 2:
        raise ValueError("x must be [n, d_model]")
    n, d = x.shape
    ncols = n_q_heads * head_dim
    _check_weights(d, ncols, gain, w_q)
    if out is not None:
        _check_shape("out", out, (n, n_q_heads, head_dim))
    _on_device(x, w_q, gain, out)
    with _on(stream):
        if out is None:
            out = torch.empty((n, n_q_heads, head_dim), dtype=out_dtype or x.dtype, device=x.device)
        ws, ws_bytes = _ws_args(_proj_workspace(x, n, d, ncols, 1, w_q, workspace, stream))
    args = (_ptr(x), _dt(x), n, d, _ptr(gain), eps, _ptr(w_q), _dt(w_q), n_q_heads, head_dim, _ptr(out), _dt(out))
    if rope_theta is None:
        check(lib().yoco_q_project(*args, ws, ws_bytes, _stream(stream)))
    else:
        pos = None
        if positions is not None:
            pos = np.ascontiguousarray(positions, dtype=np.int64)
            if pos.shape != (n,):
                raise ValueError(f"positions must hold {n} entries")
        pos_ptr = None if pos is None else pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        check(lib().yoco_q_project_rope(*args, pos_ptr, int(pos0), float(rope_theta), ws, ws_bytes,
                                        _stream(stream)))
    return out


def fold_norm_gain(w: torch.Tensor, gain: torch.Tensor, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """diag(gain) W in bf16 (``[d_model, n_cols]``), each element the fp32
    product gain[c] * w[c][j] rounded once: the projections given it and no
    gain compute RMSNorm(x) W.  ``out`` may be ``w`` itself for a bf16 ``w``."""
    if w.dim() != 2:
        raise ValueError("w must be [d_model, n_cols]")
    d, ncols = w.shape
    if gain is None:
        raise ValueError("gain is required")
    _check_shape("gain", gain, (d,), torch.float32)
    if out is not None:
        _check_shape("out", out, (d, ncols), torch.bfloat16)
    _on_device(w, gain, out)
    with _on(stream):
        if out is None:
            out = torch.empty((d, ncols), dtype=torch.bfloat16, device=w.device)
    check(lib().yoco_fold_norm_gain(_ptr(w), _dt(w), _ptr(gain), d, ncols, _ptr(out), _stream(stream)))
    return out


def _scale(softmax_scale, head_dim: int) -> float:
    return default_softmax_scale(head_dim) if softmax_scale is None else float(softmax_scale)


def cross_attn_prefill(q: torch.Tensor, cache: KVCache, seq: int = 0, q_start: int = 0,
                       softmax_scale: Optional[float] = None,
                       out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                       want_lse: bool = False, stream=None, lse_out: Optional[torch.Tensor] = None):
    """Causal attention of q ``[t, H_q, d_h]`` (row i at position q_start+i)
    over sequence ``seq`` of the shared cache.  Returns o (and lse).  The
    scale defaults to the library's 1/sqrt(d_h)."""
    if q.dim() != 3 or q.shape[2] != cache.head_dim:
        raise ValueError(f"q must be [t, H_q, {cache.head_dim}], got {tuple(q.shape)}")
    t, hq, dh = q.shape
    if out is not None:
        _check_shape("out", out, (t, hq, dh))
    _check_shape("lse_out", lse_out, (t, hq), torch.float32)
    _on_device(q, out, lse_out)
    scale = _scale(softmax_scale, dh)
    with _on(stream):
        if out is None:
            out = torch.empty((t, hq, dh), dtype=out_dtype, device=q.device)
        lse = lse_out
        if lse is None and want_lse:
            lse = torch.empty((t, hq), dtype=torch.float32, device=q.device)
    s = cache.struct()
    check(lib().yoco_cross_attn_prefill(_ptr(q), _dt(q), q_start, t, hq, ctypes.byref(s), seq,
                                        scale, _ptr(out), _dt(out), _ptr(lse), _stream(stream)))
    return (out, lse) if (want_lse or lse_out is not None) else out


def prefill_bwd_workspace_bytes(t: int, n_q_heads: int) -> int:
    out = ctypes.c_size_t(0)
    check(lib().yoco_cross_attn_prefill_bwd_workspace(t, n_q_heads, ctypes.byref(out)))
    return int(out.value)


def cross_attn_prefill_bwd(q: torch.Tensor, o: torch.Tensor, d_o: torch.Tensor, lse: torch.Tensor,
                           cache: KVCache, seq: int = 0, q_start: int = 0,
                           softmax_scale: Optional[float] = None, d_q: Optional[torch.Tensor] = None,
                           d_k: Optional[torch.Tensor] = None, d_v: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward of ``cross_attn_prefill`` for one layer: returns (d_q, d_k,
    d_v).  d_k, d_v ``[q_start+t, H_kv, d_h]`` fp32 are ADDED to (zeros when
    not given), so passing the same tensors for every cross layer sums the
    layers' shares of the shared cache's gradient."""
    _on_device(q, o, d_o, lse)
    if q.dim() != 3 or q.shape[2] != cache.head_dim:
        raise ValueError(f"q must be [t, H_q, {cache.head_dim}], got {tuple(q.shape)}")
    t, hq, dh = q.shape
    _check_shape("o", o, (t, hq, dh))
    _check_shape("d_o", d_o, (t, hq, dh))
    scale = _scale(softmax_scale, dh)
    rows = q_start + t
    with _on(stream):
        if d_q is None:
            d_q = torch.empty((t, hq, dh), dtype=torch.float32, device=q.device)
        if d_k is None:
            d_k = torch.zeros((rows, cache.n_kv_heads, dh), dtype=torch.float32, device=q.device)
        if d_v is None:
            d_v = torch.zeros((rows, cache.n_kv_heads, dh), dtype=torch.float32, device=q.device)
    for name, x in (("d_q", d_q), ("d_k", d_k), ("d_v", d_v)):
        if x.dtype != torch.float32 or not x.is_contiguous():
            raise TypeError(f"{name} must be a contiguous float32 tensor")
    if d_k.shape != (rows, cache.n_kv_heads, dh) or d_v.shape != d_k.shape or d_q.shape != (t, hq, dh):
        raise ValueError("d_q must be [t, H_q, d_h]; d_k, d_v [q_start + t, H_kv, d_h]")
    if lse.dtype != torch.float32 or lse.shape != (t, hq):
        raise ValueError("lse must be the forward's float32 [t, H_q]")
    nbytes = prefill_bwd_workspace_bytes(t, hq)
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    s = cache.struct()
    check(lib().yoco_cross_attn_prefill_bwd(_ptr(q), _ptr(o), _dt(o), _ptr(d_o), _ptr(lse), q_start, t, hq,
                                            ctypes.byref(s), seq, scale, _ptr(d_q), _ptr(d_k), _ptr(d_v),
                                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(stream)))
    return d_q, d_k, d_v


def project_bwd_workspace_bytes(n: int, d_model: int, n_cols: int, n_out: int) -> int:
    out = ctypes.c_size_t(0)
    check(lib().yoco_project_bwd_workspace(n, d_model, n_cols, n_out, ctypes.byref(out)))
    return int(out.value)


def _grad_buffers(x, ws_bytes, weights, d_x, d_ws, d_gain, want_gain, workspace, stream):
    n, d = x.shape
    with _on(stream):
        if d_x is None:
            d_x = torch.empty((n, d), dtype=torch.float32, device=x.device)
        d_ws = [torch.zeros(w.shape, dtype=torch.float32, device=x.device) if g is None else g
                for w, g in zip(weights, d_ws)]
        if d_gain is None and want_gain:
            d_gain = torch.zeros(d, dtype=torch.float32, device=x.device)
    for name, t in [("d_x", d_x), ("d_gain", d_gain)] + [("d_w", g) for g in d_ws]:
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous float32 tensor")
    if d_x.shape != (n, d) or any(g.shape != w.shape for g, w in zip(d_ws, weights)):
        raise ValueError("d_x must be [n, d_model] and each d_w the shape of its weight")
    if d_gain is not None and d_gain.shape != (d,):
        raise ValueError("d_gain must be [d_model]")
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    return d_x, d_ws, d_gain, workspace


def kv_project_bwd(m: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor, dz_k: torch.Tensor,
                   dz_v: torch.Tensor, n_kv_heads: int, head_dim: int, gain: Optional[torch.Tensor] = None,
                   eps: float = 1e-6, d_m: Optional[torch.Tensor] = None, d_w_k: Optional[torch.Tensor] = None,
                   d_w_v: Optional[torch.Tensor] = None, d_gain: Optional[torch.Tensor] = None,
                   want_gain: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward of ``kv_project``: returns (d_m, d_w_k, d_w_v, d_gain).  d_m is
    written; d_w_k, d_w_v and d_gain are ADDED to (zeros when not given;
    d_gain is None unless given or ``want_gain``).  dz_k, dz_v:
    ``[n, H_kv, d_h]`` or ``[n, H_kv*d_h]``, float32 or bfloat16."""
    _on_device(m, w_k, w_v, dz_k, dz_v, gain)
    if w_k.dtype != w_v.dtype or dz_k.dtype != dz_v.dtype:
        raise TypeError("w_k/w_v and dz_k/dz_v must share a dtype")
    n, d = m.shape
    ncols = n_kv_heads * head_dim
    if dz_k.numel() != n * ncols or dz_v.numel() != n * ncols:
        raise ValueError(f"dz_k, dz_v must hold [n, {ncols}] values")
    ws_bytes = project_bwd_workspace_bytes(n, d, ncols, 2)
    d_m, (d_w_k, d_w_v), d_gain, workspace = _grad_buffers(m, ws_bytes, (w_k, w_v), d_m, (d_w_k, d_w_v), d_gain,
                                                           want_gain, workspace, stream)
    check(lib().yoco_kv_project_bwd(_ptr(m), _dt(m), n, d, _ptr(gain), eps, _ptr(w_k), _ptr(w_v), _dt(w_k),
                                    n_kv_heads, head_dim, _ptr(dz_k), _ptr(dz_v), _dt(dz_k), _ptr(d_m),
                                    _ptr(d_w_k), _ptr(d_w_v), _ptr(d_gain), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))
    return d_m, d_w_k, d_w_v, d_gain


def q_project_bwd(x: torch.Tensor, w_q: torch.Tensor, dz_q: torch.Tensor, n_q_heads: int, head_dim: int,
                  gain: Optional[torch.Tensor] = None, eps: float = 1e-6, d_x: Optional[torch.Tensor] = None,
                  d_w_q: Optional[torch.Tensor] = None, d_gain: Optional[torch.Tensor] = None,
                  want_gain: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward of ``q_project``: returns (d_x, d_w_q, d_gain), with the
    conventions of ``kv_project_bwd``."""
    _on_device(x, w_q, dz_q, gain)
    n, d = x.shape
    ncols = n_q_heads * head_dim
    if dz_q.numel() != n * ncols:
        raise ValueError(f"dz_q must hold [n, {ncols}] values")
    ws_bytes = project_bwd_workspace_bytes(n, d, ncols, 1)
    d_x, (d_w_q,), d_gain, workspace = _grad_buffers(x, ws_bytes, (w_q,), d_x, (d_w_q,), d_gain, want_gain,
                                                     workspace, stream)
    check(lib().yoco_q_project_bwd(_ptr(x), _dt(x), n, d, _ptr(gain), eps, _ptr(w_q), _dt(w_q), n_q_heads,
                                   head_dim, _ptr(dz_q), _dt(dz_q), _ptr(d_x), _ptr(d_w_q), _ptr(d_gain),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))
    return d_x, d_w_q, d_gain


def gret_prefill_workspace_bytes(n: int, n_heads: int, head_dim: int, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t(0)
    check(lib().yoco_gret_prefill_workspace(n, n_heads, head_dim, _DT.get(dtype, -1), ctypes.byref(out)))
    return int(out.value)


def gret_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate_logits: torch.Tensor, tau: float,
                 state_in: Optional[torch.Tensor] = None, want_state: bool = False,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Gated retention over a block: q, k, v ``[n, H, D]``, gate_logits
    ``[n, H]`` fp32, state_in ``[H, D, D]`` fp32 or None.  Returns o
    ``[n, H, D]`` fp32 (and the state after the block)."""
    _on_device(q, k, v, gate_logits, state_in)
    n, heads, dh = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must be matching [n, H, D] tensors")
    if gate_logits.dtype != torch.float32 or gate_logits.shape != (n, heads):
        raise ValueError("gate_logits must be float32 [n, H]")
    nbytes = gret_prefill_workspace_bytes(n, heads, dh, q.dtype)
    with _on(stream):
        if out is None:
            out = torch.empty((n, heads, dh), dtype=torch.float32, device=q.device)
        state_out = torch.empty((heads, dh, dh), dtype=torch.float32, device=q.device) if want_state else None
        if workspace is None and nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().yoco_gret_prefill(_ptr(q), _ptr(k), _ptr(v), _dt(q), _ptr(gate_logits), float(tau), n, heads, dh,
                                  _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(workspace), ws_bytes,
                                  _stream(stream)))
    return (out, state_out) if want_state else out


def gret_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate_logits: torch.Tensor, tau: float,
                state: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One recurrent step per sequence: q, k, v ``[B, H, D]``, gate_logits
    ``[B, H]``, state ``[B, H, D, D]`` fp32 updated in place.  Returns o."""
    _on_device(q, k, v, gate_logits, state)
    b, heads, dh = q.shape
    if state.dtype != torch.float32 or state.shape != (b, heads, dh, dh):
        raise ValueError("state must be float32 [B, H, D, D]")
    if out is None:
        with _on(stream):
            out = torch.empty((b, heads, dh), dtype=torch.float32, device=q.device)
    check(lib().yoco_gret_decode(_ptr(q), _ptr(k), _ptr(v), _dt(q), _ptr(gate_logits), float(tau), b, heads, dh,
                                 _ptr(state), _ptr(out), _stream(stream)))
    return out


def decode_workspace_bytes(cache: KVCache, n_q_heads: int, rows_per_split: int = 0) -> int:
    out = ctypes.c_size_t(0)
    s = cache.struct()
    check(lib().yoco_cross_attn_decode_workspace(ctypes.byref(s), n_q_heads, rows_per_split,
                                                 ctypes.byref(out)))
    return int(out.value)


def decode_workspace(cache: KVCache, n_q_heads: int, rows_per_split: int = 0, stream=None) -> torch.Tensor:
    """A zero-filled workspace large enough for any length up to capacity."""
    nbytes = decode_workspace_bytes(cache, n_q_heads, rows_per_split)
    with _on(stream):
        return torch.zeros(nbytes, dtype=torch.uint8, device=cache.k.device)


def cross_attn_decode(q: torch.Tensor, cache: KVCache, softmax_scale: Optional[float] = None,
                      workspace: Optional[torch.Tensor] = None, rows_per_split: int = 0,
                      out: Optional[torch.Tensor] = None, want_lse: bool = False, stream=None,
                      lse_out: Optional[torch.Tensor] = None):
    """One decode step of one cross layer: q ``[n_seq, H_q, d_h]`` at position
    len-1 of every sequence.  Returns o ``[n_seq, H_q, d_h]`` fp32 (and lse).
    The scale defaults to the library's 1/sqrt(d_h)."""
    if q.dim() != 3 or q.shape[0] != cache.n_seq or q.shape[2] != cache.head_dim:
        raise ValueError(f"q must be [{cache.n_seq}, H_q, {cache.head_dim}], got {tuple(q.shape)}")
    n_seq, hq, dh = q.shape
    _check_shape("out", out, (n_seq, hq, dh), torch.float32)
    _check_shape("lse_out", lse_out, (n_seq, hq), torch.float32)
    _on_device(q, out, lse_out, workspace)
    scale = _scale(softmax_scale, dh)
    with _on(stream):
        if workspace is None:
            workspace = decode_workspace(cache, hq, rows_per_split)
        if out is None:
            out = torch.empty((n_seq, hq, dh), dtype=torch.float32, device=q.device)
        lse = lse_out
        if lse is None and want_lse:
            lse = torch.empty((n_seq, hq), dtype=torch.float32, device=q.device)
    s = cache.struct()
    check(lib().yoco_cross_attn_decode(_ptr(q), _dt(q), hq, ctypes.byref(s), scale, _ptr(out),
                                       _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       rows_per_split, _stream(stream)))
    return (out, lse) if (want_lse or lse_out is not None) else out


def cross_attn_decode_noalloc(q: torch.Tensor, cache: KVCache, out: torch.Tensor,
                              softmax_scale: Optional[float] = None, rows_per_split: int = 0,
                              lse_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``cross_attn_decode`` through ``yoco_cross_attn_decode_noalloc``: no
    workspace, and nothing allocated here either (the caller passes ``out``
    ``[n_seq, H_q, d_h]`` fp32 and optionally ``lse_out`` ``[n_seq, H_q]``).
    Calls that overlap in time on one device race on the library's scratch."""
    if q.dim() != 3 or q.shape[0] != cache.n_seq or q.shape[2] != cache.head_dim:
        raise ValueError(f"q must be [{cache.n_seq}, H_q, {cache.head_dim}], got {tuple(q.shape)}")
    n_seq, hq, dh = q.shape
    _check_shape("out", out, (n_seq, hq, dh), torch.float32)
    _check_shape("lse_out", lse_out, (n_seq, hq), torch.float32)
    _on_device(q, out, lse_out)
    s = cache.struct()
    check(lib().yoco_cross_attn_decode_noalloc(_ptr(q), _dt(q), hq, ctypes.byref(s), _scale(softmax_scale, dh),
                                               _ptr(out), _ptr(lse_out), rows_per_split, _stream(stream)))
    return out
