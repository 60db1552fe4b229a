"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments before it touches the GPU (no compute calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

from tests.conftest import ROOT, gpu_available

HEADER = os.path.join(ROOT, "include", "yoco.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "cache_sizes.txt")


def _lib():
    from yoco_shared_kv_amd._native import lib
    return lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(yoco_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib()
    names = _declared_functions()
    assert len(names) == 25, names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in yoco.h but not exported"


def test_abi_version_matches_header():
    ver = int(re.search(r"#define YOCO_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert _lib().yoco_abi_version() == ver


def test_kv_cache_bytes_matches_printed_size():
    import yoco_shared_kv_amd as y
    import torch
    per_tensor = y.kv_cache_bytes(1, 131072, 8, 128, torch.bfloat16)
    golden = {}
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            name, value, unit = line.split()
            golden[name] = float(value) * {"GiB": 2 ** 30, "MiB": 2 ** 20}[unit]
    assert 2 * per_tensor == golden["yoco_shared_kv"]
    assert y.kv_cache_bytes(1, 1, 1, 64, torch.float32) == 256
    with pytest.raises(y.YocoError) as e:
        y.kv_cache_bytes(0, 1, 1, 64)
    assert e.value.name == "YOCO_ERR_BAD_SHAPE"


def test_cache_row_stride_rule():
    """Rows of >= 1 KiB whose size is a multiple of 512 B get 128 B of padding;
    others stay dense.  The byte count follows the stride; bad strides are
    rejected."""
    import yoco_shared_kv_amd as y
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    assert y.kv_cache_row_stride(8, 128, bf) == 8 * 128 + 64       # 2048 B rows -> 2176 B
    assert y.kv_cache_row_stride(4, 128, bf) == 4 * 128 + 64       # 1 KiB
    assert y.kv_cache_row_stride(8, 128, f32) == 8 * 128 + 32      # 4 KiB rows, 128 B of fp32
    assert y.kv_cache_row_stride(2, 128, bf) == 2 * 128            # 512 B: dense
    assert y.kv_cache_row_stride(1, 128, bf) == 128
    assert y.kv_cache_row_stride(3, 128, bf) == 3 * 128            # 768 B: not a multiple of 512
    assert y.kv_cache_row_stride(6, 128, bf) == 6 * 128 + 64       # 1536 B
    assert y.kv_cache_bytes(1, 131072, 8, 128, bf, row_stride=1088) == 131072 * 1088 * 2
    assert y.kv_cache_bytes(2, 10, 8, 128, f32, row_stride=0) == 2 * 10 * 1024 * 4
    for rs in (1023, 1028, (1 << 20) + 8, -8):                     # short, not 16 B, too long, negative
        with pytest.raises(y.YocoError) as e:
            y.kv_cache_bytes(1, 10, 8, 128, bf, row_stride=rs)
        assert e.value.name == "YOCO_ERR_BAD_SHAPE"
    c, lens = _cache(hkv=2, dh=64)
    c.row_stride = 130                                             # 260 B rows: not a multiple of 16 B
    assert _project(c) == _status("YOCO_ERR_BAD_SHAPE")
    c.row_stride = 64                                              # shorter than the 128-element row
    assert _project(c) == _status("YOCO_ERR_BAD_SHAPE")
    assert lens.tolist() == [10, 20]


# ---- error paths with placeholder pointers (never dereferenced) ----------
FAKE = ctypes.c_void_p(0x1000)


def _cache(n_seq=2, cap=64, hkv=2, dh=64, dtype=1, lens=(10, 20)):
    from yoco_shared_kv_amd._native import KVCacheStruct
    lens_arr = np.array(lens, dtype=np.int64)
    c = KVCacheStruct()
    c.k, c.v = 0x2000, 0x3000
    c.len_host = lens_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    c.seq_capacity, c.n_seq, c.n_kv_heads, c.head_dim, c.dtype = cap, n_seq, hkv, dh, dtype
    return c, lens_arr


def _status(name):
    from yoco_shared_kv_amd._native import STATUS
    return {v: k for k, v in STATUS.items()}[name]


def _project(c, **kw):
    args = dict(m=FAKE, m_dt=1, n=4, d=32, gain=None, eps=1e-6, wk=FAKE, wv=FAKE, w_dt=1, seq=0, row_start=0,
                ws=None, ws_bytes=0)
    args.update(kw)
    return _lib().yoco_kv_project(args["m"], args["m_dt"], args["n"], args["d"], args["gain"], args["eps"],
                                  args["wk"], args["wv"], args["w_dt"], ctypes.byref(c), args["seq"],
                                  args["row_start"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(m=None), "YOCO_ERR_NULL_POINTER"),
    (dict(wv=None), "YOCO_ERR_NULL_POINTER"),
    (dict(d=0), "YOCO_ERR_BAD_SHAPE"),
    (dict(seq=2), "YOCO_ERR_BAD_SHAPE"),
    (dict(m_dt=5), "YOCO_ERR_BAD_DTYPE"),
    (dict(eps=-1.0), "YOCO_ERR_BAD_VALUE"),
    (dict(eps=float("nan")), "YOCO_ERR_BAD_VALUE"),
    (dict(row_start=61), "YOCO_ERR_OUT_OF_RANGE"),
    (dict(row_start=-1), "YOCO_ERR_OUT_OF_RANGE"),
    (dict(n=65), "YOCO_ERR_OUT_OF_RANGE"),
])
def test_kv_project_rejects(kw, status):
    c, lens = _cache()
    assert _project(c, **kw) == _status(status)
    assert lens.tolist() == [10, 20]
    assert len(_lib().yoco_last_error()) > 0


def test_kv_project_zero_rows_is_noop():
    c, lens = _cache()
    assert _project(c, n=0) == 0
    assert lens.tolist() == [10, 20]


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, "YOCO_ERR_BAD_SHAPE"),
    ("n_seq", 0, "YOCO_ERR_BAD_SHAPE"),
    ("n_seq", 257, "YOCO_ERR_BAD_SHAPE"),
    ("n_kv_heads", 0, "YOCO_ERR_BAD_SHAPE"),
    ("n_kv_heads", 65, "YOCO_ERR_BAD_SHAPE"),
    ("dtype", 3, "YOCO_ERR_BAD_DTYPE"),
    ("seq_capacity", 0, "YOCO_ERR_BAD_SHAPE"),
])
def test_bad_cache_descriptor(field, value, status):
    c, lens = _cache()
    setattr(c, field, value)
    assert _project(c) == _status(status)
    assert lens.tolist() == [10, 20]


def test_cache_pointers_required():
    c, _ = _cache()
    c.k = None
    assert _project(c) == _status("YOCO_ERR_NULL_POINTER")
    assert _lib().yoco_kv_project(FAKE, 1, 4, 32, None, 1e-6, FAKE, FAKE, 1, None, 0, 0, None, 0, None) == \
        _status("YOCO_ERR_NULL_POINTER")


def test_append_at_capacity_rejected_and_lengths_kept():
    c, lens = _cache(lens=(10, 64))
    st = _lib().yoco_kv_append(FAKE, 1, 32, None, 1e-6, FAKE, FAKE, 1, ctypes.byref(c), None, 0, None)
    assert st == _status("YOCO_ERR_OUT_OF_RANGE")
    assert lens.tolist() == [10, 64]


def _prefill(c, q_start=0, t=4, hq=4, q_dt=1, o_dt=0, scale=0.125, seq=0):
    return _lib().yoco_cross_attn_prefill(FAKE, q_dt, q_start, t, hq, ctypes.byref(c), seq, scale, FAKE,
                                          o_dt, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q_start=8, t=3), "YOCO_ERR_OUT_OF_RANGE"),     # 8 + 3 > len 10
    (dict(q_start=-1), "YOCO_ERR_OUT_OF_RANGE"),
    (dict(t=-1), "YOCO_ERR_OUT_OF_RANGE"),
    (dict(hq=3), "YOCO_ERR_BAD_SHAPE"),                  # 3 % 2 != 0
    (dict(hq=10), "YOCO_ERR_BAD_SHAPE"),                 # group 5 unsupported
    (dict(q_dt=0), "YOCO_ERR_BAD_DTYPE"),                # q f32, cache bf16
    (dict(o_dt=4), "YOCO_ERR_BAD_DTYPE"),
    (dict(scale=0.0), "YOCO_ERR_BAD_VALUE"),
    (dict(scale=float("inf")), "YOCO_ERR_BAD_VALUE"),
    (dict(seq=5), "YOCO_ERR_BAD_SHAPE"),
])
def test_prefill_rejects(kw, status):
    c, _ = _cache()
    assert _prefill(c, **kw) == _status(status)


def test_prefill_zero_rows_is_noop():
    c, _ = _cache()
    assert _prefill(c, q_start=10, t=0) == 0


def _ws_bytes(c, hq=4, rows=0):
    out = ctypes.c_size_t(0)
    st = _lib().yoco_cross_attn_decode_workspace(ctypes.byref(c), hq, rows, ctypes.byref(out))
    return st, out.value


def test_decode_workspace_sizes():
    c, _ = _cache(n_seq=1, cap=131072, hkv=8, dh=128, lens=(131072,))
    st, auto = _ws_bytes(c, hq=24)
    assert st == 0
    counters = 256 * 64 * 4
    # library split size: splits <= min(n_seq*ceil(cap/256), ceil(4096/H_kv) + n_seq)
    assert auto == counters + min(131072 // 256, 4096 // 8 + 1) * 8 * 3 * (128 + 4) * 4
    st, fixed = _ws_bytes(c, hq=24, rows=256)
    assert st == 0 and fixed == counters + 512 * 8 * 3 * 132 * 4
    assert _ws_bytes(c, hq=24, rows=100)[0] == _status("YOCO_ERR_BAD_VALUE")
    assert _ws_bytes(c, hq=20)[0] == _status("YOCO_ERR_BAD_SHAPE")


def _decode(c, ws_bytes=1 << 30, hq=4, rows=0, q_dt=1):
    return _lib().yoco_cross_attn_decode(FAKE, q_dt, hq, ctypes.byref(c), 0.125, FAKE, None, FAKE,
                                         ws_bytes, rows, None)


def test_decode_rejects():
    c, _ = _cache(lens=(10, 0))
    assert _decode(c) == _status("YOCO_ERR_OUT_OF_RANGE")       # empty sequence
    c, _ = _cache(lens=(10, 65))
    assert _decode(c) == _status("YOCO_ERR_OUT_OF_RANGE")       # past capacity
    c, _ = _cache()
    assert _decode(c, ws_bytes=16) == _status("YOCO_ERR_WORKSPACE")
    assert _decode(c, rows=300) == _status("YOCO_ERR_BAD_VALUE")
    assert _decode(c, q_dt=0) == _status("YOCO_ERR_BAD_DTYPE")
    assert _lib().yoco_cross_attn_decode(FAKE, 1, 4, ctypes.byref(c), 0.125, FAKE, None, None, 1 << 30, 0,
                                         None) == _status("YOCO_ERR_NULL_POINTER")


def test_q_project_rejects():
    L = _lib()
    assert L.yoco_q_project(FAKE, 1, 4, 32, None, 1e-6, FAKE, 1, 4, 96, FAKE, 1, None, 0, None) == _status("YOCO_ERR_BAD_SHAPE")
    assert L.yoco_q_project(None, 1, 4, 32, None, 1e-6, FAKE, 1, 4, 64, FAKE, 1, None, 0, None) == _status("YOCO_ERR_NULL_POINTER")
    assert L.yoco_q_project(FAKE, 1, 4, 32, None, 1e-6, FAKE, 1, 4, 64, FAKE, 2, None, 0, None) == _status("YOCO_ERR_BAD_DTYPE")
    assert L.yoco_q_project(FAKE, 1, 0, 32, None, 1e-6, FAKE, 1, 4, 64, FAKE, 1, None, 0, None) == 0


@pytest.mark.skipif(gpu_available(), reason="checks the no-GPU failure mode")
def test_valid_call_without_gpu_fails_loudly():
    c, lens = _cache()
    st = _project(c)
    assert st == _status("YOCO_ERR_HIP")
    assert lens.tolist() == [10, 20]
    assert b"hip" in _lib().yoco_last_error().lower()


def test_python_binding_refuses_host_tensors():
    import torch
    import yoco_shared_kv_amd as y
    with pytest.raises(ValueError):
        y.q_project(torch.zeros(2, 32), torch.zeros(32, 256), 4, 64)


def test_rope_entry_points_reject_bad_theta_and_positions():
    L = _lib()
    c, lens = _cache()
    for theta in (0.0, 1.0, 0.5, float("inf"), float("nan")):
        st = L.yoco_kv_project_rope(FAKE, 1, 4, 32, None, 1e-6, FAKE, FAKE, 1, ctypes.byref(c), 0, 0, theta, None, 0,
                                    None)
        assert st == _status("YOCO_ERR_BAD_VALUE"), theta
        st = L.yoco_kv_append_rope(FAKE, 1, 32, None, 1e-6, FAKE, FAKE, 1, ctypes.byref(c), theta, None, 0, None)
        assert st == _status("YOCO_ERR_BAD_VALUE"), theta
    assert lens.tolist() == [10, 20]
    pos = (ctypes.c_int64 * 3)(5, -1, 7)
    assert L.yoco_q_project_rope(FAKE, 1, 3, 32, None, 1e-6, FAKE, 1, 4, 64, FAKE, 1, pos, 0, 1e4, None, 0, None) == \
        _status("YOCO_ERR_OUT_OF_RANGE")
    assert L.yoco_q_project_rope(FAKE, 1, 3, 32, None, 1e-6, FAKE, 1, 4, 64, FAKE, 1, None, -2, 1e4, None, 0, None) == \
        _status("YOCO_ERR_OUT_OF_RANGE")
    big = (ctypes.c_int64 * 257)()
    assert L.yoco_q_project_rope(FAKE, 1, 257, 32, None, 1e-6, FAKE, 1, 4, 64, FAKE, 1, big, 0, 1e4, None, 0, None) == \
        _status("YOCO_ERR_BAD_SHAPE")
    assert L.yoco_q_project_rope(FAKE, 1, 0, 32, None, 1e-6, FAKE, 1, 4, 64, FAKE, 1, None, 0, 1e4, None, 0, None) == 0


def _bwd(c, **kw):
    args = dict(q=FAKE, o=FAKE, o_dt=0, d_o=FAKE, lse=FAKE, q_start=0, t=8, hq=4, seq=0, scale=0.125,
                d_q=FAKE, d_k=FAKE, d_v=FAKE, ws=FAKE, ws_bytes=1 << 20)
    args.update(kw)
    return _lib().yoco_cross_attn_prefill_bwd(args["q"], args["o"], args["o_dt"], args["d_o"], args["lse"],
                                              args["q_start"], args["t"], args["hq"], ctypes.byref(c), args["seq"],
                                              args["scale"], args["d_q"], args["d_k"], args["d_v"], args["ws"],
                                              args["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d_o=None), "YOCO_ERR_NULL_POINTER"),
    (dict(lse=None), "YOCO_ERR_NULL_POINTER"),
    (dict(d_k=None), "YOCO_ERR_NULL_POINTER"),
    (dict(ws=None), "YOCO_ERR_NULL_POINTER"),
    (dict(hq=3), "YOCO_ERR_BAD_SHAPE"),
    (dict(seq=2), "YOCO_ERR_BAD_SHAPE"),
    (dict(o_dt=7), "YOCO_ERR_BAD_DTYPE"),
    (dict(scale=0.0), "YOCO_ERR_BAD_VALUE"),
    (dict(q_start=5, t=8), "YOCO_ERR_OUT_OF_RANGE"),
    (dict(t=-1), "YOCO_ERR_OUT_OF_RANGE"),
    (dict(ws_bytes=2 * 8 * 4 * 4 - 1), "YOCO_ERR_WORKSPACE"),
])
def test_prefill_bwd_rejects(kw, status):
    c, lens = _cache()
    assert _bwd(c, **kw) == _status(status)
    assert len(_lib().yoco_last_error()) > 0


def test_prefill_bwd_needs_bf16_cache_and_sizes_workspace():
    c, _ = _cache(dtype=0)
    assert _bwd(c) == _status("YOCO_ERR_BAD_DTYPE")
    c, _ = _cache()
    assert _bwd(c, t=0, ws_bytes=0) == 0
    out = ctypes.c_size_t(0)
    assert _lib().yoco_cross_attn_prefill_bwd_workspace(1000, 24, ctypes.byref(out)) == 0
    assert out.value == 2 * 1000 * 24 * 4


def _pbwd(**kw):
    args = dict(m=FAKE, m_dt=1, n=300, d=512, gain=None, eps=1e-6, wk=FAKE, wv=FAKE, w_dt=1, hkv=2, dh=128,
                dzk=FAKE, dzv=FAKE, dz_dt=0, dm=FAKE, dwk=FAKE, dwv=FAKE, dg=None, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    a = args
    return _lib().yoco_kv_project_bwd(a["m"], a["m_dt"], a["n"], a["d"], a["gain"], a["eps"], a["wk"], a["wv"],
                                      a["w_dt"], a["hkv"], a["dh"], a["dzk"], a["dzv"], a["dz_dt"], a["dm"],
                                      a["dwk"], a["dwv"], a["dg"], a["ws"], a["ws_bytes"], None)


def _pbwd_ws(n, d, ncols, n_out):
    out = ctypes.c_size_t(0)
    st = _lib().yoco_project_bwd_workspace(n, d, ncols, n_out, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw,status", [
    (dict(m=None), "YOCO_ERR_NULL_POINTER"),
    (dict(dzv=None), "YOCO_ERR_NULL_POINTER"),
    (dict(dwk=None), "YOCO_ERR_NULL_POINTER"),
    (dict(ws=None), "YOCO_ERR_NULL_POINTER"),
    (dict(dm=None), "YOCO_ERR_NULL_POINTER"),
    (dict(d=0), "YOCO_ERR_BAD_SHAPE"),
    (dict(d=4097), "YOCO_ERR_BAD_SHAPE"),
    (dict(n=-1), "YOCO_ERR_BAD_SHAPE"),
    (dict(hkv=0), "YOCO_ERR_BAD_SHAPE"),
    (dict(dh=96), "YOCO_ERR_BAD_SHAPE"),
    (dict(dz_dt=3), "YOCO_ERR_BAD_DTYPE"),
    (dict(w_dt=2), "YOCO_ERR_BAD_DTYPE"),
    (dict(eps=-1.0), "YOCO_ERR_BAD_VALUE"),
    (dict(ws_bytes=1024), "YOCO_ERR_WORKSPACE"),
])
def test_project_bwd_rejects(kw, status):
    assert _pbwd(**kw) == _status(status)
    assert len(_lib().yoco_last_error()) > 0


def test_project_bwd_workspace_layout():
    # matrix-core shapes: 1/r, y and dz in bf16, split partials, dgain shares
    st, b = _pbwd_ws(32768, 3072, 1024, 2)
    assert st == 0
    splits = 8  # ceil(768 / (12 * 4 * 2)) tiles, 4096 rows each
    expect = 32768 * 4 + 32768 * 3072 * 2 + 2 * 32768 * 1024 * 2 + splits * 2 * 3072 * 1024 * 4 + 512 * 3072 * 4
    assert b == expect
    # shapes the tiles do not cover: 1/r and dgain shares only (256-byte aligned)
    st, b = _pbwd_ws(257, 256, 128, 2)
    assert st == 0 and b == 1280 + 5 * 256 * 4
    assert _pbwd_ws(10, 64, 128, 3)[0] == _status("YOCO_ERR_BAD_SHAPE")
    st, b = _pbwd_ws(0, 512, 256, 2)
    assert st == 0 and b == 0 and _pbwd(n=0, ws_bytes=0) == 0
    L = _lib()
    assert L.yoco_q_project_bwd(FAKE, 1, 4, 32, None, 1e-6, FAKE, 1, 4, 96, FAKE, 0, FAKE, FAKE, None, FAKE,
                                1 << 20, None) == _status("YOCO_ERR_BAD_SHAPE")
    assert L.yoco_q_project_bwd(FAKE, 1, 4, 32, None, 1e-6, None, 1, 4, 64, FAKE, 0, FAKE, FAKE, None, FAKE,
                                1 << 20, None) == _status("YOCO_ERR_NULL_POINTER")


def test_gret_rejects_and_sizes_workspace():
    L = _lib()
    def pre(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, dt=1, g=FAKE, tau=16.0, n=300, h=3, dh=128, s_in=None, o=FAKE, s_out=None,
                 ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return L.yoco_gret_prefill(a["q"], a["k"], a["v"], a["dt"], a["g"], a["tau"], a["n"], a["h"], a["dh"],
                                   a["s_in"], a["o"], a["s_out"], a["ws"], a["ws_bytes"], None)
    assert pre(q=None) == _status("YOCO_ERR_NULL_POINTER")
    assert pre(g=None) == _status("YOCO_ERR_NULL_POINTER")
    assert pre(dh=96) == _status("YOCO_ERR_BAD_SHAPE")
    assert pre(h=0) == _status("YOCO_ERR_BAD_SHAPE")
    assert pre(n=-1) == _status("YOCO_ERR_BAD_SHAPE")
    assert pre(dt=4) == _status("YOCO_ERR_BAD_DTYPE")
    for tau in (0.0, -1.0, float("inf"), float("nan")):
        assert pre(tau=tau) == _status("YOCO_ERR_BAD_VALUE")
    assert pre(ws_bytes=100) == _status("YOCO_ERR_WORKSPACE")
    assert pre(n=0) == 0
    out = ctypes.c_size_t(0)
    # chunkwise path, 256-byte aligned regions: cumulative gates, per-group log decays, group totals
    # and group start states (fp32); 3 chunks, 1 group
    assert L.yoco_gret_prefill_workspace(300, 3, 128, 1, ctypes.byref(out)) == 0
    up = lambda b: (b + 255) // 256 * 256
    assert out.value == up(300 * 3 * 4) + up(1 * 3 * 4) + 2 * 1 * 3 * 128 * 128 * 4
    assert L.yoco_gret_prefill_workspace(2049, 1, 128, 1, ctypes.byref(out)) == 0  # 17 chunks, 3 groups
    assert out.value == up(2049 * 4) + up(3 * 4) + 2 * 3 * 1 * 128 * 128 * 4
    assert L.yoco_gret_prefill_workspace(300, 3, 128, 0, ctypes.byref(out)) == 0 and out.value == 0
    assert L.yoco_gret_prefill_workspace(300, 3, 64, 1, ctypes.byref(out)) == 0 and out.value == 0
    assert pre(dt=0, ws=None, ws_bytes=0) != _status("YOCO_ERR_WORKSPACE")
    dec = lambda **kw: L.yoco_gret_decode(kw.get("q", FAKE), FAKE, FAKE, 1, FAKE, kw.get("tau", 16.0),
                                         kw.get("b", 2), 3, kw.get("dh", 128), kw.get("st", FAKE), FAKE, None)
    assert dec(st=None) == _status("YOCO_ERR_NULL_POINTER")
    assert dec(dh=32) == _status("YOCO_ERR_BAD_SHAPE")
    assert dec(b=-1) == _status("YOCO_ERR_BAD_SHAPE")
    assert dec(tau=0.0) == _status("YOCO_ERR_BAD_VALUE")
    assert dec(b=0) == 0


def test_status_table_matches_header():
    from yoco_shared_kv_amd._native import STATUS
    text = open(HEADER).read()
    codes = {int(v): k for k, v in re.findall(r"\b(YOCO_(?:OK|ERR_[A-Z_]+)) = (\d+)", text)}
    assert codes == STATUS


MIS = ctypes.c_void_p(0x1008)   # 8-byte but not 16-byte aligned
MIS4 = ctypes.c_void_p(0x1002)  # not 4-byte aligned
AL4 = ctypes.c_void_p(0x1004)   # 4-byte aligned


def test_misaligned_pointers_rejected():
    L = _lib()
    bad = _status("YOCO_ERR_ALIGNMENT")
    c, lens = _cache()
    assert _project(c, m=MIS) == bad
    assert _project(c, gain=MIS) == bad
    assert lens.tolist() == [10, 20]
    assert "aligned" in L.yoco_last_error().decode()
    c.k = MIS
    assert _project(c) == bad
    c, lens = _cache()
    assert L.yoco_kv_append(FAKE, 1, 32, None, 1e-6, FAKE, MIS, 1, ctypes.byref(c), None, 0, None) == bad
    assert lens.tolist() == [10, 20]
    assert L.yoco_q_project(FAKE, 1, 4, 32, None, 1e-6, FAKE, 1, 4, 64, MIS, 1, None, 0, None) == bad
    assert L.yoco_cross_attn_prefill(MIS, 1, 0, 4, 4, ctypes.byref(c), 0, 0.125, FAKE, 0, None, None) == bad
    assert L.yoco_cross_attn_prefill(FAKE, 1, 0, 4, 4, ctypes.byref(c), 0, 0.125, FAKE, 0, MIS4, None) == bad
    assert L.yoco_cross_attn_decode(FAKE, 1, 4, ctypes.byref(c), 0.125, MIS, None, FAKE, 1 << 30, 0, None) == bad
    assert L.yoco_cross_attn_decode(FAKE, 1, 4, ctypes.byref(c), 0.125, FAKE, None, MIS, 1 << 30, 0, None) == bad
    assert _bwd(c, d_v=MIS) == bad
    assert _bwd(c, lse=MIS4) == bad
    assert _pbwd(dzv=MIS) == bad
    assert _pbwd(dm=MIS) == bad
    # 4-byte scalar arrays pass the alignment check (and fail later only for other reasons)
    assert _bwd(c, lse=AL4, ws_bytes=16) == _status("YOCO_ERR_WORKSPACE")
    gret = lambda **kw: L.yoco_gret_prefill(kw.get("q", FAKE), FAKE, FAKE, 1, kw.get("g", FAKE), 16.0, 300, 3, 128,
                                           kw.get("s_in"), FAKE, None, FAKE, kw.get("ws_bytes", 1 << 30), None)
    assert gret(q=MIS) == bad
    assert gret(s_in=MIS) == bad
    assert gret(g=MIS4) == bad
    assert gret(g=AL4, ws_bytes=100) == _status("YOCO_ERR_WORKSPACE")
    assert L.yoco_gret_decode(FAKE, FAKE, FAKE, 1, FAKE, 16.0, 2, 3, 128, MIS, FAKE, None) == bad


def test_kvcache_wrap_reads_the_row_stride():
    """KVCache.wrap takes dense or row-padded [n_seq, capacity, H_kv, d_h]
    tensors and rejects layouts whose heads are not packed inside a row
    (host tensors: only the layout logic runs)."""
    import torch
    import yoco_shared_kv_amd as y
    dense = torch.zeros(2, 5, 8, 128, dtype=torch.bfloat16)
    assert y.KVCache.wrap(dense, dense.clone(), [1, 2]).row_stride == 1024
    rows = torch.zeros(2, 5, 1088, dtype=torch.bfloat16)
    padded = rows[:, :, :1024].unflatten(2, (8, 128))
    assert y.KVCache.wrap(padded, rows.clone()[:, :, :1024].unflatten(2, (8, 128)), [1, 2]).row_stride == 1088
    one = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16)
    assert y.KVCache.wrap(one, one.clone(), [0]).row_stride == 1024
    swapped = torch.zeros(2, 5, 128, 8, dtype=torch.bfloat16).transpose(2, 3)
    with pytest.raises(ValueError):
        y.KVCache.wrap(swapped, swapped, [1, 1])
    with pytest.raises(ValueError):
        y.KVCache.wrap(dense, padded, [1, 1])                     # k and v strides differ


def test_project_workspace_sizes_and_rules():
    L = _lib()
    out = ctypes.c_size_t(0)
    # one appended row at 3B widths: K^ and V^ of 8 heads x 128, bf16 weights
    assert L.yoco_project_workspace(1, 3072, 1024, 2, 1, ctypes.byref(out)) == 0
    kv = out.value
    assert kv > 16384 and (kv - 16384) % 16 == 0
    # the partials are sized for a launch of 8 rows whatever n is (1..32)
    for n in (2, 8, 32):
        assert L.yoco_project_workspace(n, 3072, 1024, 2, 1, ctypes.byref(out)) == 0 and out.value == kv
    # shapes that do not take the few-row path need none
    for args in ((33, 3072, 1024, 2, 1), (0, 3072, 1024, 2, 1), (1, 256, 96, 1, 1), (1, 256, 32, 1, 0)):
        assert L.yoco_project_workspace(*args, ctypes.byref(out)) == 0 and out.value == 0, args
    assert L.yoco_project_workspace(1, 256, 64, 1, 0, ctypes.byref(out)) == 0 and out.value > 16384
    # at most 128 column blocks (one arrival counter per 128-byte line of the 16 KiB)
    assert L.yoco_project_workspace(1, 256, 128 * 64, 2, 1, ctypes.byref(out)) == 0 and out.value > 0
    assert L.yoco_project_workspace(1, 256, 130 * 64, 2, 1, ctypes.byref(out)) == 0 and out.value == 0
    assert L.yoco_project_workspace(1, 0, 1024, 2, 1, ctypes.byref(out)) == _status("YOCO_ERR_BAD_SHAPE")
    assert L.yoco_project_workspace(1, 64, 1024, 3, 1, ctypes.byref(out)) == _status("YOCO_ERR_BAD_SHAPE")
    assert L.yoco_project_workspace(1, 64, 1024, 2, 7, ctypes.byref(out)) == _status("YOCO_ERR_BAD_DTYPE")
    assert L.yoco_project_workspace(1, 64, 1024, 2, 1, None) == _status("YOCO_ERR_NULL_POINTER")

    # A workspace that is given but too small for a call that uses it is an
    # error before anything is enqueued; a misaligned one too.
    c, lens = _cache()   # 2 sequences, 2 KV heads x 64
    need = ctypes.c_size_t(0)
    ncols = c.n_kv_heads * c.head_dim
    assert L.yoco_project_workspace(4, 32, ncols, 2, 1, ctypes.byref(need)) == 0
    if need.value:
        assert _project(c, ws=FAKE, ws_bytes=need.value - 1) == _status("YOCO_ERR_WORKSPACE")
        assert _project(c, ws=MIS, ws_bytes=need.value) == _status("YOCO_ERR_ALIGNMENT")
        st = L.yoco_kv_append(FAKE, 1, 32, None, 1e-6, FAKE, FAKE, 1, ctypes.byref(c), FAKE, 16, None)
        assert st == _status("YOCO_ERR_WORKSPACE")
    assert lens.tolist() == [10, 20]
    assert L.yoco_q_project(FAKE, 1, 4, 32, None, 1e-6, FAKE, 1, 4, 64, FAKE, 1, FAKE, 16, None) == \
        _status("YOCO_ERR_WORKSPACE")


def test_fold_norm_gain_rejects():
    L = _lib()
    OUT = ctypes.c_void_p(0x100000)
    fold = lambda w=FAKE, dt=1, g=FAKE, d=4, n=8, out=OUT: L.yoco_fold_norm_gain(w, dt, g, d, n, out, None)
    assert fold(w=None) == _status("YOCO_ERR_NULL_POINTER")
    assert fold(g=None) == _status("YOCO_ERR_NULL_POINTER")
    assert fold(out=None) == _status("YOCO_ERR_NULL_POINTER")
    assert fold(d=0) == _status("YOCO_ERR_BAD_SHAPE")
    assert fold(n=-8) == _status("YOCO_ERR_BAD_SHAPE")
    assert fold(dt=2) == _status("YOCO_ERR_BAD_DTYPE")
    assert fold(w=MIS) == _status("YOCO_ERR_ALIGNMENT")
    assert fold(out=MIS) == _status("YOCO_ERR_ALIGNMENT")
    # bf16 4 x 8 spans 64 bytes: an output 16 bytes further on overlaps it
    assert fold(out=ctypes.c_void_p(0x1010)) == _status("YOCO_ERR_BAD_VALUE")
    assert "overlaps" in L.yoco_last_error().decode()
    # fp32 weights to bf16 in the same array would overwrite unread weights
    assert fold(dt=0, out=FAKE) == _status("YOCO_ERR_BAD_VALUE")
    assert fold(dt=0, out=ctypes.c_void_p(0x1000 + 4 * 4 * 8)) != _status("YOCO_ERR_BAD_VALUE")  # just past it
    if not gpu_available():
        assert fold(out=FAKE) == _status("YOCO_ERR_HIP")   # in place, bf16: valid, so it reaches the device check


def test_fold_binding_checks_shapes():
    import torch
    import yoco_shared_kv_amd as y
    with pytest.raises(ValueError, match="gain must"):
        y.fold_norm_gain(torch.zeros(32, 64, dtype=torch.bfloat16), torch.ones(16))
    with pytest.raises(TypeError, match="gain must"):
        y.fold_norm_gain(torch.zeros(32, 64, dtype=torch.bfloat16), torch.ones(32, dtype=torch.float64))
    with pytest.raises(TypeError, match="out must"):
        y.fold_norm_gain(torch.zeros(32, 64), torch.ones(32), out=torch.zeros(32, 64))
    with pytest.raises(ValueError, match="gain is required"):
        y.fold_norm_gain(torch.zeros(32, 64), None)
    with pytest.raises(ValueError, match="device"):
        y.fold_norm_gain(torch.zeros(32, 64), torch.ones(32))


def test_default_softmax_scale():
    L = _lib()
    out = ctypes.c_float(0.0)
    for dh in (64, 128):
        assert L.yoco_default_softmax_scale(dh, ctypes.byref(out)) == 0
        assert out.value == np.float32(1.0 / np.sqrt(dh))
    assert L.yoco_default_softmax_scale(0, ctypes.byref(out)) == _status("YOCO_ERR_BAD_SHAPE")
    assert L.yoco_default_softmax_scale(128, None) == _status("YOCO_ERR_NULL_POINTER")


def test_binding_checks_shapes_before_the_library():
    """The C ABI sees raw pointers only, so the binding checks every tensor
    against the cache and the weights (host tensors: nothing reaches the
    device)."""
    import torch
    import yoco_shared_kv_amd as y
    k = torch.zeros(2, 16, 8, 64, dtype=torch.bfloat16)
    cache = y.KVCache.wrap(k, k.clone(), [4, 4])
    with pytest.raises(ValueError, match="q must be"):
        y.cross_attn_decode(torch.zeros(3, 8, 64, dtype=torch.bfloat16), cache)
    with pytest.raises(ValueError, match="q must be"):
        y.cross_attn_decode(torch.zeros(2, 8, 128, dtype=torch.bfloat16), cache)
    with pytest.raises(ValueError, match="out must"):
        y.cross_attn_decode(torch.zeros(2, 8, 64, dtype=torch.bfloat16), cache, out=torch.zeros(2, 8, 32))
    with pytest.raises(TypeError, match="out must"):
        y.cross_attn_decode(torch.zeros(2, 8, 64, dtype=torch.bfloat16), cache,
                            out=torch.zeros(2, 8, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="m_new must be"):
        y.kv_append(cache, torch.zeros(1, 32), torch.zeros(32, 512), torch.zeros(32, 512))
    with pytest.raises(ValueError, match="weight must"):
        y.kv_append(cache, torch.zeros(2, 32), torch.zeros(32, 256), torch.zeros(32, 512))
    with pytest.raises(ValueError, match="weight must"):
        y.kv_project(cache, torch.zeros(5, 32), torch.zeros(32, 512), torch.zeros(16, 512))
    with pytest.raises(ValueError, match="gain must"):
        y.kv_project(cache, torch.zeros(5, 32), torch.zeros(32, 512), torch.zeros(32, 512), torch.ones(16))
    with pytest.raises(ValueError, match="weight must"):
        y.q_project(torch.zeros(2, 32), torch.zeros(32, 200), 4, 64)
    with pytest.raises(ValueError, match="q must be"):
        y.cross_attn_prefill(torch.zeros(4, 8, 128, dtype=torch.bfloat16), cache)


def test_cache_descriptor_follows_a_replaced_length_array(monkeypatch):
    """The descriptor keeps the length array it points into and is rebuilt
    when ``len`` is a different array, even one at a reused address."""
    import torch
    import yoco_shared_kv_amd as y
    monkeypatch.setattr(y, "_on_device", lambda *ts: None)
    k = torch.zeros(2, 16, 8, 64, dtype=torch.bfloat16)
    cache = y.KVCache.wrap(k, k.clone(), [4, 4])
    addr = lambda s: ctypes.cast(s.len_host, ctypes.c_void_p).value
    s1 = cache.struct()
    assert addr(s1) == cache.len.ctypes.data
    for _ in range(3):
        cache.len = np.array([5, 6], dtype=np.int64)
        s2 = cache.struct()
        assert addr(s2) == cache.len.ctypes.data
        assert cache.struct() is s2


def test_noalloc_decode_rejects_plans_beyond_its_scratch():
    """The decode that allocates nothing refuses, before anything is enqueued,
    a split plan whose partials exceed its fixed scratch, with a reason."""
    L = _lib()
    c, lens = _cache(n_seq=1, cap=131072, hkv=8, dh=128, lens=(131072,))
    # 512 splits x 8 KV heads x 8 query heads of 132 floats: 16.6 MiB > 8 MiB
    st = L.yoco_cross_attn_decode_noalloc(FAKE, 1, 64, ctypes.byref(c), 0.125, FAKE, None, 256, None)
    assert st == _status("YOCO_ERR_WORKSPACE")
    assert b"scratch" in L.yoco_last_error()
    assert lens.tolist() == [131072]
    # the same cache at a larger split size fits (then fails only for want of a GPU here)
    st = L.yoco_cross_attn_decode_noalloc(FAKE, 1, 64, ctypes.byref(c), 0.125, FAKE, None, 4096, None)
    assert st != _status("YOCO_ERR_WORKSPACE")
    assert L.yoco_cross_attn_decode_noalloc(None, 1, 64, ctypes.byref(c), 0.125, FAKE, None, 256, None) == \
        _status("YOCO_ERR_NULL_POINTER")
    assert L.yoco_cross_attn_decode_noalloc(FAKE, 1, 64, ctypes.byref(c), 0.125, MIS, None, 256, None) == \
        _status("YOCO_ERR_ALIGNMENT")
