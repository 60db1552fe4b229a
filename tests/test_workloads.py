"""The seeded input generators: storage rounding, draw order, planted
structure, and the cache sizes the pages print."""
import math
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_sizes.txt")
UNITS = {"GiB": 2 ** 30, "MiB": 2 ** 20}


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            name, value, unit = line.split()
            out[name] = float(value) * UNITS[unit]
    return out


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100_000).astype(np.float32) * 10
    # exact ties: low 16 bits 0x8000 with even and odd kept parts
    ties = (np.arange(0x3F80, 0x3F80 + 64, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_ragged_lengths_first_draw():
    lens = W.ragged_lengths()
    assert lens.tolist() == [112717, 86462, 71000, 41343, 46018, 13226, 17437, 10222,
                             29729, 108127, 87992, 120352, 70078, 82736, 127477, 97833]
    assert int(lens.sum()) == 1_122_749
    case = W.make_ragged_decode(n_seq=3, lo=5, hi=40, n_q_heads=4, n_kv_heads=2,
                                head_dim=8, layers=2)
    assert case.lens.tolist() == W.ragged_lengths(3, 5, 40).tolist()
    assert [k.shape[0] for k in case.k] == case.lens.tolist()
    assert case.q.shape == (2, 3, 4, 8)


def test_tiny_case_shapes_and_scales():
    c = W.make_tiny()
    assert c.m.shape == (257, 256) and c.x.shape == (257, 256)
    assert c.w_k.shape == (256, 128) and c.w_v.shape == (256, 128) and c.w_q.shape == (256, 256)
    assert abs(c.w_q.std() - 1 / 16) < 2e-3   # N(0, 1/d_model)
    assert abs(c.m.std() - 1) < 1e-2
    again = W.make_tiny()
    assert np.array_equal(again.w_v, c.w_v)


def test_prefill_peaked_rows():
    c = W.make_prefill(n=1000, n_q_heads=4, n_kv_heads=2, head_dim=16)
    assert len(c.peaked_rows) == 10 and len(set(c.peaked_rows.tolist())) == 10
    k = W.as_f32(c.k)
    peak_norm = np.linalg.norm(k[c.peaked_rows], axis=-1).mean()
    rest = np.setdiff1d(np.arange(1000), c.peaked_rows)
    assert 6 < peak_norm / np.linalg.norm(k[rest], axis=-1).mean() < 10
    # 32 Ki tokens: floor(1% of 32768) = 327 rows
    assert math.floor(W.PEAK_FRACTION * 32768) == 327


def test_needle_plants_twelve_sigma_key():
    c = W.make_needle_decode(n_rows=4096, layers=13)
    q = W.as_f32(c.q).astype(np.float64)
    k = W.as_f32(c.k[0]).astype(np.float64)
    for g in range(8):
        p = c.needle_pos[0, g]
        qs = q[:, 0, 3 * g:3 * g + 3, :].reshape(-1, 128)        # 39 queries
        ratio = (qs @ k[p, g]) / np.linalg.norm(qs, axis=1)
        assert np.all(np.abs(ratio - 12.0) < 0.2), ratio           # bf16 storage rounding


def test_cache_sizes_printed_on_pages():
    g = _golden()
    n, hkv, dh, b = W.DECODE_128K["n_rows"], W.DECODE_128K["n_kv_heads"], W.DECODE_128K["head_dim"], 2
    per_layer = 2 * n * hkv * dh * b
    assert per_layer == g["yoco_shared_kv"] == 536_870_912
    assert 26 * per_layer == g["transformer_26_layer_kv"]
    assert 13 * 24 * 128 * 128 * b == g["gret_state_13_layers"]


@pytest.mark.slow
def test_decode_workload_is_half_gib():
    c = W.make_decode(n_rows=131072, layers=1)
    assert c.k[0].nbytes + c.v[0].nbytes == _golden()["yoco_shared_kv"]
