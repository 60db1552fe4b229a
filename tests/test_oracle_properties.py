"""Property tests of the oracle on random tiny shapes (hypothesis): for any
group size G in {1, 2, 3}, head width d_h in {8, 16, 64}, cache length,
query positions (repeated and out of order), scale and storage type, the
oracle's causal GQA attention equals torch's fp64 scaled-dot-product
attention with an explicit position mask over repeat-interleaved K/V
([Notes] section 2.1 Eq. 3; [Blog] section 2), its gradients equal fp64
autograd, decode equals the last prefill row, and the shared-KV result for
several layers equals per-layer copies of the same K/V ([Deep] section 2.2).
The references are library routines, not the oracle's formulas retyped."""
import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402

from tests.oracle_pins import _torch_attn_grads, _torch_reference  # noqa: E402
from workloads import store  # noqa: E402

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])


@st.composite
def attention_case(draw):
    g = draw(st.sampled_from([1, 2, 3]))
    hkv = draw(st.integers(1, 3))
    dh = draw(st.sampled_from([8, 16, 64]))
    rows = draw(st.integers(1, 40))
    n_q = draw(st.integers(1, 12))
    pos = draw(st.lists(st.integers(0, rows - 1), min_size=n_q, max_size=n_q))
    dtype = draw(st.sampled_from(["f32", "bf16"]))
    scale = draw(st.sampled_from([1.0 / np.sqrt(dh), 0.05, 1.5]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    r = np.random.default_rng(seed)
    q = store((r.standard_normal((n_q, g * hkv, dh)) * 1.5).astype(np.float32), dtype)
    k = store((r.standard_normal((rows, hkv, dh)) * 1.5).astype(np.float32), dtype)
    v = store(r.standard_normal((rows, hkv, dh)).astype(np.float32), dtype)
    dout = store(r.standard_normal((n_q, g * hkv, dh)).astype(np.float32), dtype)
    return q, np.array(pos, dtype=np.int64), k, v, dout, float(scale)


@SETTINGS
@given(attention_case())
def test_attention_equals_torch_sdpa(orc, case):
    q, pos, k, v, _, scale = case
    o, lse = orc.attention(q, pos, k, v, scale, want_lse=True)
    ro, rl = _torch_reference(q, pos, k, v, scale)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


@SETTINGS
@given(attention_case())
def test_attention_gradients_equal_autograd(orc, case):
    q, pos, k, v, dout, scale = case
    dq, dk, dv = orc.attention_bwd(q, pos, k, v, dout, scale)
    rq, rk, rv = _torch_attn_grads(q, pos, k, v, dout, scale)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11, err_msg=name)


@SETTINGS
@given(attention_case())
def test_decode_is_the_last_prefill_row_and_layers_share_one_cache(orc, case):
    q, pos, k, v, _, scale = case
    rows = k.shape[0]
    full = orc.prefill(np.repeat(q[:1], rows, axis=0), 0, k, v, scale)
    dec = orc.decode(q[:1], rows, k, v, scale)
    np.testing.assert_array_equal(dec[0], full[-1])
    # three "layers" (queries) over one shared slab == each over its own copy
    layers = [q[i % q.shape[0]:i % q.shape[0] + 1] for i in range(3)]
    shared = [orc.decode(ql, rows, k, v, scale) for ql in layers]
    own = [orc.decode(ql, rows, k.copy(), v.copy(), scale) for ql in layers]
    for a, b in zip(shared, own):
        np.testing.assert_array_equal(a, b)
