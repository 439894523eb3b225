"""Seeded generators: deterministic, right shapes and distributions (CPU only)."""
import numpy as np

from inputs import synth


def test_deterministic():
    a = synth.layer_prefill(T=64)
    b = synth.layer_prefill(T=64)
    for f in ("q", "k", "v", "g", "beta", "A_log", "dt_bias"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = synth.long_context_call(1, T=64)
    d = synth.long_context_call(2, T=64)
    assert np.array_equal(c.A_log, d.A_log) and not np.array_equal(c.q, d.q)


def test_shapes_and_ranges():
    x = synth.tiny_config()
    assert x.q.shape == (1, 128, 2, 32) and x.v.shape == (1, 128, 6, 32) and x.g.shape == (1, 128, 6)
    assert x.dtype == "f32" and x.chunk_size == 32
    np.testing.assert_allclose(np.linalg.norm(x.q, axis=-1), 1.0, rtol=1e-6)
    y = synth.layer_prefill(T=256)
    assert y.q.shape == (1, 256, 16, 128) and y.v.shape == (1, 256, 48, 128)
    assert not np.any(y.q.view(np.uint32) & 0xFFFF)  # bf16-representable
    np.testing.assert_allclose(np.linalg.norm(y.k, axis=-1), 1.0, rtol=2e-2)
    assert np.all(y.g < 0) and np.all((y.beta > 0) & (y.beta < 1))
    assert np.all((y.A_log >= 0) & (y.A_log <= np.log(16))) and np.all(np.abs(y.dt_bias) <= 1)


def test_decode_inputs():
    A_log, dt, s0 = synth.decode_inputs(N=2, hv=6, hk=2, d=8)
    assert s0.shape == (2, 6, 8, 8) and s0.dtype == np.float32
    assert 0.03 < s0.std() < 0.07
    st = synth.decode_step_inputs(5, N=2, hv=6, hk=2, d=8)
    assert st.q.shape == (2, 2, 8) and st.v.shape == (2, 6, 8) and st.g.shape == (2, 6)
    assert np.array_equal(st.A_log, A_log)


def test_varlen_lengths():
    lens = synth.varlen_lengths()
    assert len(lens) == 8 and lens.sum() == 65536
    assert lens.min() >= 1024 and lens.max() <= 32768
    cu = synth.cu_seqlens_of(lens)
    assert cu.dtype == np.int32 and cu[0] == 0 and cu[-1] == 65536


def test_pipeline_small():
    p = synth.pipeline_inputs(lengths=[3, 5], hk=2, hv=6, d=16)
    assert p.x.shape == (8, 2 * 2 * 16 + 6 * 16) and p.conv_w.shape == (p.x.shape[1], 4)
    assert p.z.shape == (8, 96) and p.a.shape == (8, 6) and p.norm_w.shape == (16,)
    assert not np.any(p.conv_w.view(np.uint32) & 0xFFFF)
