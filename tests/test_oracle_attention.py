"""Pins of the global-attention oracle (CPU only): rotary encoding and RMS
norm against their defining properties, the attention core against closed
forms, and the decode step against the prefill."""
import numpy as np

from oracle import attention as A


def _rng(s):
    return np.random.default_rng(s)


def test_rope_identity_at_zero_and_passthrough():
    x = _rng(0).standard_normal((3, 2, 256))
    assert np.array_equal(A.rope(x, np.zeros(3)), x)
    y = A.rope(x, np.array([5, 1000, 262143]))
    assert np.array_equal(y[..., 64:], x[..., 64:])
    assert not np.allclose(y[..., :64], x[..., :64])


def test_rope_is_a_rotation_by_the_stated_angles():
    """Each pair (j, j + 32) is rotated by pos * 1e7^(-j/32): norms kept,
    inverse rotation restores, and pair 0 turns by exactly pos radians."""
    rng = _rng(1)
    x = rng.standard_normal((4, 256))
    pos = np.array([0, 1, 17, 40000])
    y = A.rope(x, pos)
    for j in (0, 5, 31):
        assert np.allclose(np.hypot(y[:, j], y[:, j + 32]), np.hypot(x[:, j], x[:, j + 32]), rtol=1e-13)
    ang0 = np.arctan2(y[:, 32], y[:, 0]) - np.arctan2(x[:, 32], x[:, 0])
    assert np.allclose(np.angle(np.exp(1j * (ang0 - pos))), 0, atol=1e-9)
    ang31 = np.arctan2(y[:, 63], y[:, 31]) - np.arctan2(x[:, 63], x[:, 31])
    want = pos * 1e7 ** (-31 / 32)
    assert np.allclose(np.angle(np.exp(1j * (ang31 - want))), 0, atol=1e-9)
    # inverse: rotating each row back by the same angles
    ang = A.rope_angles(pos)
    back = y.copy()
    c, s = np.cos(ang), np.sin(ang)
    back[:, :32] = y[:, :32] * c + y[:, 32:64] * s
    back[:, 32:64] = y[:, 32:64] * c - y[:, :32] * s
    assert np.allclose(back, x, atol=1e-12)


def test_rope_scores_depend_only_on_relative_position():
    """<R(p) q, R(p') k> is unchanged when both positions shift."""
    rng = _rng(2)
    q, k = rng.standard_normal((1, 256)), rng.standard_normal((1, 256))
    for p, pp, sft in ((3, 1, 100), (1000, 20, 7777), (5, 5, 31)):
        a = A.rope(q, [p])[0] @ A.rope(k, [pp])[0]
        b = A.rope(q, [p + sft])[0] @ A.rope(k, [pp + sft])[0]
        assert abs(a - b) < 1e-9 * (1 + abs(a))


def test_rms_norm_unit_rms_and_scale_invariance():
    rng = _rng(3)
    x = rng.standard_normal((5, 256)) * rng.uniform(0.1, 10, (5, 1))
    y = A.rms_norm(x, np.ones(256), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    assert np.allclose(A.rms_norm(7.5 * x, np.ones(256), eps=0.0), y, rtol=1e-13)
    w = rng.standard_normal(256)
    assert np.allclose(A.rms_norm(x, w, eps=0.0), y * w, rtol=1e-13)


def test_core_two_key_softmax_closed_form():
    """Scores 0 and ln 3 weight the two values 1/4 and 3/4."""
    D = 256
    q_rot = np.zeros((2, 1, D))
    k_rot = np.zeros((2, 1, D))
    q_rot[1, 0, 100] = 16.0 * np.log(3.0)
    k_rot[1, 0, 100] = 1.0
    v = _rng(4).standard_normal((2, 1, D))
    gate = _rng(5).standard_normal((2, 1, D))
    r = A.core_prefill(q_rot, k_rot, v, gate, np.array([0, 2]))
    sg = 1 / (1 + np.exp(-gate))
    assert np.allclose(r["out"][1, 0], (0.25 * v[0, 0] + 0.75 * v[1, 0]) * sg[1, 0], rtol=1e-13, atol=1e-15)
    assert np.allclose(r["out"][0, 0], v[0, 0] * sg[0, 0], rtol=1e-14)


def test_first_token_and_uniform_keys():
    """A sequence's first token sees only itself; keys with no rotary part
    and equal values give uniform weights, so each query averages the
    values of its causal prefix."""
    rng = _rng(6)
    T, Hq, Hk, D = 9, 6, 1, 256
    cu = np.array([0, 4, 9])
    q = rng.standard_normal((T, Hq, D))
    k = np.tile(rng.standard_normal(D), (T, Hk, 1))
    k[..., :64] = 0.0
    v = rng.standard_normal((T, Hk, D))
    gate = rng.standard_normal((T, Hq, D))
    r = A.prefill(q, k, v, gate, np.ones(D), np.ones(D), cu)
    sg = 1 / (1 + np.exp(-gate))
    for t in range(T):
        t0 = 0 if t < 4 else 4
        for h in range(Hq):
            want = v[t0:t + 1, 0].mean(axis=0) * sg[t, h]
            assert np.allclose(r["out"][t, h], want, rtol=1e-12, atol=1e-14)


def test_gqa_head_mapping():
    """Query heads 0..5 read key/value head 0 and 6..11 head 1: with the
    second kv head equal to the first, heads h and h + 6 (same q) agree,
    and changing kv head 1 changes only heads 6..11."""
    rng = _rng(7)
    T, D = 6, 256
    q = rng.standard_normal((T, 12, D))
    q[:, 6:] = q[:, :6]
    k = rng.standard_normal((T, 2, D))
    v = rng.standard_normal((T, 2, D))
    k[:, 1], v[:, 1] = k[:, 0], v[:, 0]
    gate = rng.standard_normal((T, 12, D))
    gate[:, 6:] = gate[:, :6]
    cu = np.array([0, T])
    r = A.prefill(q, k, v, gate, np.ones(D), np.ones(D), cu)
    assert np.allclose(r["out"][:, :6], r["out"][:, 6:], rtol=1e-13)
    v2 = v.copy()
    v2[:, 1] += 1.0
    r2 = A.prefill(q, k, v2, gate, np.ones(D), np.ones(D), cu)
    assert np.array_equal(r2["out"][:, :6], r["out"][:, :6])
    assert not np.allclose(r2["out"][:, 6:], r["out"][:, 6:])


def test_packed_equals_separate():
    rng = _rng(8)
    D = 256
    lens = [3, 1, 5]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, gate = rng.standard_normal((T, 6, D)), rng.standard_normal((T, 6, D))
    k, v = rng.standard_normal((T, 1, D)), rng.standard_normal((T, 1, D))
    wq, wk = 1 + 0.1 * rng.standard_normal(D), 1 + 0.1 * rng.standard_normal(D)
    packed = A.prefill(q, k, v, gate, wq, wk, cu)["out"]
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        sep = A.prefill(q[a:b], k[a:b], v[a:b], gate[a:b], wq, wk, np.array([0, b - a]))["out"]
        assert np.array_equal(packed[a:b], sep)


def test_decode_equals_last_prefill_row():
    """Decoding token t against the cached, rotated keys of tokens 0..t-1 of
    the same sequence gives the prefill's output row t."""
    rng = _rng(9)
    D, T = 256, 11
    q, gate = rng.standard_normal((T, 6, D)), rng.standard_normal((T, 6, D))
    k, v = rng.standard_normal((T, 1, D)), rng.standard_normal((T, 1, D))
    wq, wk = 1 + 0.1 * rng.standard_normal(D), 1 + 0.1 * rng.standard_normal(D)
    pre = A.prefill(q, k, v, gate, wq, wk, np.array([0, T]))
    L = 16
    kc = np.zeros((1, L, 1, D))
    vc = np.zeros((1, L, 1, D))
    kc[0, :T - 1] = pre["k_rot"][:T - 1]
    vc[0, :T - 1] = v[:T - 1]
    dec = A.decode(q[T - 1:], k[T - 1:], v[T - 1:], gate[T - 1:], wq, wk, kc, vc, np.array([T - 1]))
    assert np.allclose(dec["out"][0], pre["out"][T - 1], rtol=1e-12, atol=1e-14)
    assert np.allclose(dec["k_cache"][0, T - 1], pre["k_rot"][T - 1], rtol=1e-13)
    assert np.array_equal(dec["v_cache"][0, T - 1], v[T - 1])
