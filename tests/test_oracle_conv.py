"""Pins of the conv / gate / gated-norm oracle (CPU only)."""
import numpy as np
import pytest

from oracle import conv
from inputs import synth


def _bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


# --- bf16 rounding -----------------------------------------------------------

def test_round_bf16_ties_to_even_and_exact_values():
    one = 1.0
    vals = np.array([one, one + 2 ** -8, one + 3 * 2 ** -8, one + 2 ** -8 + 2 ** -20, -2.5, 0.0, -0.0,
                     np.inf, 3.0e38], dtype=np.float32)
    out = conv.round_bf16(vals)
    assert out[0] == 1.0
    assert out[1] == 1.0  # tie -> even mantissa
    assert out[2] == one + 2 ** -6  # tie -> even (odd neighbour rejected)
    assert out[3] == one + 2 ** -7  # above the tie -> up
    assert out[4] == -2.5 and out[5] == 0.0 and np.signbit(out[6])
    assert out[7] == np.inf
    assert np.isnan(conv.round_bf16(np.float32([np.nan])))[0]
    # every result is a bf16 value: low 16 bits clear
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    b = conv.round_bf16(r)
    assert not np.any(b.view(np.uint32) & 0xFFFF)
    assert np.all(np.abs(b - r) <= 0.5 * _bf16_ulp(r) * (1 + 1e-7))


# --- exp32 / silu32 ----------------------------------------------------------

def test_exp32_within_2_ulp_of_exp():
    x = np.linspace(-87.0, 88.7, 1_000_001).astype(np.float32)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(conv.exp32(x) - ref) / ulp) <= 2.0


def test_exp32_special_values():
    e = conv.exp32(np.float32([0.0, -0.0, 100.0, -200.0, np.inf, -np.inf, np.nan]))
    assert e[0] == 1.0 and e[1] == 1.0
    assert e[2] == np.inf and e[3] == 0.0 and e[4] == np.inf and e[5] == 0.0
    assert np.isnan(e[6])


def test_silu32_special_values_and_accuracy():
    s = conv.silu32(np.float32([0.0, 30.0, -30.0, -200.0]))
    assert s[0] == 0.0
    assert s[1] == np.float32(30.0)  # sigmoid(30) rounds to 1 in float32
    assert -1e-11 < s[2] < 0.0
    assert s[3] == 0.0 and np.signbit(s[3])  # v / inf = -0
    v = np.random.default_rng(1).standard_normal(200000).astype(np.float32) * 5
    ref = v / (1 + np.exp(-v.astype(np.float64)))
    assert np.max(np.abs(conv.silu32(v) - ref) / np.maximum(np.abs(ref), 1e-30)) < 5e-7


# --- conv --------------------------------------------------------------------

def _small_conv_case(seed=2, lens=(7, 1, 12, 3, 0, 20), C=24):
    r = np.random.default_rng(seed)
    cu = synth.cu_seqlens_of(lens)
    T = int(cu[-1])
    x = synth.round_bf16(r.standard_normal((T, C)))
    w = synth.round_bf16(r.uniform(-0.5, 0.5, (C, 4)))
    return x, w, cu


def test_conv_fp32_within_one_bf16_ulp_of_fp64():
    x, w, cu = _small_conv_case()
    y64 = conv.conv_silu(x, w, cu)
    y32 = conv.conv_silu_fp32(x, w, cu)
    assert np.all(np.abs(y32 - y64) <= _bf16_ulp(y64) + 1e-30)
    p = synth.pipeline_inputs(lengths=[40, 300, 7], hk=2, hv=6, d=16)
    y64 = conv.conv_silu(p.x, p.conv_w, p.cu_seqlens)
    y32 = conv.conv_silu_fp32(p.x, p.conv_w, p.cu_seqlens)
    assert np.all(np.abs(y32 - y64) <= _bf16_ulp(y64) + 1e-30)


def test_conv_tap_order():
    """Tap 3 multiplies the current token, tap 0 the token three steps back."""
    x, w, cu = _small_conv_case(lens=(10,), C=4)
    x, w = x.astype(np.float64), w.astype(np.float64)
    silu = lambda p: p / (1 + np.exp(-p))
    w3 = np.zeros_like(w)
    w3[:, 3] = w[:, 3]
    np.testing.assert_allclose(conv.conv_silu(x, w3, cu), silu(w[:, 3] * x), rtol=1e-15)
    w0 = np.zeros_like(w)
    w0[:, 0] = w[:, 0]
    shifted = np.concatenate([np.zeros((3, 4)), x[:-3]])
    np.testing.assert_allclose(conv.conv_silu(x, w0, cu), silu(w[:, 0] * shifted), rtol=1e-15)


def test_conv_history_zero_per_sequence():
    x, w, cu = _small_conv_case()
    y = conv.conv_silu_fp32(x, w, cu)
    for n in range(len(cu) - 1):
        sl = slice(cu[n], cu[n + 1])
        yn = conv.conv_silu_fp32(x[sl], w, np.array([0, cu[n + 1] - cu[n]]))
        assert np.array_equal(y[sl], yn)


def test_conv_state_carry_equals_single_pass():
    x, w, _ = _small_conv_case(lens=(30,))
    full = conv.conv_silu_fp32(x, w, np.array([0, 30]))
    st = None
    parts = []
    for a, b in ((0, 2), (2, 3), (3, 17), (17, 30)):
        cu = np.array([0, b - a])
        parts.append(conv.conv_silu_fp32(x[a:b], w, cu, st))
        st = conv.conv_state_out(x[a:b], cu, st)
    assert np.array_equal(np.concatenate(parts), full)
    assert np.array_equal(st[0], x[-3:].T)


def test_conv_state_out_short_sequences():
    x = np.arange(1, 13, dtype=np.float32).reshape(6, 2)
    cu = np.array([0, 1, 1, 6])
    hist = np.full((3, 2, 3), -1.0, dtype=np.float32)
    st = conv.conv_state_out(x, cu, hist)
    assert st.shape == (3, 2, 3)
    np.testing.assert_array_equal(st[0], [[-1, -1, 1], [-1, -1, 2]])  # one token
    np.testing.assert_array_equal(st[1], hist[1])  # empty sequence
    np.testing.assert_array_equal(st[2], x[3:6].T)


# --- gates -------------------------------------------------------------------

def test_gates_special_values():
    A_log = np.log(np.array([1.0, 4.0]))
    dt = np.array([0.0, 0.5])
    a = np.array([[0.0, -0.5], [800.0, 800.0], [-800.0, -800.0]])
    b = np.array([[0.0, 0.0], [40.0, -40.0], [1.0, -1.0]])
    g, beta = conv.gates(a, b, A_log, dt)
    np.testing.assert_allclose(g[0], [-np.log(2.0), -4 * np.log(2.0)], rtol=1e-15)
    np.testing.assert_allclose(g[1], [-800.0, -4 * 800.5], rtol=1e-15)  # softplus(x) -> x
    assert np.all(g[2] <= 0) and np.all(g[2] > -1e-300)  # softplus(-800) underflows to 0
    np.testing.assert_allclose(beta[0], [0.5, 0.5], rtol=0)
    np.testing.assert_allclose(beta[2, 0] + beta[2, 1], 1.0, rtol=1e-15)
    assert beta[1, 0] == 1.0 and 0 < beta[1, 1] < 1e-17


def test_gates_match_naive_formula():
    r = np.random.default_rng(3)
    a, b = r.standard_normal((2, 50, 6)) * 3
    A_log, dt = r.uniform(0, np.log(16), 6), r.uniform(-1, 1, 6)
    g, beta = conv.gates(a, b, A_log, dt)
    np.testing.assert_allclose(g, -np.exp(A_log) * np.log(1 + np.exp(a + dt)), rtol=1e-11)
    np.testing.assert_allclose(beta, np.exp(b) / (np.exp(b) + 1), rtol=1e-14)
    assert np.all(g < 0)


# --- gated RMSNorm -----------------------------------------------------------

def test_gated_rmsnorm_properties():
    r = np.random.default_rng(4)
    o = r.standard_normal((5, 3, 16))
    z = r.standard_normal((5, 3, 16))
    w = 1 + 0.1 * r.standard_normal(16)
    y = conv.gated_rmsnorm(o, z, w, eps=0.0)
    silu = z / (1 + np.exp(-z))
    u = y / (w * silu)
    np.testing.assert_allclose(np.mean(u * u, -1), 1.0, rtol=1e-13)  # unit RMS before the gate
    np.testing.assert_allclose(u * np.sqrt(np.mean(o * o, -1, keepdims=True)), o, rtol=1e-13)
    # scale invariance in o, and a constant row normalises to sign(c)
    np.testing.assert_allclose(conv.gated_rmsnorm(7.5 * o, z, w, eps=0.0), y, rtol=1e-13)
    c = np.full((1, 16), -3.0)
    np.testing.assert_allclose(conv.gated_rmsnorm(c, np.full((1, 16), 50.0), np.ones(16), eps=0.0),
                               np.full((1, 16), -50.0), rtol=1e-15)
    # eps only matters for tiny rows
    tiny = np.full((1, 16), 1e-4)
    yt = conv.gated_rmsnorm(tiny, np.full((1, 16), 50.0), np.ones(16), eps=1e-6)
    np.testing.assert_allclose(yt, 50.0 * 1e-4 / np.sqrt(1e-8 + 1e-6), rtol=1e-13)


def test_decode_layer_steps_equal_prefill_definitions():
    """Four chained decode-layer steps from zero conv and recurrent state equal,
    token for token, the prefill definitions on the 4-token sequences: the conv
    front (bit for bit), the recurrence on its outputs, and the gated norm; the
    conv pool ends holding each row's last three inputs, slots by index."""
    from oracle import gdr
    cref = conv
    r = np.random.default_rng(40)
    N, hk, hv, d, T, P = 3, 1, 2, 8, 4, 5
    C = (2 * hk + hv) * d
    idx = np.array([4, 0, 2])
    x = cref.round_bf16(r.standard_normal((N, T, C)))
    w = cref.round_bf16(r.uniform(-0.5, 0.5, (C, 4)))
    a = r.standard_normal((N, T, hv))
    b = r.standard_normal((N, T, hv))
    A_log, dt = r.uniform(0, 1, hv), r.uniform(-1, 1, hv)
    z = r.standard_normal((N, T, hv * d))
    nw = 1 + 0.1 * r.standard_normal(d)
    conv_pool = np.zeros((P, C, 3), np.float32)
    pool = np.zeros((P, hv, d, d))
    ys, os_, qkvs = [], [], []
    for t in range(T):
        y, o, qkv, conv_pool, pool = gdr.decode_layer_step(x[:, t], w, conv_pool, a[:, t], b[:, t], A_log, dt, pool,
                                                           z[:, t], nw, hk, hv, state_indices=idx)
        ys.append(y), os_.append(o), qkvs.append(qkv)
    cu = np.arange(0, N * T + 1, T)
    flat = x.reshape(N * T, C)
    conv_ref = cref.conv_silu_fp32(flat, w, cu).reshape(N, T, C)
    assert np.array_equal(np.stack(qkvs, 1), conv_ref)
    assert np.array_equal(conv_pool[idx], cref.conv_state_out(flat, cu))
    q = conv_ref[..., :hk * d].reshape(N, T, hk, d)
    k = conv_ref[..., hk * d:2 * hk * d].reshape(N, T, hk, d)
    v = conv_ref[..., 2 * hk * d:].reshape(N, T, hv, d)
    g, beta = cref.gates(a, b, A_log, dt)
    o_ref, s_ref = gdr.forward(q, k, v, g, beta)
    np.testing.assert_allclose(np.stack(os_, 1), o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(pool[idx], s_ref, rtol=1e-12, atol=1e-14)
    y_ref = cref.gated_rmsnorm(o_ref, z.reshape(N, T, hv, d), nw).reshape(N, T, hv * d)
    np.testing.assert_allclose(np.stack(ys, 1), y_ref, rtol=1e-12, atol=1e-14)
    assert np.all(pool[[1, 3]] == 0) and np.all(conv_pool[[1, 3]] == 0)
