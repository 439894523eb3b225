"""Pins of the fp64 recurrence oracle (CPU only).

Each test checks the oracle against something other than itself: a hand-worked
example, exact rational closed forms, textbook special cases of the delta rule,
invariants of the recurrence, or the independent chunk-form rewrite.  A dropped
term, a wrong sign, a transposed state or a wrong head/sequence index fails at
least one of them.
"""
import json
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import gdr
from inputs import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac_array(rows):
    return np.array([[Fr(x) for x in r] for r in rows], dtype=object)


def _rand_inputs(seed, B=1, T=40, hk=2, hv=6, d=8, dv=None, scale_g=1.0):
    r = np.random.default_rng(seed)
    dv = d if dv is None else dv
    q = r.standard_normal((B, T, hk, d))
    k = r.standard_normal((B, T, hk, d))
    v = r.standard_normal((B, T, hv, dv))
    g = -scale_g * np.abs(r.standard_normal((B, T, hv)))
    beta = r.uniform(0.05, 0.95, (B, T, hv))
    return q, k, v, g, beta


# --- hand-worked example ---------------------------------------------------

def test_hand_worked_example_exact():
    """Oracle core vs a d=2, T=3 example worked by hand in fractions."""
    ex = json.load(open(os.path.join(GOLDEN, "hand_worked_d2.json")))
    alpha = np.array([[Fr(a)] for a in ex["alpha"]], dtype=object)
    beta = np.array([[Fr(b)] for b in ex["beta"]], dtype=object)
    k = _frac_array(ex["k"])[:, None, :]
    v = _frac_array(ex["v"])[:, None, :]
    q = _frac_array(ex["q"])[:, None, :]
    S0 = np.zeros((1, 2, 2), dtype=object) * Fr(0)
    for T in (1, 2, 3):
        o, S = gdr.recurrence(S0, alpha[:T], beta[:T], k[:T], v[:T], q[:T], Fr(1))
        assert (S[0] == _frac_array(ex["expected_states"][T - 1])).all()
    assert (o[:, 0] == _frac_array(ex["expected_o"])).all()


def test_hand_worked_example_public_api():
    """Same example through ``forward`` (g = log alpha, no normalisation), fp64."""
    ex = json.load(open(os.path.join(GOLDEN, "hand_worked_d2.json")))
    f = lambda rows: np.array([[float(Fr(x)) for x in r] for r in rows])
    alpha = np.array([float(Fr(a)) for a in ex["alpha"]])
    beta = np.array([float(Fr(b)) for b in ex["beta"]])
    q, k, v = f(ex["q"]), f(ex["k"]), f(ex["v"])
    o, S = gdr.forward(q[None, :, None], k[None, :, None], v[None, :, None],
                       np.log(alpha)[None, :, None], beta[None, :, None], use_qk_l2norm=False)
    np.testing.assert_allclose(o[0, :, 0], f(ex["expected_o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], f(ex["expected_states"][2]), rtol=0, atol=1e-14)


# --- closed form (unrolled product of matrices), exact rational arithmetic ---

def _closed_form_states(S0, alpha, beta, k, v):
    """S_t = S0 prod_{s<=t} A_s + sum_{j<=t} beta_j v_j k_j^T prod_{j<s<=t} A_s,
    A_s = alpha_s (I - beta_s k_s k_s^T), evaluated literally with explicit matrices."""
    T, d = len(alpha), S0.shape[1]
    I = np.array([[Fr(int(i == j)) for j in range(d)] for i in range(d)], dtype=object)
    A = [alpha[s] * (I - beta[s] * np.outer(k[s], k[s])) for s in range(T)]
    out = []
    for t in range(T):
        P = I.copy()
        for s in range(t + 1):
            P = P.dot(A[s])
        St = S0.dot(P)
        for j in range(t + 1):
            Pj = I.copy()
            for s in range(j + 1, t + 1):
                Pj = Pj.dot(A[s])
            St = St + (beta[j] * np.outer(v[j], k[j])).dot(Pj)
        out.append(St)
    return out


@pytest.mark.parametrize("seed,T,d,dv", [(0, 6, 3, 3), (1, 9, 4, 2), (2, 12, 2, 5)])
def test_closed_form_exact_rational(seed, T, d, dv):
    r = np.random.default_rng(seed)
    rat = lambda *shape: np.vectorize(lambda x: Fr(int(x), 7))(r.integers(-9, 10, size=shape)).astype(object)
    S0 = rat(dv, d)
    alpha = np.array([Fr(int(x), 8) for x in r.integers(1, 9, size=T)], dtype=object)
    beta = np.array([Fr(int(x), 5) for x in r.integers(0, 6, size=T)], dtype=object)
    k, v, q = rat(T, d), rat(T, dv), rat(T, d)
    states = _closed_form_states(S0, alpha, beta, k, v)
    o, S = gdr.recurrence(S0[None], alpha[:, None], beta[:, None], k[:, None], v[:, None],
                          q[:, None], Fr(1))
    assert (S[0] == states[-1]).all()
    for t in range(T):
        assert (o[t, 0] == states[t].dot(q[t])).all()


def test_closed_form_fp64_random():
    r = np.random.default_rng(3)
    T, d = 10, 5
    S0 = r.standard_normal((d, d))
    alpha = r.uniform(0.2, 1.0, T)
    beta = r.uniform(0, 1, T)
    k = gdr.l2_normalise(r.standard_normal((T, d)), 0.0)
    v = r.standard_normal((T, d))
    q = r.standard_normal((T, d))
    I = np.eye(d)
    S_lit = S0.copy()
    for t in range(T):  # literal form of the formula, one matrix product per token
        S_lit = alpha[t] * S_lit @ (I - beta[t] * np.outer(k[t], k[t])) + beta[t] * np.outer(v[t], k[t])
    o, S = gdr.recurrence(S0[None], alpha[:, None], beta[:, None], k[:, None], v[:, None], q[:, None])
    np.testing.assert_allclose(S[0], S_lit, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[-1, 0], S_lit @ q[-1], rtol=0, atol=1e-12)


# --- special cases -----------------------------------------------------------

def test_identity_when_beta_and_g_zero():
    q, k, v, g, beta = _rand_inputs(4)
    S0 = np.random.default_rng(5).standard_normal((1, 6, 8, 8))
    o, S = gdr.forward(q, k, v, 0 * g, 0 * beta, S0)
    assert np.array_equal(S, S0)  # bit-exact: S*1 + 0
    qh = gdr.l2_normalise(q)
    kmap = gdr.head_map(2, 6)
    ref = np.einsum("hvk,thk->thv", S0[0], qh[0][:, kmap])
    np.testing.assert_allclose(o[0], ref, rtol=1e-14, atol=1e-14)


def test_recall_with_unit_key_and_beta_one():
    """beta = 1, unit k: S_t k_t = v_t (erase-then-write)."""
    q, k, v, g, _ = _rand_inputs(6, T=30)
    S0 = np.random.default_rng(7).standard_normal((1, 6, 8, 8))
    kh = gdr.l2_normalise(k, 0.0)
    kmap = gdr.head_map(2, 6)
    for T in (1, 5, 30):
        _, S = gdr.forward(q[:, :T], kh[:, :T], v[:, :T], g[:, :T], np.ones((1, T, 6)), S0,
                           use_qk_l2norm=False)
        recall = np.einsum("hvk,hk->hv", S[0], kh[0, T - 1][kmap])
        np.testing.assert_allclose(recall, v[0, T - 1], rtol=0, atol=1e-13 * np.abs(v).max())


def test_orthonormal_keys_associative_memory():
    """g = 0, beta = 1, standard-basis keys: every stored pair is recalled exactly;
    writing a key again overwrites its value and leaves the others."""
    d, dv = 4, 3
    r = np.random.default_rng(8)
    keys = [0, 2, 1, 3, 2]
    vals = r.integers(-5, 6, size=(len(keys), dv)).astype(float)
    k = np.eye(d)[keys][None, :, None]
    v = vals[None, :, None]
    T = len(keys)
    _, S = gdr.forward(np.zeros((1, T, 1, d)), k, v, np.zeros((1, T, 1)), np.ones((1, T, 1)),
                       use_qk_l2norm=False)
    latest = {kk: vals[t] for t, kk in enumerate(keys)}
    for kk, val in latest.items():
        assert np.array_equal(S[0, 0][:, kk], val)
    assert set(latest) == set(range(d))


def test_decay_only_when_beta_zero():
    q, k, v, g, beta = _rand_inputs(9, T=25)
    S0 = np.random.default_rng(10).standard_normal((1, 6, 8, 8))
    o, S = gdr.forward(q, k, v, g, 0 * beta, S0)
    decay = np.exp(np.cumsum(g[0], axis=0))  # [T, H]
    np.testing.assert_allclose(S[0], decay[-1][:, None, None] * S0[0], rtol=1e-12)
    qh = gdr.l2_normalise(q)[0][:, gdr.head_map(2, 6)]
    ref = decay[:, :, None] * np.einsum("hvk,thk->thv", S0[0], qh)
    np.testing.assert_allclose(o[0], ref, rtol=1e-12, atol=1e-300)


def test_full_reset_when_alpha_zero():
    """g = -inf (alpha = 0): S_t = beta v k^T, o_t = beta (k.q) v."""
    q, k, v, g, beta = _rand_inputs(11, T=7)
    S0 = np.random.default_rng(12).standard_normal((1, 6, 8, 8))
    o, S = gdr.forward(q, k, v, np.full_like(g, -np.inf), beta, S0)
    kmap = gdr.head_map(2, 6)
    kh, qh = gdr.l2_normalise(k)[0][:, kmap], gdr.l2_normalise(q)[0][:, kmap]
    np.testing.assert_allclose(S[0], beta[0, -1][:, None, None] * v[0, -1][:, :, None] * kh[-1][:, None, :],
                               rtol=1e-14, atol=1e-15)
    ref = (beta[0] * np.sum(kh * qh, -1))[:, :, None] * v[0]
    np.testing.assert_allclose(o[0], ref, rtol=1e-13, atol=1e-15)


def test_repeated_key_geometric_closed_form():
    """Same unit key and value n times with constant alpha = a, beta = b (the
    Widrow-Hoff / LMS step with gain b): x_n = S_n k obeys x_n = a(1-b) x_{n-1} + b v,
    so x_n = (a(1-b))^n x_0 + b v sum_{i<n} (a(1-b))^i."""
    d, n = 6, 20
    r = np.random.default_rng(13)
    kk = gdr.l2_normalise(r.standard_normal(d), 0.0)
    vv = r.standard_normal(d)
    a, b = 0.9, 0.3
    S0 = r.standard_normal((1, 1, d, d))
    _, S = gdr.forward(np.zeros((1, n, 1, d)), np.tile(kk, (1, n, 1, 1)), np.tile(vv, (1, n, 1, 1)),
                       np.full((1, n, 1), np.log(a)), np.full((1, n, 1), b), S0, use_qk_l2norm=False)
    x0 = S0[0, 0] @ kk
    rho = a * (1 - b)
    xn = rho ** n * x0 + b * vv * sum(rho ** i for i in range(n))
    np.testing.assert_allclose(S[0, 0] @ kk, xn, rtol=1e-12, atol=1e-13)


# --- invariants --------------------------------------------------------------

def test_linear_in_state_and_values():
    q, k, v, g, beta = _rand_inputs(14, T=30)
    r = np.random.default_rng(15)
    S1, S2 = r.standard_normal((2, 1, 6, 8, 8))
    v2 = r.standard_normal(v.shape)
    a, b = 0.7, -1.3
    o1, f1 = gdr.forward(q, k, v, g, beta, S1)
    o2, f2 = gdr.forward(q, k, v2, g, beta, S2)
    o3, f3 = gdr.forward(q, k, a * v + b * v2, g, beta, a * S1 + b * S2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(f3, a * f1 + b * f2, rtol=1e-11, atol=1e-12)


def test_state_norm_bound():
    """||S_t||_2 <= alpha_t ||S_{t-1}||_2 + beta_t ||v_t|| for beta in [0,1], unit k."""
    q, k, v, g, beta = _rand_inputs(16, T=40, hk=1, hv=1, scale_g=0.05)
    kh = gdr.l2_normalise(k, 0.0)
    S = np.random.default_rng(17).standard_normal((1, 1, 8, 8))
    for t in range(40):
        _, S_new = gdr.forward(q[:, t:t + 1], kh[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1],
                               beta[:, t:t + 1], S, use_qk_l2norm=False)
        bound = np.exp(g[0, t, 0]) * np.linalg.norm(S[0, 0], 2) + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert np.linalg.norm(S_new[0, 0], 2) <= bound * (1 + 1e-12)
        S = S_new


def test_head_map_groups_of_three():
    """Value head h must read key head h // 3: perturb key head 1 only."""
    q, k, v, g, beta = _rand_inputs(18, T=12, hk=2, hv=6)
    o1, _ = gdr.forward(q, k, v, g, beta)
    k2 = k.copy()
    k2[:, :, 1] = np.random.default_rng(19).standard_normal(k2[:, :, 1].shape)
    o2, _ = gdr.forward(q, k2, v, g, beta)
    changed = [h for h in range(6) if not np.array_equal(o1[..., h, :], o2[..., h, :])]
    assert changed == [3, 4, 5]
    assert list(gdr.head_map(16, 48)[[0, 2, 3, 47]]) == [0, 0, 1, 15]


def test_l2norm_scale_invariance():
    q, k, v, g, beta = _rand_inputs(20, T=16)
    o1, s1 = gdr.forward(q, k, v, g, beta, eps=0.0)
    o2, s2 = gdr.forward(3.0 * q, 0.25 * k, v, g, beta, eps=0.0)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s2, s1, rtol=1e-12, atol=1e-13)


def test_query_scale_is_linear():
    q, k, v, g, beta = _rand_inputs(21, T=9)
    o1, s1 = gdr.forward(q, k, v, g, beta)
    o2, s2 = gdr.forward(q, k, v, g, beta, scale=0.125)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-15)
    assert np.array_equal(s1, s2)


def test_varlen_equals_separate_sequences():
    lens = [5, 0, 17, 1, 33]
    cu = synth.cu_seqlens_of(lens)
    q, k, v, g, beta = _rand_inputs(22, T=int(cu[-1]))
    S0 = np.random.default_rng(23).standard_normal((len(lens), 6, 8, 8))
    o, S = gdr.forward(q, k, v, g, beta, S0, cu)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        o_n, S_n = gdr.forward(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], S0[n:n + 1])
        assert np.array_equal(o[:, sl], o_n)
        assert np.array_equal(S[n], S_n[0])
    assert np.array_equal(S[1], S0[1])  # empty sequence: final = initial


def test_nan_in_one_sequence_stays_there():
    lens = [9, 14, 6]
    cu = synth.cu_seqlens_of(lens)
    q, k, v, g, beta = _rand_inputs(24, T=int(cu[-1]))
    o1, S1 = gdr.forward(q, k, v, g, beta, None, cu)
    v2 = v.copy()
    v2[0, cu[1] + 3] = np.nan
    o2, S2 = gdr.forward(q, k, v2, g, beta, None, cu)
    for n in (0, 2):
        sl = slice(cu[n], cu[n + 1])
        assert np.array_equal(o1[:, sl], o2[:, sl]) and np.array_equal(S1[n], S2[n])
    assert np.isnan(S2[1]).any()


def test_chained_calls_equal_single_call():
    q, k, v, g, beta = _rand_inputs(25, T=96)
    o, S = gdr.forward(q, k, v, g, beta)
    state, outs = None, []
    for a, b in ((0, 32), (32, 33), (33, 96)):
        o_p, state = gdr.forward(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], state)
        outs.append(o_p)
    assert np.array_equal(np.concatenate(outs, 1), o)
    assert np.array_equal(state, S)


def test_decode_step_equals_one_token_prefill():
    r = np.random.default_rng(26)
    N, hk, hv, d = 5, 2, 6, 8
    q, k = r.standard_normal((2, N, hk, d))
    v = r.standard_normal((N, hv, d))
    g = -np.abs(r.standard_normal((N, hv)))
    beta = r.uniform(0, 1, (N, hv))
    S0 = r.standard_normal((N, hv, d, d))
    o, S = gdr.decode_step(q, k, v, g, beta, S0)
    o_ref, S_ref = gdr.forward(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None], S0)
    np.testing.assert_allclose(o, o_ref[:, 0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S, S_ref, rtol=1e-14, atol=1e-15)


def test_decode_step_pool_indexing():
    """Pool decode = per-row one-token prefill from the named slot; padding rows
    (index < 0 or >= pool size) give o = 0; unnamed slots keep their values."""
    r = np.random.default_rng(28)
    N, hk, hv, d, P = 6, 2, 6, 8, 9
    q, k = r.standard_normal((2, N, hk, d))
    v = r.standard_normal((N, hv, d))
    g = -np.abs(r.standard_normal((N, hv)))
    beta = r.uniform(0, 1, (N, hv))
    pool = r.standard_normal((P, hv, d, d))
    idx = np.array([7, -1, 0, 4, 9, 2])
    o, new = gdr.decode_step_pool(q, k, v, g, beta, pool, idx)
    for n in range(N):
        if 0 <= idx[n] < P:
            o1, s1 = gdr.forward(q[n:n + 1, None], k[n:n + 1, None], v[n:n + 1, None], g[n:n + 1, None],
                                 beta[n:n + 1, None], pool[idx[n]][None])
            np.testing.assert_allclose(o[n], o1[0, 0], rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(new[idx[n]], s1[0], rtol=1e-14, atol=1e-15)
        else:
            assert np.all(o[n] == 0)
    untouched = [p for p in range(P) if p not in set(idx.tolist())]
    assert np.array_equal(new[untouched], pool[untouched])
    with pytest.raises(ValueError):
        gdr.decode_step_pool(q, k, v, g, beta, pool, np.array([1, 1, -1, 2, 3, 4]))


def test_parallel_equals_serial():
    q, k, v, g, beta = _rand_inputs(27, T=20, hk=2, hv=6)
    o, S = gdr.forward(q, k, v, g, beta)
    o2, S2, n = gdr.forward_parallel(q, k, v, g, beta, processes=3)
    assert n == 3
    assert np.array_equal(o, o2) and np.array_equal(S, S2)


# --- chunk form equals token-serial form -------------------------------------

@pytest.mark.parametrize("C", [1, 2, 8, 32, 64, 100])
def test_chunked_equals_stepwise(C):
    lens = [100, 37, 64, 1]
    cu = synth.cu_seqlens_of(lens)
    q, k, v, g, beta = _rand_inputs(28, T=int(cu[-1]), d=16, dv=12)
    S0 = np.random.default_rng(29).standard_normal((len(lens), 6, 12, 16))
    o, S = gdr.forward(q, k, v, g, beta, S0, cu)
    oc, Sc = gdr.chunked(q, k, v, g, beta, S0, cu, chunk_size=C)
    scale_o, scale_s = np.abs(o).max(), np.abs(S).max()
    assert np.abs(oc - o).max() <= 1e-12 * scale_o
    assert np.abs(Sc - S).max() <= 1e-12 * scale_s


def test_chunked_equals_stepwise_tiny_config():
    x = synth.tiny_config()
    o, S = gdr.forward(x.q, x.k, x.v, x.g, x.beta)
    oc, Sc = gdr.chunked(x.q, x.k, x.v, x.g, x.beta, chunk_size=32)
    assert np.abs(oc - o).max() <= 1e-12 * np.abs(o).max()
    assert np.abs(Sc - S).max() <= 1e-12 * np.abs(S).max()


def test_chunked_equals_stepwise_layer_shape_strong_decay():
    """Full head geometry (d=128, chunk 64) with the recipe's strong decays, 3 heads."""
    x = synth.layer_prefill(T=160)
    heads = [0, 17, 47]
    o, S = gdr.forward(x.q, x.k, x.v, x.g, x.beta, heads=heads)
    oc, Sc = gdr.chunked(x.q, x.k, x.v, x.g, x.beta, chunk_size=64, heads=heads)
    assert np.abs(oc - o).max() <= 1e-12 * np.abs(o).max()
    assert np.abs(Sc - S).max() <= 1e-12 * np.abs(S).max()
