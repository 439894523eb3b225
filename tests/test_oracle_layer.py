"""Pins of the whole-layer oracle (CPU only): the projection product against
exact rational arithmetic, and the layer's block order and rounding points
against selection weights whose products are known exactly."""
from fractions import Fraction

import numpy as np

from inputs import synth
from oracle import conv as cv
from oracle import gdr
from oracle import layer


def test_linear_is_exact_for_small_bf16_products():
    """x W^T for bf16 values: every product is exact and, at K = 7 with this
    value range, so is the float64 sum; compared with Fraction arithmetic,
    element by element, on a non-square case (a transposed operand fails)."""
    x, w = synth.matmul_inputs(3, 5, 3, 7)
    y = layer.linear(x, w)
    assert y.shape == (5, 3)
    for m in range(5):
        for n in range(3):
            exact = sum(Fraction(float(x[m, k])) * Fraction(float(w[n, k])) for k in range(7))
            assert Fraction(float(y[m, n])) == exact


def _selection_layer(hk=1, hv=2, d=32, H=256, lengths=(37, 0, 5)):
    """A layer whose input projection copies hidden columns 0..C+V+2hv-1 and
    whose output projection copies y into output columns 0..V-1."""
    C, V = (2 * hk + hv) * d, hv * d
    L = synth.layer_inputs(11, lengths=lengths, hk=hk, hv=hv, d=d, hidden=H)
    w_in = np.zeros((C + V + 2 * hv, H), np.float32)
    w_in[:, :C + V + 2 * hv] = np.eye(C + V + 2 * hv, dtype=np.float32)
    w_out = np.zeros((H, V), np.float32)
    w_out[:V] = np.eye(V, dtype=np.float32)
    return L, w_in, w_out, C, V


def test_layer_block_order_and_rounding_points():
    """With selection weights the projections are exact copies of hidden
    columns, so every stage must equal the stage oracles applied to the
    matching slices: q|k|v first, then z, then b, then a; y rounded to bf16
    and carried unchanged into the output's first V columns."""
    hk, hv, d = 1, 2, 32
    L, w_in, w_out, C, V = _selection_layer(hk, hv, d)
    st0 = np.random.default_rng(4).standard_normal((3, hv, d, d)) * 0.1
    r = layer.delta_layer_forward(L.hidden, w_in, L.conv_w, L.A_log, L.dt_bias, L.norm_w, w_out, L.cu_seqlens,
                                  hk, hv, initial_state=st0)
    h = L.hidden
    T = h.shape[0]
    assert np.array_equal(r["qkv"], h[:, :C])
    assert np.array_equal(r["z"], h[:, C:C + V])
    assert np.array_equal(r["b"], h[:, C + V:C + V + hv])
    assert np.array_equal(r["a"], h[:, C + V + hv:C + V + 2 * hv])
    xc = cv.conv_silu_fp32(h[:, :C], L.conv_w, L.cu_seqlens)
    g, beta = cv.gates(h[:, C + V + hv:C + V + 2 * hv], h[:, C + V:C + V + hv], L.A_log, L.dt_bias)
    o, fin = gdr.forward(xc[:, :hk * d].reshape(1, T, hk, d), xc[:, hk * d:2 * hk * d].reshape(1, T, hk, d),
                         xc[:, 2 * hk * d:].reshape(1, T, hv, d), g[None], beta[None], st0, L.cu_seqlens)
    assert np.array_equal(r["o"], o) and np.array_equal(r["final_state"], fin)
    y = cv.round_bf16(cv.gated_rmsnorm(o[0], h[:, C:C + V].reshape(T, hv, d), L.norm_w).reshape(T, V))
    assert np.array_equal(r["y"], y)
    assert not np.any(r["y"].view(np.uint32) & 0xFFFF)
    assert np.array_equal(r["out"][:, :V], y) and not np.any(r["out"][:, V:])


def test_layer_swapped_gates_change_the_output():
    """b and a play different roles (write strength vs decay): exchanging
    their projection rows changes the layer output, so the block order pin
    above has teeth."""
    hk, hv, d = 1, 2, 32
    L, w_in, w_out, C, V = _selection_layer(hk, hv, d, lengths=(40,))
    sw = w_in.copy()
    sw[C + V:C + V + hv], sw[C + V + hv:] = w_in[C + V + hv:], w_in[C + V:C + V + hv]
    args = (L.conv_w, L.A_log, L.dt_bias, L.norm_w, w_out, L.cu_seqlens, hk, hv)
    r1 = layer.delta_layer_forward(L.hidden, w_in, *args)
    r2 = layer.delta_layer_forward(L.hidden, sw, *args)
    assert np.max(np.abs(r1["out"] - r2["out"])) > 1e-2
