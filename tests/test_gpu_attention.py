"""GPU parity of the global attention layer (GQA, head dim 256, q/k RMS norm,
partial rotary, sigmoid gate) against the fp64 oracle.

Tolerances (derived from the arithmetic):
  * q' and k' are computed in fp32 (angles reduced in fp64) and rounded to
    bf16: within one bf16 ulp of the fp64 value plus 2^-20 of the magnitude
    of the terms that make it (the normed x_j, and for rotated dims also its
    pair partner), which covers the fp32 error where the two rotation terms
    cancel;
  * the attention output, checked against the oracle fed the GPU's own q'
    and k': the kernel rounds each probability to bf16 before the value
    product (relative error <= 2^-9) and sums in fp32, so each output is
    within 2^-9 of sum_j p_j |v_j| sigmoid(gate) of the exact value; the test
    allows 2^-8 of it, plus half a bf16 ulp for the output's own rounding.
"""
import numpy as np
import pytest

from gated_delta_rule_amd import synth
from oracle import attention as aref
from helpers import bf16_ulp, bits_equal, gpu, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _dev(x, dev):
    return (to_dev(x.q, "bf16", dev), to_dev(x.k, "bf16", dev), to_dev(x.v, "bf16", dev), to_dev(x.gate, "bf16", dev),
            to_dev(x.q_norm_w, "f32", dev), to_dev(x.k_norm_w, "f32", dev), to_dev(x.cu_seqlens, "i32", dev))


def _check_out(got, ref, mass):
    got = np.asarray(got, np.float64)
    tol = 2.0 ** -8 * mass + 0.5 * bf16_ulp(np.abs(ref)) + 1e-6
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"max err {err.max():.3e}, worst excess {(err - tol).max():.3e}"


@pytest.mark.parametrize("lengths", [(5, 1, 0, 130, 300), (1,), (40000,)])
def test_qk_norm_rope_within_one_ulp(lengths):
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    x = synth.attn_inputs(41, lengths=lengths)
    say(f"attention q/k norm + rotary, lengths {lengths}")
    q, k, v, g, qw, kw, cu = _dev(x, dev)
    qo, ko = gdr.attn_qk_norm_rope(q, k, qw, kw, cu)
    torch.cuda.synchronize()
    T = len(x.q)
    rows = np.unique(np.concatenate([np.arange(min(T, 64)), np.arange(max(0, T - 64), T)]))
    pos = aref.positions(x.cu_seqlens, T)[rows]
    qr, kr = aref.prep(x.q[rows], x.k[rows], pos, x.q_norm_w, x.k_norm_w)
    for got, ref, raw, w in ((qo, qr, x.q, x.q_norm_w), (ko, kr, x.k, x.k_norm_w)):
        xn = np.abs(aref.rms_norm(raw[rows], w))
        mag = xn.copy()
        mag[..., :32] += xn[..., 32:64]
        mag[..., 32:64] += xn[..., :32]
        err = np.abs(to_host(got)[rows] - ref)
        assert np.all(err <= bf16_ulp(ref) + 2.0 ** -20 * mag + 1e-30)


@pytest.mark.parametrize("lengths,hq,hk", [((1, 63, 64, 65, 200, 0, 129), 24, 4), ((300,), 8, 2),
                                           ((130, 257), 6, 1)])
def test_prefill_against_oracle(lengths, hq, hk):
    """Ragged and empty sequences, several kv-head groupings: the output
    within its bound of the oracle run on the GPU's q' and k'; the KV cache
    holds k' and v bit for bit."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    x = synth.attn_inputs(42, lengths=lengths, hq=hq, hk=hk)
    N, T = len(lengths), len(x.q)
    L = max(lengths) + 3
    say(f"attention prefill lengths {lengths} Hq={hq} Hk={hk}")
    q, k, v, g, qw, kw, cu = _dev(x, dev)
    kc = torch.zeros((N, L, hk, 256), device=dev, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    out = gdr.attn_prefill(q, k, v, g, qw, kw, cu, k_cache=kc, v_cache=vc)
    qo, ko = gdr.attn_qk_norm_rope(q, k, qw, kw, cu)
    torch.cuda.synchronize()
    r = aref.core_prefill(to_host(qo), to_host(ko), x.v, x.gate, x.cu_seqlens)
    _check_out(to_host(out), r["out"], r["mass"])
    for n in range(N):
        a, b = x.cu_seqlens[n], x.cu_seqlens[n + 1]
        assert bits_equal(kc[n, :b - a], ko[a:b])
        assert bits_equal(vc[n, :b - a], v[a:b])
        assert not torch.any(kc[n, b - a:].float() != 0)


def test_prefill_full_size_sampled():
    """One 32768-token sequence at the layer's head shape: 24 sampled query
    rows (tile edges, the last row) on 6 heads against the oracle."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    T = 32768
    x = synth.attn_inputs(43, lengths=(T,))
    say("attention prefill full size T=32768")
    q, k, v, g, qw, kw, cu = _dev(x, dev)
    out = gdr.attn_prefill(q, k, v, g, qw, kw, cu)
    qo, ko = gdr.attn_qk_norm_rope(q, k, qw, kw, cu)
    torch.cuda.synchronize()
    rng = synth.rng(44)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 4095, T - 129, T - 1], rng.choice(T, 15, replace=False)]))
    heads = [0, 5, 6, 13, 18, 23]
    r = aref.core_prefill(to_host(qo), to_host(ko), x.v, x.gate, x.cu_seqlens, heads=heads, rows=rows)
    got = to_host(out)
    for h in heads:
        _check_out(got[rows, h], r["out"][rows, h], r["mass"][rows, h])


def test_prefill_deterministic_and_finite():
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    x = synth.attn_inputs(45, lengths=(700, 33))
    q, k, v, g, qw, kw, cu = _dev(x, dev)
    say("attention prefill determinism")
    a = gdr.attn_prefill(q, k, v, g, qw, kw, cu)
    b = gdr.attn_prefill(q, k, v, g, qw, kw, cu)
    torch.cuda.synchronize()
    assert bits_equal(a, b)
    assert torch.isfinite(a.float()).all()
