"""GPU parity of the projection GEMM (gdr_linear) and the whole-layer prefill
(gdr_delta_layer_fwd) against the fp64 oracle.

Tolerance of a projection (derived from the arithmetic, not measured): the
GPU sums K exact bf16 x bf16 products in fp32, in some order, so each fp32
result is within K * 2^-24 * sum_k |x_k w_k| of the exact sum; a bf16 result
is that value rounded to nearest, so it is within the bound plus half a bf16
ulp of the result.
"""
import numpy as np
import pytest

from inputs import synth
from oracle import conv as cref
from oracle import gdr as gref
from oracle import layer as lref
from helpers import BF16_TOL, bf16_ulp, bits_equal, gpu, rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _bound(x, w, rows=None):
    """Per-element fp32 accumulation bound K 2^-24 sum |x||w| for rows of x."""
    xa = np.abs(np.asarray(x if rows is None else x[rows], np.float64))
    return x.shape[1] * 2.0 ** -24 * (xa @ np.abs(np.asarray(w, np.float64)).T)


def _check(got, ref, bound, bf16):
    got = np.asarray(got, np.float64)
    tol = bound + (0.5 * bf16_ulp(np.abs(ref) + bound) if bf16 else 0.0) + 1e-30
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"max err {err.max():.3e}, worst excess {(err - tol).max():.3e}"


@pytest.mark.parametrize("M,N,K", [(1, 4, 32), (70, 36, 64), (130, 200, 96), (256, 256, 128), (300, 260, 256),
                                   (513, 1000, 384), (4097, 772, 640), (77, 16480, 5120)])
def test_linear_matches_oracle(M, N, K):
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    x, w = synth.matmul_inputs(M + N + K, M, N, K)
    say(f"linear M={M} N={N} K={K}")
    xd, wd = to_dev(x, "bf16", dev), to_dev(w, "bf16", dev)
    y32 = gdr.linear(xd, wd, out_dtype=torch.float32)
    y16 = gdr.linear(xd, wd)
    torch.cuda.synchronize()
    ref = lref.linear(x, w)
    b = _bound(x, w)
    _check(to_host(y32), ref, b, False)
    _check(to_host(y16), ref, b, True)
    # bf16 output is the fp32 result rounded: the two calls agree bit for bit
    assert torch.equal(y16, y32.to(torch.bfloat16))


def test_linear_column_blocks():
    """Four output blocks of different widths and kinds, one of them empty and
    the others starting at columns that are not multiples of 4 (per-element
    stores at the seams): each receives exactly its columns."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    M, K = 333, 256
    blocks = [(517, torch.bfloat16), (0, torch.bfloat16), (103, torch.float32, True), (15, torch.float32)]
    N = sum(b[0] for b in blocks)
    x, w = synth.matmul_inputs(12, M, N, K)
    say("linear column blocks")
    xd, wd = to_dev(x, "bf16", dev), to_dev(w, "bf16", dev)
    outs = gdr.linear(xd, wd, blocks=blocks)
    full = gdr.linear(xd, wd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, b = lref.linear(x, w), _bound(x, w)
    c0 = 0
    for t, blk in zip(outs, blocks):
        cols = slice(c0, c0 + blk[0])
        rounded = blk[1] == torch.bfloat16 or (len(blk) > 2 and blk[2])
        _check(to_host(t), ref[:, cols], b[:, cols], rounded)
        if rounded:
            assert torch.equal(t.to(torch.float32), full[:, cols].to(torch.bfloat16).to(torch.float32))
        else:
            assert bits_equal(t, full[:, cols].contiguous())
        c0 += blk[0]


@pytest.mark.parametrize("M,N,K", [(32768, 16480, 5120), (32768, 5120, 6144)])
def test_linear_full_size_sampled_rows(M, N, K):
    """The layer's two projections at a 32768-token call: 40 sampled rows
    (both ends of the row tiles, the last row) checked in every column."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    gen = synth.rng(M, N, K)
    say(f"linear full size M={M} N={N} K={K}")
    x = torch.randn((M, K), generator=torch.Generator().manual_seed(K), dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=torch.Generator().manual_seed(N), dtype=torch.float32)
         / K ** 0.5).to(torch.bfloat16)
    y = gdr.linear(x.to(dev), w.to(dev))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095, M - 256, M - 1], gen.choice(M, 33, replace=False)]))
    xs = x[rows].float().numpy()
    wn = w.float().numpy()
    ref = lref.linear(xs, wn)
    b = K * 2.0 ** -24 * (np.abs(xs.astype(np.float64)) @ np.abs(wn.astype(np.float64)).T)
    _check(to_host(y[torch.as_tensor(rows, device=dev)]), ref, b, True)


def _layer_gpu(L, dev, st0=None, cs0=None):
    import gated_delta_rule_amd as gdr
    w = dict(hidden=to_dev(L.hidden, "bf16", dev), w_in=to_dev(L.w_in, "bf16", dev),
             conv_w=to_dev(L.conv_w, "bf16", dev), A_log=to_dev(L.A_log, "f32", dev),
             dt_bias=to_dev(L.dt_bias, "f32", dev), norm_w=to_dev(L.norm_w, "f32", dev),
             w_out=to_dev(L.w_out, "bf16", dev), cu_seqlens=to_dev(L.cu_seqlens, "i32", dev))
    out, fin, cso = gdr.delta_layer_fwd(**w, num_k_heads=L.hk, num_v_heads=L.hv, head_dim=L.d,
                                        initial_state=st0, output_final_state=True,
                                        conv_state_in=cs0, output_conv_state=True)
    return w, out, fin, cso


def _stages(L, w, dev, st0=None, cs0=None):
    """The layer as five separate ABI calls (same arguments)."""
    import gated_delta_rule_amd as gdr
    import torch
    hk, hv, d = L.hk, L.hv, L.d
    C, V = (2 * hk + hv) * d, hv * d
    qkv, z, b, a = gdr.linear(w["hidden"], w["w_in"], blocks=[(C, torch.bfloat16), (V, torch.bfloat16),
                                                               (hv, torch.float32, True), (hv, torch.float32, True)])
    q, k, v, g, beta, cso = gdr.conv_gate_fused(qkv, w["conv_w"], w["cu_seqlens"], a, b, w["A_log"], w["dt_bias"],
                                                hk, hv, d, conv_state_in=cs0, output_conv_state=True)
    o, fin = gdr.chunk_gated_delta_rule(q, k, v, g, beta, st0, output_final_state=True, cu_seqlens=w["cu_seqlens"])
    y = gdr.gated_rmsnorm(o[0], z, w["norm_w"])
    out = gdr.linear(y, w["w_out"])
    torch.cuda.synchronize()
    return dict(qkv=qkv, z=z, b=b, a=a, q=q, k=k, v=v, g=g, beta=beta, o=o, final_state=fin, y=y, out=out,
                conv_state=cso)


@pytest.mark.parametrize("lengths,hidden,hk,hv", [((300, 45, 1, 0), 256, 2, 6), ((700,), 512, 1, 3)])
def test_layer_small_against_oracle(lengths, hidden, hk, hv):
    """Whole layer on a packed batch (ragged lengths, an empty sequence,
    carried conv and recurrent state): equal bit for bit to the five steps
    called one by one, each step within its bound of the oracle fed that
    step's GPU inputs, and the output close to the oracle run end to end."""
    import torch
    dev = gpu()
    L = synth.layer_inputs(31, lengths=lengths, hk=hk, hv=hv, d=128, hidden=hidden)
    N = len(lengths)
    C, V = (2 * hk + hv) * 128, hv * 128
    gen = synth.rng(32)
    st0 = (0.05 * gen.standard_normal((N, hv, 128, 128))).astype(np.float32)
    cs0 = synth.round_bf16(gen.standard_normal((N, C, 3)))
    say(f"delta layer lengths={lengths} hidden={hidden} hk={hk} hv={hv}")
    st0d, cs0d = to_dev(st0, "f32", dev), to_dev(cs0, "bf16", dev)
    w, out, fin, cso = _layer_gpu(L, dev, st0d, cs0d)
    torch.cuda.synchronize()
    s = _stages(L, w, dev, st0d, cs0d)
    assert bits_equal(out, s["out"]) and bits_equal(fin, s["final_state"]) and bits_equal(cso, s["conv_state"])

    # in-projection
    ref = lref.linear(L.hidden, L.w_in)
    b = _bound(L.hidden, L.w_in)
    proj = np.concatenate([to_host(s[n]).reshape(len(L.hidden), -1) for n in ("qkv", "z", "b", "a")], 1)
    _check(proj, ref, b, True)
    # front, bit-exact on the GPU's projections
    qkv = to_host(s["qkv"]).astype(np.float32)
    xc = cref.conv_silu_fp32(qkv, L.conv_w, L.cu_seqlens, cs0)
    T = qkv.shape[0]
    gq = np.concatenate([to_host(s[n]).reshape(T, -1) for n in ("q", "k", "v")], 1)
    assert np.array_equal(gq, xc)
    assert np.array_equal(to_host(s["conv_state"]), cref.conv_state_out(qkv, L.cu_seqlens, cs0))
    # recurrence on the GPU's front outputs
    o_ref, f_ref = gref.forward(*(to_host(s[n]).astype(np.float32) for n in ("q", "k", "v", "g", "beta")), st0,
                                L.cu_seqlens)
    assert rel_err(to_host(s["o"]), o_ref) <= BF16_TOL
    assert rel_err(to_host(s["final_state"]), f_ref) <= BF16_TOL
    # norm on the GPU's o and z (one bf16 ulp)
    y_ref = cref.gated_rmsnorm(to_host(s["o"])[0], to_host(s["z"]).reshape(T, hv, 128), L.norm_w).reshape(T, V)
    assert np.all(np.abs(to_host(s["y"]) - y_ref) <= bf16_ulp(y_ref) + 1e-30)
    # out-projection on the GPU's y
    yh = to_host(s["y"]).astype(np.float32)
    _check(to_host(out), lref.linear(yh, L.w_out), _bound(yh, L.w_out), True)
    # end to end from the hidden states: the stage errors above, carried
    # through; a sanity check of the composition, not a parity bound
    r = lref.delta_layer_forward(L.hidden, L.w_in, L.conv_w, L.A_log, L.dt_bias, L.norm_w, L.w_out, L.cu_seqlens,
                                 hk, hv, conv_state=cs0, initial_state=st0)
    e2e = rel_err(to_host(out), r["out"])
    say(f"  end-to-end max err / RMS = {e2e:.3e}")
    assert e2e <= 5e-2


def test_layer_full_size_sampled():
    """The layer at the benchmark's size: one 32768-token sequence, hidden
    5120, 16/48 heads.  Equal bit for bit to its five steps; the projections
    checked on sampled rows, the front on sampled channels (bit-exact), the
    recurrence on two value heads over the first 2048 tokens, the norm and
    the output projection on sampled rows, each against the oracle fed that
    step's GPU inputs."""
    import torch
    dev = gpu()
    T, hk, hv, d = 32768, 16, 48, 128
    L = synth.layer_inputs(6, lengths=(T,))
    C, V = (2 * hk + hv) * d, hv * d
    say("delta layer full size T=32768 hidden=5120")
    w, out, fin, cso = _layer_gpu(L, dev)
    torch.cuda.synchronize()
    s = _stages(L, w, dev)
    assert bits_equal(out, s["out"]) and bits_equal(fin, s["final_state"])
    rng = synth.rng(77)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, T - 1], rng.choice(T, 27, replace=False)]))
    rd = torch.as_tensor(rows, device=dev)
    # in-projection on sampled rows, every column
    proj = np.concatenate([to_host(s[n][rd]) for n in ("qkv", "z", "b", "a")], 1)
    _check(proj, lref.linear(L.hidden[rows], L.w_in), _bound(L.hidden[rows], L.w_in), True)
    # front on sampled channels, every token
    cols = np.unique(np.concatenate([np.arange(0, 16), np.arange(2040, 2056), np.arange(C - 16, C),
                                     rng.choice(C, 48, replace=False)]))
    qkv_c = to_host(s["qkv"][:, torch.as_tensor(cols, device=dev)]).astype(np.float32)
    gq = torch.cat([s[n].reshape(T, -1) for n in ("q", "k", "v")], 1)[:, torch.as_tensor(cols, device=dev)]
    assert np.array_equal(to_host(gq), cref.conv_silu_fp32(qkv_c, L.conv_w[cols], L.cu_seqlens))
    # recurrence: two value heads, first 2048 tokens
    heads = [0, 47]
    qh, kh, vh, gh, bh = (to_host(s[n]).astype(np.float32) for n in ("q", "k", "v", "g", "beta"))
    o_ref, _ = gref.forward(qh, kh, vh, gh, bh, None, L.cu_seqlens, heads=heads, token_limit=2048)
    og = to_host(s["o"])
    assert rel_err(og[:, :2048][:, :, heads], o_ref[:, :2048][:, :, heads]) <= BF16_TOL
    # norm and out-projection on sampled rows
    y_ref = cref.gated_rmsnorm(og[0][rows], to_host(s["z"][rd]).reshape(len(rows), hv, d), L.norm_w)
    assert np.all(np.abs(to_host(s["y"][rd]) - y_ref.reshape(len(rows), V)) <= bf16_ulp(y_ref.reshape(len(rows), V)) + 1e-30)
    yh = to_host(s["y"][rd]).astype(np.float32)
    _check(to_host(out[rd]), lref.linear(yh, L.w_out), _bound(yh, L.w_out), True)
