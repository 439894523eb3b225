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

from inputs import synth
from oracle import attention as aref
from helpers import bf16_ulp, bits_equal, gpu, say, to_dev, to_host, v_cache_blocked, v_cache_natural

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
    L = (L + 63) // 64 * 64
    kc = torch.zeros((N, L, hk, 256), device=dev, dtype=torch.bfloat16)
    vc = torch.zeros((N, hk, L // 32, 256, 32), device=dev, dtype=torch.bfloat16)
    out = gdr.attn_prefill(q, k, v, g, qw, kw, cu, k_cache=kc, v_cache=vc)
    qo, ko = gdr.attn_qk_norm_rope(q, k, qw, kw, cu)
    torch.cuda.synchronize()
    r = aref.core_prefill(to_host(qo), to_host(ko), x.v, x.gate, x.cu_seqlens)
    _check_out(to_host(out), r["out"], r["mass"])
    vn = v_cache_natural(vc)
    for n in range(N):
        a, b = x.cu_seqlens[n], x.cu_seqlens[n + 1]
        assert bits_equal(kc[n, :b - a], ko[a:b])
        assert bits_equal(vn[n, :b - a], v[a:b])
        assert not torch.any(kc[n, b - a:].float() != 0) and not torch.any(vn[n, b - a:].float() != 0)


def test_prefill_sequence_longer_than_cache():
    """A 200-token and a 70-token sequence into 128-slot caches: positions
    below 128 receive k' and v (the blocked V cache through its converter),
    the 70-token sequence leaves its tail slots untouched, and the output
    does not depend on the cache."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    lengths, L, hk = (200, 70), 128, 2
    x = synth.attn_inputs(57, lengths=lengths, hq=6, hk=hk)
    say(f"attention prefill lengths {lengths} into {L}-slot caches")
    q, k, v, g, qw, kw, cu = _dev(x, dev)
    kc = torch.full((2, L, hk, 256), 7.0, device=dev, dtype=torch.bfloat16)
    vc = torch.full((2, hk, L // 32, 256, 32), 7.0, device=dev, dtype=torch.bfloat16)
    out = gdr.attn_prefill(q, k, v, g, qw, kw, cu, k_cache=kc, v_cache=vc)
    ref_out = gdr.attn_prefill(q, k, v, g, qw, kw, cu)
    _, ko = gdr.attn_qk_norm_rope(q, k, qw, kw, cu)
    torch.cuda.synchronize()
    assert bits_equal(out, ref_out)
    vn = v_cache_natural(vc)
    assert bits_equal(kc[0], ko[:L]) and bits_equal(vn[0], v[:L])
    assert bits_equal(kc[1, :70], ko[200:270]) and bits_equal(vn[1, :70], v[200:270])
    assert torch.all(kc[1, 70:].float() == 7.0) and torch.all(vn[1, 70:].float() == 7.0)


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


def _gpu_qrot_at(q_row, k_row, qw, kw, pos, dev):
    """The library's q' and k' of one token at position pos: the same kernel
    run on a sequence whose last token is that one."""
    import gated_delta_rule_amd as gdr
    import torch
    Hq, D = q_row.shape
    Hk = k_row.shape[0]
    qf = torch.zeros((pos + 1, Hq, D), device=dev, dtype=torch.bfloat16)
    kf = torch.zeros((pos + 1, Hk, D), device=dev, dtype=torch.bfloat16)
    qf[pos], kf[pos] = q_row, k_row
    cu = torch.tensor([0, pos + 1], device=dev, dtype=torch.int32)
    qo, ko = gdr.attn_qk_norm_rope(qf, kf, qw, kw, cu)
    return qo[pos], ko[pos]


@pytest.mark.parametrize("lens,L,hq,hk", [((0, 1, 255, 256, 1000), 1024, 24, 4), ((63, 64, 65), 128, 8, 2)])
def test_decode_against_oracle(lens, L, hq, hk):
    """One token per sequence against caches of different fill (empty, one
    split, exactly a split, several): the token's k' and v land at its
    position, nothing else in the caches moves, and the output is within
    its bound of the oracle run on the GPU's q' and caches."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    N = len(lens)
    x = synth.attn_inputs(46, lengths=(1,) * N, hq=hq, hk=hk)
    rng = synth.rng(47)
    kc0 = synth.round_bf16(rng.standard_normal((N, L, hk, 256)))
    vc0 = synth.round_bf16(rng.standard_normal((N, L, hk, 256)))  # natural order
    say(f"attention decode lens {lens} L={L} Hq={hq} Hk={hk}")
    q, k, v, g, qw, kw, _ = _dev(x, dev)
    kc, vc = to_dev(kc0, "bf16", dev), to_dev(v_cache_blocked(vc0), "bf16", dev)
    cl = torch.tensor(lens, device=dev, dtype=torch.int32)
    out = gdr.attn_decode(q, k, v, g, qw, kw, kc, vc, cl)
    torch.cuda.synchronize()
    kch, vch = to_host(kc), v_cache_natural(to_host(vc))
    qrot = np.zeros((N, hq, 256))
    for n, p in enumerate(lens):
        qg, kg = _gpu_qrot_at(q[n], k[n], qw, kw, p, dev)
        qrot[n] = to_host(qg)
        assert bits_equal(kc[n, p], kg)
        assert np.array_equal(vch[n, p], to_host(v[n]))
        keep = np.ones(L, bool)
        keep[p] = False
        assert np.array_equal(kch[n, keep], kc0[n, keep]) and np.array_equal(vch[n, keep], vc0[n, keep])
    r = aref.core_decode(qrot, x.gate, kch, vch, np.asarray(lens) + 1)
    _check_out(to_host(out), r["out"], r["mass"])


def test_decode_continues_prefill():
    """Prefill 700 tokens into the caches, then decode tokens 700 and 701:
    each output matches the oracle on the full causal prefix."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    T, L = 702, 768
    x = synth.attn_inputs(48, lengths=(T,))
    q, k, v, g, qw, kw, _ = _dev(x, dev)
    say("attention prefill 700 then decode 2")
    kc = torch.zeros((1, L, 4, 256), device=dev, dtype=torch.bfloat16)
    vc = torch.zeros((1, 4, L // 32, 256, 32), device=dev, dtype=torch.bfloat16)
    cu = torch.tensor([0, 700], device=dev, dtype=torch.int32)
    gdr.attn_prefill(q[:700], k[:700], v[:700], g[:700], qw, kw, cu, k_cache=kc, v_cache=vc)
    outs = []
    for t in (700, 701):
        cl = torch.tensor([t], device=dev, dtype=torch.int32)
        outs.append(gdr.attn_decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], qw, kw, kc, vc, cl))
    torch.cuda.synchronize()
    qo, ko = gdr.attn_qk_norm_rope(q, k, qw, kw, torch.tensor([0, T], device=dev, dtype=torch.int32))
    assert bits_equal(kc[0, :T], ko)
    r = aref.core_prefill(to_host(qo), to_host(ko), x.v, x.gate, x.cu_seqlens, rows=[700, 701])
    for i, t in enumerate((700, 701)):
        _check_out(to_host(outs[i])[0], r["out"][t], r["mass"][t])


def test_decode_full_size_sampled():
    """64 sequences with 32768-slot caches filled to 32000 .. 32767 tokens (the
    serving shape of the layer): 3 sequences checked on every head."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    N, L = 64, 32768
    say("attention decode full size N=64 L=32768")
    gen = torch.Generator(device=dev).manual_seed(49)
    kc = torch.randn((N, L, 4, 256), device=dev, generator=gen).to(torch.bfloat16)
    vc = torch.randn((N, 4, L // 32, 256, 32), device=dev, generator=gen).to(torch.bfloat16)
    x = synth.attn_inputs(50, lengths=(1,) * N)
    q, k, v, g, qw, kw, _ = _dev(x, dev)
    lens = np.asarray(synth.rng(51).integers(32000, L, size=N), dtype=np.int32)
    cl = torch.as_tensor(lens, device=dev)
    out = gdr.attn_decode(q, k, v, g, qw, kw, kc, vc, cl)
    torch.cuda.synchronize()
    for n in (0, 31, 63):
        p = int(lens[n])
        qg, _ = _gpu_qrot_at(q[n], k[n], qw, kw, p, dev)
        kn = to_host(kc[n:n + 1, :p + 1])
        vn = v_cache_natural(to_host(vc[n:n + 1]))[:, :p + 1]
        r = aref.core_decode(to_host(qg)[None], x.gate[n:n + 1], kn, vn, np.array([p + 1]))
        _check_out(to_host(out[n:n + 1]), r["out"], r["mass"])


def test_prefill_many_short_sequences():
    """300 sequences of 0 .. 70 tokens (more sequences than the offset
    table's threads, many of them empty or single-token)."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    lens = [int(x) for x in synth.rng(53).integers(0, 71, size=300)]
    lens[7] = 0
    lens[8] = 1
    x = synth.attn_inputs(54, lengths=lens, hq=8, hk=2)
    say("attention prefill 300 short sequences")
    q, k, v, g, qw, kw, cu = _dev(x, dev)
    out = gdr.attn_prefill(q, k, v, g, qw, kw, cu)
    qo, ko = gdr.attn_qk_norm_rope(q, k, qw, kw, cu)
    torch.cuda.synchronize()
    r = aref.core_prefill(to_host(qo), to_host(ko), x.v, x.gate, x.cu_seqlens)
    _check_out(to_host(out), r["out"], r["mass"])


def test_decode_full_cache():
    """A token at the cache's last slot attends to every cached position;
    one at slot 0 to itself only."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    N, L, hq, hk = 2, 320, 24, 4
    lens = (L - 1, 0)
    x = synth.attn_inputs(55, lengths=(1,) * N, hq=hq, hk=hk)
    rng = synth.rng(56)
    kc0 = synth.round_bf16(rng.standard_normal((N, L, hk, 256)))
    vc0 = synth.round_bf16(rng.standard_normal((N, L, hk, 256)))  # natural order
    say("attention decode at the last cache slot")
    q, k, v, g, qw, kw, _ = _dev(x, dev)
    kc, vc = to_dev(kc0, "bf16", dev), to_dev(v_cache_blocked(vc0), "bf16", dev)
    out = gdr.attn_decode(q, k, v, g, qw, kw, kc, vc, torch.tensor(lens, device=dev, dtype=torch.int32))
    torch.cuda.synchronize()
    qrot = np.stack([to_host(_gpu_qrot_at(q[n], k[n], qw, kw, p, dev)[0]) for n, p in enumerate(lens)])
    r = aref.core_decode(qrot, x.gate, to_host(kc), v_cache_natural(to_host(vc)), np.asarray(lens) + 1)
    _check_out(to_host(out), r["out"], r["mass"])


def test_decode_padding_rows():
    """A decode row whose cache_lens entry lies outside [0, cache_len) is a
    padding row: zero output, neither cache written, and the other rows equal
    the same call without the padding rows, bit for bit."""
    import gated_delta_rule_amd as gdr
    import torch
    dev = gpu()
    L, lens = 128, [5, -1, 127, 128, 70, 1 << 20]
    live = [i for i, p in enumerate(lens) if 0 <= p < L]
    N = len(lens)
    x = synth.attn_inputs(52, lengths=(1,) * N)
    rng = synth.rng(53)
    kc0 = synth.round_bf16(rng.standard_normal((N, L, 4, 256)))
    vc0 = synth.round_bf16(rng.standard_normal((N, L, 4, 256)))
    say(f"attention decode padding rows lens {lens}")
    q, k, v, g, qw, kw, _ = _dev(x, dev)
    kc, vc = to_dev(kc0, "bf16", dev), to_dev(v_cache_blocked(vc0), "bf16", dev)
    out = gdr.attn_decode(q, k, v, g, qw, kw, kc, vc, torch.tensor(lens, device=dev, dtype=torch.int32))
    # the same live rows alone
    sel = torch.tensor(live, device=dev)
    kc2, vc2 = to_dev(kc0[live], "bf16", dev), to_dev(v_cache_blocked(vc0[live]), "bf16", dev)
    out2 = gdr.attn_decode(q[sel].contiguous(), k[sel].contiguous(), v[sel].contiguous(), g[sel].contiguous(), qw,
                           kw, kc2, vc2, torch.tensor([lens[i] for i in live], device=dev, dtype=torch.int32))
    torch.cuda.synchronize()
    assert bits_equal(out[sel].contiguous(), out2)
    assert bits_equal(kc[sel].contiguous(), kc2) and bits_equal(vc[sel].contiguous(), vc2)
    for i in range(N):
        if i in live:
            continue
        assert not torch.any(out[i].float() != 0), f"padding row {i} has output"
        assert np.array_equal(to_host(kc[i]), kc0[i]), f"padding row {i} wrote the k cache"
        assert np.array_equal(v_cache_natural(to_host(vc[i:i + 1]))[0], vc0[i]), f"padding row {i} wrote the v cache"
