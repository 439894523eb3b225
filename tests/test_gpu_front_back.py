"""GPU parity of the layer front (conv + SiLU + gates) and back (gated RMSNorm),
and the whole delta-layer path checked stage by stage."""
import numpy as np
import pytest

from inputs import synth
from oracle import conv as cref
from oracle import gdr as ref
from helpers import BF16_TOL, bf16_ulp, gpu, rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _front(p, dev, state_in=None, output_state=False):
    import gated_delta_rule_amd as gdr_amd
    import torch
    out = gdr_amd.conv_gate_fused(to_dev(p.x, "bf16", dev), to_dev(p.conv_w, "bf16", dev),
                                  to_dev(p.cu_seqlens, "i32", dev), to_dev(p.a, "f32", dev),
                                  to_dev(p.b, "f32", dev), to_dev(p.A_log, "f32", dev),
                                  to_dev(p.dt_bias, "f32", dev), p.hk, p.hv, p.d,
                                  conv_state_in=state_in, output_conv_state=output_state)
    torch.cuda.synchronize()
    return out


def _y_of(q, k, v):
    import torch
    T = q.shape[1]
    return torch.cat([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], 1)


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy()


def _bits_np(a):
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16).view(np.int16)


@pytest.mark.parametrize("lens", [[5, 1, 0, 37, 2, 100], [300]])
def test_conv_bit_exact_small(lens):
    dev = gpu()
    p = synth.pipeline_inputs(seed=7, lengths=lens, hk=2, hv=6, d=32)
    say(f"conv small {lens}")
    q, k, v, g, beta, st = _front(p, dev, output_state=True)
    y = _y_of(q, k, v)
    y_ref = cref.conv_silu_fp32(p.x, p.conv_w, p.cu_seqlens)
    assert np.array_equal(_bits(y), _bits_np(y_ref))
    assert np.array_equal(_bits(st), _bits_np(cref.conv_state_out(p.x, p.cu_seqlens)))
    g_ref, b_ref = cref.gates(p.a, p.b, p.A_log, p.dt_bias)
    assert np.max(np.abs(to_host(g)[0] - g_ref) / np.abs(g_ref)) < 2e-6
    assert np.max(np.abs(to_host(beta)[0] - b_ref) / b_ref) < 2e-6


def test_conv_every_bf16_input_bit_exact():
    """SiLU's general and |acc| <= 80 paths and the special values: 64 channels
    each run through all 65536 bf16 bit patterns (infinities, NaN, subnormals,
    the overflow range) in their own order, 64 more with pre-activations spread
    across +-80; bit for bit, NaN matched by position."""
    dev = gpu()
    T, C = 65536, 128
    p = synth.pipeline_inputs(seed=30, lengths=[T // 2, T // 2], hk=1, hv=2, d=32)
    rng = np.random.default_rng(31)
    pats = np.arange(65536, dtype=np.uint32) << 16
    x = np.empty((T, C), np.float32)
    for c in range(64):
        x[:, c] = rng.permutation(pats).view(np.float32)
    x[:, 64:] = synth.round_bf16(60.0 * rng.standard_normal((T, 64)))
    p = synth.PipelineInputs(x, p.conv_w, p.a, p.b, p.A_log, p.dt_bias, p.z, p.norm_w, p.cu_seqlens,
                             p.hk, p.hv, p.d)
    say("conv SiLU sweep: all bf16 inputs")
    y = _y_of(*_front(p, dev)[:3])
    with np.errstate(over="ignore", invalid="ignore"):
        y_ref = cref.conv_silu_fp32(p.x, p.conv_w, p.cu_seqlens)
    got = to_host(y.float())
    nan = np.isnan(y_ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(_bits(y)[~nan], _bits_np(y_ref)[~nan])


def test_conv_state_carry_bit_exact():
    """Conv over a sequence in pieces, carrying conv_state, equals one pass."""
    dev = gpu()
    p = synth.pipeline_inputs(seed=8, lengths=[40], hk=2, hv=6, d=32)
    say("conv state carry")
    y_full = _y_of(*_front(p, dev)[:3])
    st = None
    parts = []
    for a, b in ((0, 2), (2, 3), (3, 19), (19, 40)):
        pi = synth.PipelineInputs(p.x[a:b], p.conv_w, p.a[a:b], p.b[a:b], p.A_log, p.dt_bias, p.z[a:b],
                                  p.norm_w, synth.cu_seqlens_of([b - a]), p.hk, p.hv, p.d)
        q, k, v, _, _, st = _front(pi, dev, state_in=st, output_state=True)
        parts.append(_y_of(q, k, v))
    import torch
    assert np.array_equal(_bits(torch.cat(parts, 0)), _bits(y_full))


def test_conv_full_size_sampled_channels():
    """65536 packed tokens x 10240 channels on the GPU; every token of 320 sampled
    channels (spread over q, k and v blocks) checked bit for bit."""
    dev = gpu()
    p = synth.pipeline_inputs()
    say("conv full size (65536 x 10240)")
    q, k, v, g, beta, st = _front(p, dev, output_state=True)
    y = _y_of(q, k, v)
    rng = np.random.default_rng(9)
    cols = np.unique(np.concatenate([np.arange(0, 64), np.arange(2040, 2112), np.arange(10176, 10240),
                                     rng.choice(10240, 120, replace=False)]))
    import torch
    tc = torch.as_tensor(cols, device=dev)
    y_ref = cref.conv_silu_fp32(p.x[:, cols], p.conv_w[cols], p.cu_seqlens)
    assert np.array_equal(_bits(y[:, tc]), _bits_np(y_ref))
    st_ref = cref.conv_state_out(p.x[:, cols], p.cu_seqlens)
    assert np.array_equal(_bits(st[:, tc]), _bits_np(st_ref))
    g_ref, b_ref = cref.gates(p.a, p.b, p.A_log, p.dt_bias)
    assert np.max(np.abs(to_host(g)[0] - g_ref) / np.abs(g_ref)) < 2e-6
    assert np.max(np.abs(to_host(beta)[0] - b_ref) / b_ref) < 2e-6


@pytest.mark.parametrize("d,odt", [(128, "f32"), (128, "bf16"), (32, "f32"), (64, "f32")])
def test_gated_rmsnorm_within_one_ulp(d, odt):
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    rng = np.random.default_rng(10 + d)
    T, H = 777, 6
    o = (rng.standard_normal((T, H, d)) * rng.uniform(0.01, 3.0, (T, H, 1))).astype(np.float32)
    if odt == "bf16":
        o = synth.round_bf16(o)
    z = synth.round_bf16(rng.standard_normal((T, H * d)))
    w = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    say(f"gated rmsnorm d={d} o={odt}")
    y = gdr_amd.gated_rmsnorm(to_dev(o, odt, dev), to_dev(z, "bf16", dev), to_dev(w, "f32", dev))
    torch.cuda.synchronize()
    y_ref = cref.gated_rmsnorm(o, z.reshape(T, H, d), w).reshape(T, H * d)
    assert np.all(np.abs(to_host(y) - y_ref) <= bf16_ulp(y_ref) + 1e-30)


def test_full_layer_pipeline_stagewise():
    """Packed varlen batch (8 sequences, 65536 tokens): conv front -> chunked
    recurrence (L2 norm in kernel) -> gated RMSNorm, each stage checked against
    the oracle fed with that stage's GPU inputs."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    p = synth.pipeline_inputs()
    cu = to_dev(p.cu_seqlens, "i32", dev)
    say("pipeline: front")
    q, k, v, g, beta, _ = _front(p, dev)
    say("pipeline: recurrence")
    o, s = gdr_amd.chunk_gated_delta_rule(q, k, v, g, beta, None, output_final_state=True, cu_seqlens=cu)
    say("pipeline: norm")
    y = gdr_amd.gated_rmsnorm(o, to_dev(p.z, "bf16", dev), to_dev(p.norm_w, "f32", dev))
    torch.cuda.synchronize()
    heads = [0, 7, 17, 30, 41, 47]
    qh, kh, vh, gh, bh = (to_host(t).astype(np.float32) for t in (q, k, v, g, beta))
    o_ref, s_ref = ref.forward(qh, kh, vh, gh, bh, None, p.cu_seqlens, heads=heads)
    og, sg = to_host(o), to_host(s)
    eo = rel_err(og[:, :, heads], o_ref[:, :, heads])
    es = rel_err(sg[:, heads], s_ref[:, heads])
    say(f"  recurrence o err {eo:.2e}, state err {es:.2e}")
    assert eo <= BF16_TOL and es <= BF16_TOL
    T = og.shape[1]
    y_ref = cref.gated_rmsnorm(og[0], p.z.reshape(T, 48, 128), p.norm_w).reshape(T, -1)
    assert np.all(np.abs(to_host(y) - y_ref) <= bf16_ulp(y_ref) + 1e-30)
