"""GPU parity of gdr_decode_layer_step (one decode token of the whole layer
path in one launch) against the fp64 oracle, and against the unfused kernels."""
import numpy as np
import pytest

from inputs import synth
from oracle import conv as cref
from oracle import gdr as ref
from helpers import BF16_TOL, bf16_ulp, bits_equal, gpu, rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _inputs(seed, N, hk, hv, P):
    p = synth.pipeline_inputs(seed=seed, lengths=[1] * N, hk=hk, hv=hv, d=128)
    rng = np.random.default_rng(seed + 1)
    C = (2 * hk + hv) * 128
    conv_pool = synth.round_bf16(rng.standard_normal((P, C, 3)))
    pool = (0.05 * rng.standard_normal((P, hv, 128, 128))).astype(np.float32)
    return p, conv_pool, pool


def _bits16(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy()


def _np_bits16(a):
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16).view(np.int16)


@pytest.mark.parametrize("hk,hv", [(16, 48), (2, 2), (2, 4), (1, 4)])
def test_decode_layer_step_against_oracle(hk, hv):
    """Three steps over shuffled pool slots with padding rows: conv outputs and
    the conv pool bit for bit, o and the state pool within tolerance, y within
    one bf16 ulp of the fp64 norm of the GPU's o."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    N, P = 20, 40
    rng = np.random.default_rng(80 + hv)
    idx = np.concatenate([rng.choice(P, 16, replace=False), [-1, P, P + 3, -9]]).astype(np.int32)
    rng.shuffle(idx)
    say(f"decode layer step hk={hk} hv={hv}: {N} rows, pools of {P}")
    p, conv_pool, pool = _inputs(90 + hv, N, hk, hv, P)
    dcp, dpool = to_dev(conv_pool, "bf16", dev), to_dev(pool, "f32", dev)
    rcp, rpool = conv_pool.copy(), pool.astype(np.float64)
    di = torch.as_tensor(idx, device=dev)
    live = (idx >= 0) & (idx < P)
    for step in range(3):
        q = synth.pipeline_inputs(seed=100 + step, lengths=[1] * N, hk=hk, hv=hv, d=128)
        y, o, qkv = gdr_amd.decode_layer_step(
            to_dev(q.x, "bf16", dev), to_dev(p.conv_w, "bf16", dev), dcp, to_dev(q.a, "f32", dev),
            to_dev(q.b, "f32", dev), to_dev(p.A_log, "f32", dev), to_dev(p.dt_bias, "f32", dev), dpool,
            to_dev(q.z, "bf16", dev), to_dev(p.norm_w, "f32", dev), hk, hv, state_indices=di,
            return_intermediates=True)
        y_ref, o_ref, qkv_ref, rcp, rpool = ref.decode_layer_step(
            q.x, p.conv_w, rcp, q.a, q.b, p.A_log, p.dt_bias, rpool, q.z, p.norm_w, hk, hv, state_indices=idx)
        torch.cuda.synchronize()
        assert np.array_equal(_bits16(qkv)[live], _np_bits16(qkv_ref)[live])
        og = to_host(o)
        assert np.all(og[~live] == 0) and np.all(to_host(y)[~live] == 0) and np.all(to_host(qkv)[~live] == 0)
        eo = rel_err(og[live], o_ref[live])
        assert eo <= BF16_TOL, eo
        y_stage = cref.gated_rmsnorm(og[live], q.z.reshape(N, hv, 128)[live], p.norm_w).reshape(-1, hv * 128)
        assert np.all(np.abs(to_host(y)[live] - y_stage) <= bf16_ulp(y_stage) + 1e-30)
    assert np.array_equal(_bits16(dcp), _np_bits16(rcp))
    slots = sorted(int(i) for i in idx[live])
    gp = to_host(dpool)
    others = [s for s in range(P) if s not in set(slots)]
    assert np.array_equal(gp[others], pool[others])
    assert rel_err(gp[slots], rpool[slots]) <= BF16_TOL


def test_decode_layer_step_equals_unfused_kernels():
    """The fused step against gdr_conv_gate_fused (one-token sequences, conv
    state in/out) + gdr_recurrent_step + gdr_gated_rmsnorm on the same inputs:
    conv outputs, conv state, o and the recurrent state bit for bit; y within
    one bf16 ulp of the norm kernel's."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    N, hk, hv = 16, 16, 48
    say("decode layer step: fused vs three kernels")
    p, conv_pool, pool = _inputs(120, N, hk, hv, N)
    x, cw = to_dev(p.x, "bf16", dev), to_dev(p.conv_w, "bf16", dev)
    a, b, A, dt = (to_dev(t, "f32", dev) for t in (p.a, p.b, p.A_log, p.dt_bias))
    z, nw = to_dev(p.z, "bf16", dev), to_dev(p.norm_w, "f32", dev)
    cs1, st1 = to_dev(conv_pool, "bf16", dev), to_dev(pool, "f32", dev)
    y1, o1, qkv1 = gdr_amd.decode_layer_step(x, cw, cs1, a, b, A, dt, st1, z, nw, hk, hv,
                                             return_intermediates=True)
    cu = torch.arange(N + 1, device=dev, dtype=torch.int32)
    cs_in = to_dev(conv_pool, "bf16", dev)
    qq, kk, vv, g, beta, cs2 = gdr_amd.conv_gate_fused(x, cw, cu, a, b, A, dt, hk, hv, 128,
                                                       conv_state_in=cs_in, output_conv_state=True)
    st2 = to_dev(pool, "f32", dev)
    o2 = gdr_amd.recurrent_step(qq[0].contiguous(), kk[0].contiguous(), vv[0].contiguous(), g[0].contiguous(),
                                beta[0].contiguous(), st2)
    y2 = gdr_amd.gated_rmsnorm(o2.reshape(1, N, hv, 128), z.reshape(1, N, hv * 128), nw)
    torch.cuda.synchronize()
    qkv2 = torch.cat([qq[0].reshape(N, -1), kk[0].reshape(N, -1), vv[0].reshape(N, -1)], 1)
    assert bits_equal(qkv1, qkv2)
    assert bits_equal(cs1, cs2)
    assert bits_equal(o1, o2) and bits_equal(st1, st2)
    y1h, y2h = to_host(y1), to_host(y2).reshape(N, -1)
    assert np.all(np.abs(y1h - y2h) <= bf16_ulp(y2h) + 1e-30)
