"""GPU parity of gdr_recurrent_step (one-token decode) against the fp64 oracle."""
import numpy as np
import pytest

from inputs import synth
from oracle import gdr as ref
from helpers import BF16_TOL, F32_TOL, bits_equal, gpu, rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run_steps(N, hk, hv, d, dtype, steps, seqs_checked=None, out_dtype="f32", elementwise=False):
    """Run ``steps`` in-place decode steps on the GPU beside the oracle.

    Returns the worst output error, the final state error (both max|gpu-ref|/RMS),
    and, if ``elementwise``, the worst ratio |gpu-ref| / (bf16 ulp(ref) + tol*RMS).
    """
    import gated_delta_rule_amd as gdr_amd
    import torch
    from helpers import bf16_ulp
    dev = gpu()
    A_log, dt, s0 = synth.decode_inputs(N=N, hk=hk, hv=hv, d=d)
    state = to_dev(s0, "f32", dev)
    sel = np.arange(N) if seqs_checked is None else np.asarray(seqs_checked)
    S_ref = s0[sel].astype(np.float64)
    worst_o, worst_ratio = 0.0, 0.0
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    for step in range(steps):
        x = synth.decode_step_inputs(step, N=N, hk=hk, hv=hv, d=d, dtype=dtype)
        o = gdr_amd.recurrent_step(to_dev(x.q, dtype, dev), to_dev(x.k, dtype, dev), to_dev(x.v, dtype, dev),
                                   to_dev(x.g, "f32", dev), to_dev(x.beta, "f32", dev), state, out_dtype=odt)
        o_ref, S_ref = ref.decode_step(x.q[sel], x.k[sel], x.v[sel], x.g[sel], x.beta[sel], S_ref)
        og = to_host(o)[sel]
        worst_o = max(worst_o, rel_err(og, o_ref))
        if elementwise:
            bound = bf16_ulp(o_ref) + BF16_TOL * np.sqrt(np.mean(o_ref ** 2))
            worst_ratio = max(worst_ratio, float(np.max(np.abs(og - o_ref) / bound)))
    torch.cuda.synchronize()
    es = rel_err(to_host(state)[sel], S_ref)
    return (worst_o, es, worst_ratio) if elementwise else (worst_o, es)


def test_decode_layer_shape_8_steps():
    say("decode N=64 Hk=16 Hv=48 d=128 bf16, 8 steps")
    eo, es = _run_steps(64, 16, 48, 128, "bf16", 8)
    say(f"  o err {eo:.2e}  state err {es:.2e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


def test_decode_layer_shape_256_steps_sampled():
    """All 64 sequences run 256 in-place steps on the GPU; the oracle follows two of them."""
    say("decode N=64 bf16, 256 steps, oracle on sequences 5 and 62")
    eo, es = _run_steps(64, 16, 48, 128, "bf16", 256, seqs_checked=[5, 62])
    say(f"  o err {eo:.2e}  state err {es:.2e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


@pytest.mark.parametrize("d", [32, 64, 128])
def test_decode_fp32(d):
    say(f"decode fp32 N=5 Hk=2 Hv=6 d={d}")
    eo, es = _run_steps(5, 2, 6, d, "f32", 6)
    say(f"  o err {eo:.2e}  state err {es:.2e}")
    assert eo <= F32_TOL and es <= F32_TOL


def test_decode_bf16_output():
    """bf16 storage of o: each output within one bf16 ulp of the oracle, plus the
    fp32-path tolerance; the state (always fp32) within the usual tolerance."""
    say("decode bf16 out N=8")
    eo, es, ratio = _run_steps(8, 16, 48, 128, "bf16", 3, out_dtype="bf16", elementwise=True)
    say(f"  worst |o - ref| / (ulp + tol*rms) = {ratio:.3f}, state err {es:.2e}")
    assert ratio <= 1.0 and es <= BF16_TOL


def test_decode_matches_one_token_prefill():
    """Cross-kernel layout check: decode step = chunked prefill with T = 1."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    say("decode vs chunk_fwd T=1, N=4")
    A_log, dt, s0 = synth.decode_inputs(N=4)
    x = synth.decode_step_inputs(0, N=4)
    st1 = to_dev(s0, "f32", dev)
    o1 = gdr_amd.recurrent_step(to_dev(x.q, "bf16", dev), to_dev(x.k, "bf16", dev), to_dev(x.v, "bf16", dev),
                                to_dev(x.g, "f32", dev), to_dev(x.beta, "f32", dev), st1)
    o2, st2 = gdr_amd.chunk_gated_delta_rule(
        to_dev(x.q[:, None], "bf16", dev), to_dev(x.k[:, None], "bf16", dev), to_dev(x.v[:, None], "bf16", dev),
        to_dev(x.g[:, None], "f32", dev), to_dev(x.beta[:, None], "f32", dev), to_dev(s0, "f32", dev),
        output_final_state=True)
    torch.cuda.synchronize()
    assert rel_err(to_host(o2)[:, 0], to_host(o1)) <= BF16_TOL
    assert rel_err(to_host(st2), to_host(st1)) <= BF16_TOL


def test_decode_deterministic_and_empty_batch():
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    say("decode determinism N=16")
    A_log, dt, s0 = synth.decode_inputs(N=16)
    x = synth.decode_step_inputs(1, N=16)
    args = [to_dev(x.q, "bf16", dev), to_dev(x.k, "bf16", dev), to_dev(x.v, "bf16", dev),
            to_dev(x.g, "f32", dev), to_dev(x.beta, "f32", dev)]
    sa, sb = to_dev(s0, "f32", dev), to_dev(s0, "f32", dev)
    oa = gdr_amd.recurrent_step(*args, sa)
    ob = gdr_amd.recurrent_step(*args, sb)
    torch.cuda.synchronize()
    assert bits_equal(oa, ob) and bits_equal(sa, sb)
    e = torch.empty((0, 16, 128), device=dev, dtype=torch.bfloat16)
    ev = torch.empty((0, 48, 128), device=dev, dtype=torch.bfloat16)
    ef = torch.empty((0, 48), device=dev)
    es = torch.empty((0, 48, 128, 128), device=dev)
    assert gdr_amd.recurrent_step(e, e, ev, ef, ef, es).shape == (0, 48, 128)


def test_decode_reset_and_no_write():
    """g = -inf resets the state to beta v k^T; beta = 0 with g = 0 keeps it bit for bit."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    say("decode degenerate gates N=4")
    A_log, dt, s0 = synth.decode_inputs(N=4)
    x = synth.decode_step_inputs(2, N=4)
    g = x.g.copy()
    g[0] = -np.inf
    g[1] = 0.0
    beta = x.beta.copy()
    beta[1] = 0.0
    state = to_dev(s0, "f32", dev)
    o = gdr_amd.recurrent_step(to_dev(x.q, "bf16", dev), to_dev(x.k, "bf16", dev), to_dev(x.v, "bf16", dev),
                               to_dev(g, "f32", dev), to_dev(beta, "f32", dev), state)
    torch.cuda.synchronize()
    o_ref, s_ref = ref.decode_step(x.q, x.k, x.v, g, beta, s0.astype(np.float64))
    assert rel_err(to_host(o), o_ref) <= BF16_TOL and rel_err(to_host(state), s_ref) <= BF16_TOL
    assert np.array_equal(to_host(state)[1], s0[1])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("f32", 32)])
def test_decode_pool_indexed(dtype, d):
    """gdr_recurrent_step_indexed on a pool of 40 slots: 16 rows naming distinct
    slots in shuffled order, plus padding rows (index -1 and >= pool size) over
    3 steps; o and the whole pool against the oracle, unnamed slots bit for bit."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    N, P, hk, hv = 20, 40, (16 if d == 128 else 2), (48 if d == 128 else 6)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    rng = np.random.default_rng(70 + d)
    idx = np.concatenate([rng.choice(P, 16, replace=False), [-1, P, P + 7, -5]]).astype(np.int32)
    rng.shuffle(idx)
    pool0 = (0.05 * rng.standard_normal((P, hv, d, d))).astype(np.float32)
    pool = to_dev(pool0, "f32", dev)
    ref_pool = pool0.astype(np.float64)
    di = torch.as_tensor(idx, device=dev)
    say(f"decode pool-indexed {dtype} d={d}: {N} rows, pool {P}")
    for step in range(3):
        x = synth.decode_step_inputs(step, N=N, hk=hk, hv=hv, d=d, dtype=dtype)
        o = gdr_amd.recurrent_step(to_dev(x.q, dtype, dev), to_dev(x.k, dtype, dev), to_dev(x.v, dtype, dev),
                                   to_dev(x.g, "f32", dev), to_dev(x.beta, "f32", dev), pool, state_indices=di)
        o_ref, ref_pool = ref.decode_step_pool(x.q, x.k, x.v, x.g, x.beta, ref_pool, idx)
        og = to_host(o)
        pad = (idx < 0) | (idx >= P)
        assert np.all(og[pad] == 0)
        assert rel_err(og[~pad], o_ref[~pad]) <= tol
    torch.cuda.synchronize()
    gp = to_host(pool)
    live = sorted(int(i) for i in idx if 0 <= i < P)
    dead = [p for p in range(P) if p not in set(live)]
    assert np.array_equal(gp[dead], pool0[dead])
    assert rel_err(gp[live], ref_pool[live]) <= tol


def test_decode_pool_identity_equals_plain_bit_exact():
    """Indices 0..N-1 over a pool of N slots give the plain call's bits."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    N = 8
    A_log, dt, s0 = synth.decode_inputs(N=N)
    x = synth.decode_step_inputs(0, N=N)
    args = [to_dev(a, t, dev) for a, t in ((x.q, "bf16"), (x.k, "bf16"), (x.v, "bf16"), (x.g, "f32"),
                                          (x.beta, "f32"))]
    s1, s2 = to_dev(s0, "f32", dev), to_dev(s0, "f32", dev)
    say("decode pool identity vs plain")
    o1 = gdr_amd.recurrent_step(*args, s1)
    o2 = gdr_amd.recurrent_step(*args, s2, state_indices=torch.arange(N, device=dev, dtype=torch.int32))
    torch.cuda.synchronize()
    assert bits_equal(o1, o2) and bits_equal(s1, s2)
