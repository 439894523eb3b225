"""GPU parity of gdr_chunk_fwd (chunked prefill) against the fp64 oracle."""
import functools

import numpy as np
import pytest

from inputs import synth
from oracle import gdr as ref
from helpers import BF16_TOL, F32_TOL, bits_equal, gpu, rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _long_call(i):
    """Inputs of call i of the 262 144-token sequence (drawing one takes ~20 s)."""
    return synth.long_context_call(i)


def _dev_inputs(x, dev, cu=None, s0=None):
    return dict(q=to_dev(x.q, x.dtype, dev), k=to_dev(x.k, x.dtype, dev), v=to_dev(x.v, x.dtype, dev),
                g=to_dev(x.g, "f32", dev), beta=to_dev(x.beta, "f32", dev),
                initial_state=None if s0 is None else to_dev(s0, "f32", dev),
                cu_seqlens=None if cu is None else to_dev(cu, "i32", dev))


def _gpu_chunk(x, cu=None, s0=None, **kw):
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    a = _dev_inputs(x, dev, cu, s0)
    o, s = gdr_amd.chunk_gated_delta_rule(a["q"], a["k"], a["v"], a["g"], a["beta"], a["initial_state"],
                                          output_final_state=True, cu_seqlens=a["cu_seqlens"],
                                          chunk_size=x.chunk_size, **kw)
    torch.cuda.synchronize()
    return o, s


def _check(x, cu=None, s0=None, tol=BF16_TOL, heads=None, procs=None, **kw):
    o, s = _gpu_chunk(x, cu, s0, **kw)
    o_ref, s_ref, _ = ref.forward_parallel(x.q, x.k, x.v, x.g, x.beta, s0, cu, processes=procs)
    og, sg = to_host(o), to_host(s)
    eo, es = rel_err(og, o_ref), rel_err(sg, s_ref)
    say(f"  o err {eo:.2e}  state err {es:.2e}  (tol {tol:g})")
    assert np.isfinite(og).all() and np.isfinite(sg).all()
    assert eo <= tol and es <= tol
    return o, s


def test_tiny_fp32_config():
    """B=1, T=128, 2/6 heads, d=32, chunk 32, all fp32 (the small oracle config)."""
    say("chunk tiny fp32 d=32 C=32")
    _check(synth.tiny_config(), tol=F32_TOL)


def test_layer_prefill_4096():
    """B=1, T=4096, 16/48 heads, d=128, bf16 q/k/v, chunk 64, zero state."""
    say("chunk layer prefill T=4096 bf16")
    _check(synth.layer_prefill(T=4096))


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_ragged_lengths_with_initial_state(T):
    x = synth.gdr_inputs(10 + T, B=2, T=T, hk=16, hv=48, d=128, dtype="bf16", initial_state_std=0.05)
    say(f"chunk bf16 B=2 T={T} with initial state")
    _check(x, s0=x.initial_state)


def test_varlen_packed_with_empty_and_short_sequences():
    lens = [0, 1, 130, 64, 3, 0, 257, 5]
    cu = synth.cu_seqlens_of(lens)
    x = synth.gdr_inputs(21, B=1, T=int(cu[-1]), dtype="bf16")
    s0 = (0.05 * np.random.default_rng(22).standard_normal((len(lens), 48, 128, 128))).astype(np.float32)
    say(f"chunk varlen {lens}")
    _check(x, cu=cu, s0=s0)


@pytest.mark.parametrize("hk,hv", [(4, 4), (2, 8), (3, 24)])
def test_head_ratios_varlen(hk, hv):
    """Value heads per key head G = 1, 4 and 8: the prepare kernel forms each
    (chunk, key head)'s Gram tiles once and serves its G value heads in turn,
    and the recurrence groups a key head's workgroups on one XCD.  Ragged
    packed lengths with an initial state, against the oracle."""
    lens = [1, 200, 64, 65, 0, 131]
    cu = synth.cu_seqlens_of(lens)
    x = synth.gdr_inputs(40 + hv, B=1, T=int(cu[-1]), hk=hk, hv=hv, d=128, dtype="bf16")
    s0 = (0.05 * np.random.default_rng(41 + hv).standard_normal((len(lens), hv, 128, 128))).astype(np.float32)
    say(f"chunk varlen {lens} heads {hk}/{hv}")
    _check(x, cu=cu, s0=s0)


def test_varlen_packed_equals_separate_bit_exact():
    import torch
    lens = [70, 1, 129, 64]
    cu = synth.cu_seqlens_of(lens)
    x = synth.gdr_inputs(23, B=1, T=int(cu[-1]), dtype="bf16")
    s0 = (0.05 * np.random.default_rng(24).standard_normal((len(lens), 48, 128, 128))).astype(np.float32)
    say("chunk varlen packed vs separate (bit-exact)")
    o, s = _gpu_chunk(x, cu=cu, s0=s0)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        xn = synth.GDRInputs(x.q[:, sl], x.k[:, sl], x.v[:, sl], x.g[:, sl], x.beta[:, sl], x.A_log,
                             x.dt_bias, "bf16", 64)
        on, sn = _gpu_chunk(xn, s0=s0[n:n + 1])
        assert bits_equal(o[:, cu[n]:cu[n + 1]], on)
        assert bits_equal(s[n:n + 1], sn)


def test_varlen_many_sequences_launch_order():
    """1031 sequences: more than one per thread of the chunk-table kernel,
    empty ones, and one of 1032 chunks (past the top class of the
    longest-first launch order).  Every (sequence, head, slice) must run once."""
    rng = np.random.default_rng(26)
    lens = list(rng.integers(0, 40, size=1030))
    lens.insert(500, 66000)
    cu = synth.cu_seqlens_of(lens)
    x = synth.gdr_inputs(27, B=1, T=int(cu[-1]), hk=1, hv=2, d=128, dtype="bf16")
    s0 = (0.05 * np.random.default_rng(28).standard_normal((len(lens), 2, 128, 128))).astype(np.float32)
    say(f"chunk varlen {len(lens)} sequences, {int(cu[-1])} tokens")
    _check(x, cu=cu, s0=s0)


def test_nan_in_one_sequence_stays_there():
    import torch
    lens = [100, 90, 80]
    cu = synth.cu_seqlens_of(lens)
    x = synth.gdr_inputs(25, B=1, T=int(cu[-1]), dtype="bf16")
    say("chunk NaN isolation")
    o1, s1 = _gpu_chunk(x, cu=cu)
    v = x.v.copy()
    v[0, cu[1] + 7] = np.nan
    x2 = synth.GDRInputs(x.q, x.k, v, x.g, x.beta, x.A_log, x.dt_bias, "bf16", 64)
    o2, s2 = _gpu_chunk(x2, cu=cu)
    for n in (0, 2):
        assert bits_equal(o1[:, cu[n]:cu[n + 1]], o2[:, cu[n]:cu[n + 1]])
        assert bits_equal(s1[n], s2[n])
    assert torch.isnan(s2[1]).any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_write_no_decay_keeps_state_bit_exact(dtype):
    """beta = 0 and g = 0 (the degenerate case of the update): the final state is
    the initial state bit for bit on both paths, and o = S0 q^ within tolerance."""
    import torch
    x = synth.gdr_inputs(44, B=1, T=200, dtype=dtype, initial_state_std=0.05)
    x = synth.GDRInputs(x.q, x.k, x.v, np.zeros_like(x.g), np.zeros_like(x.beta), x.A_log, x.dt_bias, dtype, 64,
                        x.initial_state)
    say(f"chunk beta=0, g=0, {dtype}")
    o, s = _check(x, s0=x.initial_state, tol=BF16_TOL if dtype == "bf16" else F32_TOL)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(s), x.initial_state)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reset_by_infinite_decay(dtype):
    """g = -inf (alpha = 0) on a few tokens, inside chunks and at a chunk start:
    the state restarts from beta v k^T there (oracle: exact reset)."""
    x = synth.gdr_inputs(45, B=1, T=300, dtype=dtype, initial_state_std=0.05)
    g = x.g.copy()
    g[0, [5, 64, 130, 131, 299], :] = -np.inf
    g[0, 200, ::2] = -np.inf
    x = synth.GDRInputs(x.q, x.k, x.v, g, x.beta, x.A_log, x.dt_bias, dtype, 64, x.initial_state)
    say(f"chunk g=-inf resets, {dtype}")
    _check(x, s0=x.initial_state, tol=BF16_TOL if dtype == "bf16" else F32_TOL)


def test_chained_calls_equal_single_call_bit_exact():
    """Resume at chunk multiples: 4 x 256 chained calls == one 1024-token call."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    x = synth.gdr_inputs(26, B=1, T=1024, dtype="bf16")
    say("chunk chained 4x256 vs single 1024")
    o, s = _gpu_chunk(x)
    a = _dev_inputs(x, dev)
    state = torch.zeros((1, 48, 128, 128), device=dev)
    outs = []
    for i in range(4):
        sl = slice(256 * i, 256 * (i + 1))
        oi, _ = gdr_amd.chunk_gated_delta_rule(a["q"][:, sl].contiguous(), a["k"][:, sl].contiguous(),
                                               a["v"][:, sl].contiguous(), a["g"][:, sl].contiguous(),
                                               a["beta"][:, sl].contiguous(), state, final_state=state)
        outs.append(oi)
    torch.cuda.synchronize()
    assert bits_equal(torch.cat(outs, 1), o)
    assert bits_equal(state, s)


def test_deterministic():
    x = synth.layer_prefill(T=700)
    say("chunk determinism T=700")
    o1, s1 = _gpu_chunk(x)
    o2, s2 = _gpu_chunk(x)
    assert bits_equal(o1, o2) and bits_equal(s1, s2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_two_stages_equal_one_call_bit_exact(dtype):
    """gdr_chunk_fwd_prepare then gdr_chunk_fwd_recurrence = gdr_chunk_fwd, bit for bit,
    on a packed batch with a ragged tail (both the bf16-MFMA and the fp32 path)."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    lens = [70, 0, 129]
    x = synth.gdr_inputs(41, B=1, T=sum(lens), dtype=dtype)
    cu = synth.cu_seqlens_of(lens)
    s0 = (0.05 * np.random.default_rng(42).standard_normal((len(lens), 48, 128, 128))).astype(np.float32)
    say(f"chunk two stages vs one call, {dtype}, lengths {lens}")
    a = _dev_inputs(x, dev, cu, s0)
    args = (a["q"], a["k"], a["v"], a["g"], a["beta"], a["initial_state"])
    o1, s1 = gdr_amd.chunk_gated_delta_rule(*args, output_final_state=True, cu_seqlens=a["cu_seqlens"])
    ws = gdr_amd.chunk_workspace(a["q"], a["v"], a["cu_seqlens"])
    assert (ws is None) == (dtype == "f32")
    o2 = torch.empty_like(o1)
    s2 = torch.empty_like(s1)
    for stage in ("prepare", "recurrence"):
        gdr_amd.chunk_gated_delta_rule(*args, cu_seqlens=a["cu_seqlens"], final_state=s2, out=o2, workspace=ws,
                                       stage=stage)
    torch.cuda.synchronize()
    assert bits_equal(o1, o2) and bits_equal(s1, s2)


@pytest.mark.parametrize("T,hk,hv,mode", [(8192, 16, 48, "f32"), (3 * 4096 + 77, 2, 6, "f32"),
                                          (3 * 4096 + 77, 2, 6, "inplace"), (2 * 4096 + 1, 16, 48, "nostate"),
                                          (9000, 16, 48, "bf16out")])
def test_long_single_sequence_equals_stagewise(T, hk, hv, mode):
    """One long sequence (ragged tails included) through gdr_chunk_fwd equals
    gdr_chunk_fwd_prepare + gdr_chunk_fwd_recurrence bit for bit (outputs and
    final state), with the state in place, absent, and with bf16 outputs; and
    matches the oracle."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    x = synth.gdr_inputs(60 + T % 97, B=1, T=T, hk=hk, hv=hv, dtype="bf16",
                         initial_state_std=None if mode == "nostate" else 0.05)
    say(f"chunk long single sequence T={T} heads {hk}/{hv} {mode}")
    a = _dev_inputs(x, dev, s0=x.initial_state)
    args = (a["q"], a["k"], a["v"], a["g"], a["beta"])
    odt = torch.bfloat16 if mode == "bf16out" else torch.float32
    s_in = a["initial_state"]
    if mode == "inplace":
        s1 = s_in.clone()
        o1, _ = gdr_amd.chunk_gated_delta_rule(*args, s1, final_state=s1, out_dtype=odt)
    elif mode == "nostate":
        o1, s1 = gdr_amd.chunk_gated_delta_rule(*args, None, out_dtype=odt), None
        o1 = o1[0]
    else:
        o1, s1 = gdr_amd.chunk_gated_delta_rule(*args, s_in, output_final_state=True, out_dtype=odt)
    ws = gdr_amd.chunk_workspace(a["q"], a["v"])
    o2 = torch.empty_like(o1)
    s2 = torch.empty((1, hv, 128, 128), device=dev)
    for stage in ("prepare", "recurrence"):
        gdr_amd.chunk_gated_delta_rule(*args, s_in, final_state=s2, out=o2, workspace=ws, stage=stage,
                                       out_dtype=odt)
    torch.cuda.synchronize()
    assert bits_equal(o1, o2)
    if s1 is not None:
        assert bits_equal(s1, s2)
    if hv <= 6 or T <= 8192:
        heads = list(range(hv)) if hv <= 6 else [0, 23, 47]
        o_ref, s_ref = ref.forward(x.q, x.k, x.v, x.g, x.beta, x.initial_state, None, heads=heads)
        eo = rel_err(to_host(o2)[:, :, heads], o_ref[:, :, heads])
        es = rel_err(to_host(s2)[:, heads], s_ref[:, heads])
        say(f"  o err {eo:.2e}  state err {es:.2e}")
        assert eo <= BF16_TOL and es <= BF16_TOL


@pytest.mark.parametrize("d,dtype,C", [(64, "bf16", 64), (64, "f32", 64), (128, "f32", 64), (128, "bf16", 32),
                                       (32, "bf16", 32)])
def test_other_shapes_fp32_path(d, dtype, C):
    x = synth.gdr_inputs(30 + d + C, B=1, T=150, hk=2, hv=6, d=d, dtype=dtype, chunk_size=C,
                         initial_state_std=0.05)
    say(f"chunk fp32 path d={d} {dtype} C={C}")
    _check(x, s0=x.initial_state, tol=F32_TOL if dtype == "f32" else BF16_TOL)


def test_bf16_output():
    import torch
    x = synth.layer_prefill(T=300)
    say("chunk bf16 output T=300")
    o, s = _gpu_chunk(x, out_dtype=torch.bfloat16)
    o_ref, s_ref, _ = ref.forward_parallel(x.q, x.k, x.v, x.g, x.beta)
    og = to_host(o)
    rms = np.sqrt(np.mean(o_ref ** 2))
    from helpers import bf16_ulp
    assert np.all(np.abs(og - o_ref) <= bf16_ulp(o_ref) + BF16_TOL * rms)
    assert rel_err(to_host(s), s_ref) <= BF16_TOL


def test_query_scale_and_no_l2norm():
    x = synth.gdr_inputs(40, B=1, T=130, dtype="bf16")
    say("chunk scale=0.088, use_qk_l2norm=False")
    o, s = _gpu_chunk(x, scale=0.088, use_qk_l2norm_in_kernel=False)
    o_ref, s_ref, _ = ref.forward_parallel(x.q, x.k, x.v, x.g, x.beta, use_qk_l2norm=False, scale=0.088)
    assert rel_err(to_host(o), o_ref) <= BF16_TOL and rel_err(to_host(s), s_ref) <= BF16_TOL


def test_long_context_resume():
    """T = 262144 as 8 chained 32768-token calls (final_state -> initial_state).

    Oracle: the first 4096 outputs of call 0, and the final state after a
    16384-token prefix, which the GPU computes both as one call and as 4
    chained 4096-token calls (these two must also agree bit for bit).
    """
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    x0 = _long_call(0)
    say("long context: call 0 prefix checks")
    a = _dev_inputs(x0, dev)
    o_full, _ = gdr_amd.chunk_gated_delta_rule(a["q"], a["k"], a["v"], a["g"], a["beta"])
    o_ref, _, _ = ref.forward_parallel(x0.q[:, :4096], x0.k[:, :4096], x0.v[:, :4096], x0.g[:, :4096],
                                       x0.beta[:, :4096])
    torch.cuda.synchronize()
    assert rel_err(to_host(o_full[:, :4096]), o_ref) <= BF16_TOL
    P = 16384
    sl = lambda t, i, j: t[:, i:j].contiguous()
    _, s_one = gdr_amd.chunk_gated_delta_rule(sl(a["q"], 0, P), sl(a["k"], 0, P), sl(a["v"], 0, P),
                                              sl(a["g"], 0, P), sl(a["beta"], 0, P), output_final_state=True)
    st = torch.zeros((1, 48, 128, 128), device=dev)
    for i in range(4):
        j0, j1 = 4096 * i, 4096 * (i + 1)
        gdr_amd.chunk_gated_delta_rule(sl(a["q"], j0, j1), sl(a["k"], j0, j1), sl(a["v"], j0, j1),
                                       sl(a["g"], j0, j1), sl(a["beta"], j0, j1), st, final_state=st)
    torch.cuda.synchronize()
    assert bits_equal(s_one, st)
    _, s_ref, _ = ref.forward_parallel(x0.q[:, :P], x0.k[:, :P], x0.v[:, :P], x0.g[:, :P], x0.beta[:, :P])
    assert rel_err(to_host(s_one), s_ref) <= BF16_TOL
    say("long context: 8 chained 32K calls")
    state = torch.zeros((1, 48, 128, 128), device=dev)
    norms = []
    for i in range(8):
        xi = x0 if i == 0 else synth.long_context_call(i)
        ai = a if i == 0 else _dev_inputs(xi, dev)
        o, _ = gdr_amd.chunk_gated_delta_rule(ai["q"], ai["k"], ai["v"], ai["g"], ai["beta"], state,
                                              final_state=state)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(state).all()
        norms.append(float(state.norm()))
    # beta <= 1 and unit keys bound every state row by max |v| / (1 - max alpha); no blow-up
    assert max(norms) < 1e3


def test_long_context_chained_calls_against_oracle():
    """CFG4 beyond the 16K prefix: two chained 32768-token calls (65 536
    tokens, final_state -> initial_state), against the oracle carrying its own
    fp64 state from call to call, on three sampled value heads: every output
    of each call and the state after each call."""
    import gated_delta_rule_amd as gdr_amd
    import torch
    dev = gpu()
    heads = [1, 20, 46]
    state = torch.zeros((1, 48, 128, 128), device=dev)
    s_ref = np.zeros((1, 48, 128, 128))
    for i in range(2):
        say(f"long context: chained call {i} against the oracle, heads {heads}")
        xi = _long_call(i)
        ai = _dev_inputs(xi, dev)
        o, _ = gdr_amd.chunk_gated_delta_rule(ai["q"], ai["k"], ai["v"], ai["g"], ai["beta"], state,
                                              final_state=state)
        o_ref, s_ref = ref.forward(xi.q, xi.k, xi.v, xi.g, xi.beta, s_ref, heads=heads)
        torch.cuda.synchronize()
        oh = to_host(o[:, :, heads])
        sh = to_host(state[:, heads])
        assert rel_err(oh, o_ref[:, :, heads]) <= BF16_TOL, f"call {i}: o"
        assert rel_err(sh, s_ref[:, heads]) <= BF16_TOL, f"call {i}: state"
