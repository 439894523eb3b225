"""GDR_DEBUG_CHECKS on the GPU: the index arrays the kernels trust are
checked on the host and bad ones rejected with INVALID_ARG before any launch;
the NaN-filled workspaces leave every result bit-identical (no kernel reads a
workspace entry that no kernel wrote)."""
import contextlib
import ctypes
import os

import numpy as np
import pytest

from helpers import bits_equal, gpu, say, to_dev
from inputs import synth

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def debug_checks():
    old = os.environ.get("GDR_DEBUG_CHECKS")
    os.environ["GDR_DEBUG_CHECKS"] = "1"
    try:
        yield
    finally:
        if old is None:
            del os.environ["GDR_DEBUG_CHECKS"]
        else:
            os.environ["GDR_DEBUG_CHECKS"] = old


def _expect_invalid(fn, text):
    from gated_delta_rule_amd import GDRError
    with pytest.raises(GDRError) as e:
        fn()
    assert e.value.status == -1, str(e.value)
    assert "GDR_DEBUG_CHECKS" in str(e.value) and text in str(e.value), str(e.value)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_chunk_debug_mode_bit_identical_and_rejects_bad_offsets(out_dtype):
    import torch
    import gated_delta_rule_amd as gdr_amd
    from gated_delta_rule_amd import _lib, ops
    dev = gpu()
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    lengths = [100, 0, 64, 37, 130]
    T = sum(lengths)
    inp = synth.gdr_inputs(81, T=T)
    q, k, v = (to_dev(x, "bf16", dev) for x in (inp.q, inp.k, inp.v))
    g, beta = to_dev(inp.g, "f32", dev), to_dev(inp.beta, "f32", dev)
    cu_np = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cu = to_dev(cu_np, "i32", dev)
    s0 = to_dev(np.random.Generator(np.random.PCG64(81)).normal(0, 0.05, (5, 48, 128, 128)).astype(np.float32),
                "f32", dev)
    say(f"debug checks: chunk packed T={T} out={out_dtype}")
    o_ref, s_ref = gdr_amd.chunk_gated_delta_rule(q, k, v, g, beta, s0, output_final_state=True, cu_seqlens=cu,
                                                  out_dtype=odt)
    with debug_checks():
        o, s = gdr_amd.chunk_gated_delta_rule(q, k, v, g, beta, s0, output_final_state=True, cu_seqlens=cu,
                                              out_dtype=odt)
        torch.cuda.synchronize()
        assert bits_equal(o, o_ref) and bits_equal(s, s_ref)
        # the no-allocation entry point's static scratch is filled the same way
        desc = ops.make_desc(1, T, 5, 16, 48, 128, 64, torch.bfloat16, odt, True, 1.0, 1e-6)
        o2 = torch.empty_like(o_ref)
        s2 = torch.empty_like(s_ref)
        p = lambda t: t.data_ptr()
        st = _lib.load().gdr_chunk_fwd_noalloc(ctypes.byref(desc), p(q), p(k), p(v), p(g), p(beta), p(s0), p(s2),
                                               p(cu), p(o2), torch.cuda.current_stream(dev).cuda_stream)
        _lib.check("gdr_chunk_fwd_noalloc", st)
        torch.cuda.synchronize()
        assert bits_equal(o2, o_ref) and bits_equal(s2, s_ref)
        for bad, text in (([0, 100, 90, 164, 201, T], "decreases"), ([0, 100, 100, 164, 201, T - 1], "token count"),
                          ([3, 100, 100, 164, 201, T], "must be 0")):
            bad_cu = to_dev(np.asarray(bad, np.int32), "i32", dev)
            _expect_invalid(lambda: gdr_amd.chunk_gated_delta_rule(q, k, v, g, beta, s0, output_final_state=True,
                                                                   cu_seqlens=bad_cu, out_dtype=odt), text)
    # without the mode the same call is not checked (contents are trusted): not run here


def test_decode_debug_mode_rejects_a_slot_named_twice():
    import torch
    import gated_delta_rule_amd as gdr_amd
    dev = gpu()
    A_log, dt, s0 = synth.decode_inputs(N=4)
    x = synth.decode_step_inputs(0, N=3)
    q, k, v = (to_dev(t, "bf16", dev) for t in (x.q, x.k, x.v))
    g, beta = to_dev(x.g, "f32", dev), to_dev(x.beta, "f32", dev)
    pool = to_dev(s0, "f32", dev)
    good = to_dev(np.asarray([2, -1, 0], np.int32), "i32", dev)
    say("debug checks: decode pool indices")
    ref_pool = pool.clone()
    o_ref = gdr_amd.recurrent_step(q, k, v, g, beta, ref_pool, state_indices=good)
    with debug_checks():
        p2 = pool.clone()
        o = gdr_amd.recurrent_step(q, k, v, g, beta, p2, state_indices=good)
        torch.cuda.synchronize()
        assert bits_equal(o, o_ref) and bits_equal(p2, ref_pool)
        dup = to_dev(np.asarray([2, 1, 2], np.int32), "i32", dev)
        _expect_invalid(lambda: gdr_amd.recurrent_step(q, k, v, g, beta, pool.clone(), state_indices=dup), "twice")


def test_conv_debug_mode():
    import torch
    import gated_delta_rule_amd as gdr_amd
    dev = gpu()
    p = synth.pipeline_inputs(seed=82, lengths=[70, 33])
    bf = lambda a: to_dev(a, "bf16", dev)
    f32 = lambda a: to_dev(a, "f32", dev)
    say("debug checks: conv front offsets")
    with debug_checks():
        cu = to_dev(p.cu_seqlens.astype(np.int32), "i32", dev)
        out = gdr_amd.conv_gate_fused(bf(p.x), bf(p.conv_w), cu, f32(p.a), f32(p.b), f32(p.A_log),
                                      f32(p.dt_bias), p.hk, p.hv, p.d)
        torch.cuda.synchronize()
        assert out[0].shape[1] == 103
        bad = to_dev(np.asarray([0, 80, 70], np.int32), "i32", dev)
        _expect_invalid(lambda: gdr_amd.conv_gate_fused(bf(p.x), bf(p.conv_w), bad, f32(p.a), f32(p.b),
                                                        f32(p.A_log), f32(p.dt_bias), p.hk, p.hv, p.d), "decreases")


def test_attn_prefill_debug_mode_bit_identical():
    """The attention prefill's workspace (q', the padded keys and V^T) filled
    with NaN first: keys past a sequence's end are never written, so the
    output staying bit-identical shows the mask keeps them out of every
    score, maximum and sum."""
    import torch
    import gated_delta_rule_amd as gdr_amd
    dev = gpu()
    lengths = (1, 63, 64, 65, 0, 129, 31)
    x = synth.attn_inputs(83, lengths=lengths, hq=8, hk=2)
    bf = lambda a: to_dev(a, "bf16", dev)
    f32 = lambda a: to_dev(a, "f32", dev)
    cu = to_dev(x.cu_seqlens.astype(np.int32), "i32", dev)
    args = (bf(x.q), bf(x.k), bf(x.v), bf(x.gate), f32(x.q_norm_w), f32(x.k_norm_w), cu)
    say(f"debug checks: attention prefill lengths {lengths}")
    ref = gdr_amd.attn_prefill(*args)
    with debug_checks():
        out = gdr_amd.attn_prefill(*args)
        torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert bits_equal(out, ref)
