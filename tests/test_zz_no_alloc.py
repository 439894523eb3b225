"""gdr_chunk_fwd_noalloc (static device scratch) against gdr_chunk_fwd, through
the C ABI: two calls in a row, the second smaller, each bit-identical to the
call with a caller-provided workspace."""
import ctypes

import numpy as np
import pytest

from helpers import bits_equal, gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _call_noalloc(desc, q, k, v, g, beta, init, fin, cu, o):
    import torch
    from gated_delta_rule_amd import _lib
    lib = _lib.load()
    p = lambda t: None if t is None else t.data_ptr()
    st = lib.gdr_chunk_fwd_noalloc(ctypes.byref(desc), p(q), p(k), p(v), p(g), p(beta), p(init), p(fin), p(cu),
                                   p(o), torch.cuda.current_stream(q.device).cuda_stream)
    _lib.check("gdr_chunk_fwd_noalloc", st)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_call(out_dtype):
    import torch
    import gated_delta_rule_amd as gdr_amd
    from gated_delta_rule_amd import ops
    from inputs import synth
    dev = gpu()
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    cases = [
        # packed batch with a ragged tail, zero initial state
        dict(seed=71, lengths=[700, 64, 1, 735], init=False),
        # then a smaller single sequence that resumes a state
        dict(seed=72, lengths=[300], init=True),
    ]
    for case in cases:
        lengths = case["lengths"]
        T = int(sum(lengths))
        inp = synth.gdr_inputs(case["seed"], T=T)
        cu_np = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        N = len(lengths)
        q, k, v = (to_dev(x, "bf16", dev) for x in (inp.q, inp.k, inp.v))
        g, beta = to_dev(inp.g, "f32", dev), to_dev(inp.beta, "f32", dev)
        cu = to_dev(cu_np, "i32", dev) if N > 1 else None
        init = None
        if case["init"]:
            s0 = np.random.Generator(np.random.PCG64(case["seed"])).normal(0, 0.05, (N, 48, 128, 128))
            init = to_dev(s0.astype(np.float32), "f32", dev)
        say(f"noalloc case seed={case['seed']} T={T} N={N} out={out_dtype}")
        o_ref, s_ref = gdr_amd.chunk_gated_delta_rule(q, k, v, g, beta, init, output_final_state=True,
                                                      cu_seqlens=cu, out_dtype=odt)
        desc = ops.make_desc(1, T, N, 16, 48, 128, 64, torch.bfloat16, odt, True, 1.0, 1e-6)
        o = torch.full_like(o_ref, float("nan"))
        fin = torch.full_like(s_ref, float("nan"))
        _call_noalloc(desc, q, k, v, g, beta, init, fin, cu, o)
        torch.cuda.synchronize()
        assert bits_equal(o, o_ref), "o differs from gdr_chunk_fwd"
        assert bits_equal(fin, s_ref), "final state differs from gdr_chunk_fwd"
