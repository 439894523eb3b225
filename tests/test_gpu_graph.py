"""The path under HIP graph capture, for callers that replay a recorded step
(serving loops): the entry point that allocates nothing (prefill) and the
in-place decode step are captured into a graph, the graph is replayed
several times with eager work and synchronisation between the replays, and
every replay is checked bit for bit against the same call run eagerly.  No
call on these paths enqueues a memset (none would be safe to record)."""
import ctypes

import numpy as np
import pytest

from helpers import bits_equal, gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(desc, q, k, v, g, beta, init, fin, cu, o):
    import torch
    from gated_delta_rule_amd import _lib
    p = lambda t: None if t is None else t.data_ptr()
    st = _lib.load().gdr_chunk_fwd_noalloc(ctypes.byref(desc), p(q), p(k), p(v), p(g), p(beta), p(init), p(fin),
                                           p(cu), p(o), torch.cuda.current_stream(q.device).cuda_stream)
    _lib.check("gdr_chunk_fwd_noalloc", st)


def test_noalloc_prefill_replayed_from_a_graph():
    import torch
    from gated_delta_rule_amd import ops
    from inputs import synth
    dev = gpu()
    lengths = [300, 64, 37]
    T, N = sum(lengths), len(lengths)
    cu = to_dev(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), "i32", dev)
    desc = ops.make_desc(1, T, N, 16, 48, 128, 64, torch.bfloat16, torch.float32, True, 1.0, 1e-6)

    def inputs(seed):
        inp = synth.gdr_inputs(seed, T=T)
        s0 = np.random.Generator(np.random.PCG64(seed)).normal(0, 0.05, (N, 48, 128, 128)).astype(np.float32)
        return ([to_dev(x, "bf16", dev) for x in (inp.q, inp.k, inp.v)] +
                [to_dev(inp.g, "f32", dev), to_dev(inp.beta, "f32", dev), to_dev(s0, "f32", dev)])

    # static buffers the graph reads and writes
    q, k, v, g, beta, init = inputs(91)
    o = torch.empty((T, 48, 128), device=dev, dtype=torch.float32)
    fin = torch.empty((N, 48, 128, 128), device=dev, dtype=torch.float32)

    def eager(bufs):
        o_e = torch.full_like(o, float("nan"))
        f_e = torch.full_like(fin, float("nan"))
        _noalloc(desc, *bufs[:6], f_e, cu, o_e)
        torch.cuda.synchronize()
        return o_e, f_e

    say(f"graph: noalloc prefill T={T} N={N}")
    _noalloc(desc, q, k, v, g, beta, init, fin, cu, o)  # first call on the device outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _noalloc(desc, q, k, v, g, beta, init, fin, cu, o)
    for rep, seed in enumerate((91, 92, 91, 93)):
        new = inputs(seed)
        for dst, src in zip((q, k, v, g, beta, init), new):
            dst.copy_(src)
        o_ref, f_ref = eager(new)  # eager work between the replays
        o.fill_(float("nan"))
        fin.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"graph: replay {rep} (inputs of seed {seed})")
        assert bits_equal(o, o_ref), f"replay {rep}: o differs from the eager call"
        assert bits_equal(fin, f_ref), f"replay {rep}: final state differs from the eager call"


def test_decode_step_replayed_from_a_graph():
    import torch
    import gated_delta_rule_amd as gdr
    from inputs import synth
    dev = gpu()
    N = 16
    rng = np.random.Generator(np.random.PCG64(94))
    s0 = (rng.standard_normal((N, 48, 128, 128), dtype=np.float32) * 0.05)
    steps = []
    for s in range(4):
        xi = synth.decode_step_inputs(300 + s, N=N)
        steps.append([to_dev(xi.q, "bf16", dev), to_dev(xi.k, "bf16", dev), to_dev(xi.v, "bf16", dev),
                      to_dev(xi.g, "f32", dev), to_dev(xi.beta, "f32", dev)])
    # eager reference: four steps in a row on one state
    st_ref = to_dev(s0, "f32", dev)
    o_refs = []
    for x in steps:
        o_e = torch.empty((N, 48, 128), device=dev, dtype=torch.float32)
        gdr.recurrent_step(*x, st_ref, out=o_e)
        o_refs.append(o_e)
    torch.cuda.synchronize()
    # graph: one step on static buffers, replayed once per step
    st = to_dev(s0, "f32", dev)
    xs = [t.clone() for t in steps[0]]
    o = torch.empty((N, 48, 128), device=dev, dtype=torch.float32)
    warm = to_dev(s0, "f32", dev)
    gdr.recurrent_step(*xs, warm, out=torch.empty_like(o))  # first call outside the capture
    torch.cuda.synchronize()
    say(f"graph: decode step N={N}")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdr.recurrent_step(*xs, st, out=o)
    for s, x in enumerate(steps):
        for dst, src in zip(xs, x):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _ = (o * 2).sum().item()  # eager work between the replays
        say(f"graph: decode replay {s}")
        assert bits_equal(o, o_refs[s]), f"replay {s}: output differs from the eager step"
    assert bits_equal(st, st_ref), "state after the replays differs from the eager steps"
