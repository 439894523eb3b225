#!/usr/bin/env python3
"""Throughput of the gated delta rule path on one MI355X.

A step is one 32768-token chunked-prefill call of one delta layer
(16 key / 48 value heads, d = 128, bf16 q/k/v, fp32 gates, state and output,
chunk 64) that resumes from the previous call's final state.  The calls are
the 8 consecutive pieces of one 262144-token context (distinct inputs, all
resident in HBM); step s runs piece s % 8.  ``value`` is the prefill rate in
tokens/s over the K timed steps.  The same JSON line also reports, measured
in the same run:

  decode    -- 64 sequences x 48 heads of 128x128 fp32 state, one token per
               step, state updated in place, 256 steps: state GB/s; also
               with two state sets, and from a 128-slot state pool with the
               rows naming shuffled slots and slots in row order
  decode_layer -- one token of the whole layer path for the same 64
               sequences in one launch (conv front, gates, recurrent step,
               gated RMS norm), beside the same work as three launches
               (the decode entries' frac_hbm counts every algorithmic byte,
               frac_hbm_state_only the recurrent state alone)
  pipeline  -- the whole layer path over a packed batch of 8 sequences
               (65536 tokens): conv+SiLU+gates, recurrence, gated RMSNorm
  layer     -- one whole delta layer on a 32768-token sequence with synthetic
               weights: in-projection GEMM, the path, out-projection GEMM
               (hidden 5120); stage times and the GEMMs' matrix-core rate
  attention -- the global attention layer (24/4 heads, d 256): causal prefill
               of a 32768-token sequence (matrix-core rate) and one decode
               token for 64 sequences against 32768-slot KV caches (HBM rate)
  roofline  -- the dominant kernel of the call, the state-carrying
               recurrence (gdr_chunk_fwd_recurrence): its algorithmic bf16
               matrix-core FLOPs per launch (the state-dependent products of
               the chunk form, triangle-exact) over its average launch time
               (HIP events on the launch stream, around each recurrence launch
               inside the timed loop), against the 2.5 PFLOP/s dense bf16
               peak; beside it the whole call's MFMA fraction (prepare
               included), the kernel's algorithmic HBM bytes per launch (q, k,
               v read, o written, state in and out) against 8 TB/s, and the
               HBM bytes the committed rocprofv3 counters measured for it
  achievable -- the roofline probes (libgdr_roofline.so): streaming HBM
               read-modify-write and read rates, the dense bf16 matrix-core
               rate and the fp32 vector-ALU issue rate this GPU delivers,
               beside the datasheet peaks
  clocks    -- the driver's current clock levels before and after the run
  cpu_baseline -- the fp64 CPU oracle timed on the host cores on a bounded
               sample of the same workload (the first three 32K-token calls;
               and 4 decode steps for the decode leg)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--pieces P] [--no-cpu]
                       [--only prefill|decode|decode_layer|pipeline|layer|attention|copy|roofline|all]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
HK, HV, D, C = 16, 48, 128, 64
T_CALL = 32768
N_CALLS = 8  # pieces of the 262144-token context

# Algorithmic bytes per prefill token: q, k (2*Hk*d bf16) + v (Hv*d bf16)
# + g, beta (2*Hv fp32) + o (Hv*d fp32); per call add one read and one write
# of the Hv x d x d fp32 state.
PREFILL_BYTES_PER_TOKEN = 2 * HK * D * 2 + HV * D * 2 + 2 * HV * 4 + HV * D * 4
STATE_BYTES = HV * D * D * 4
# Algorithmic FLOPs per token of the chunk form (triangle-exact):
# Hv*(6*dk*dv + 2*C*dv + C^2/3) + Hk*2*C*dk
PREFILL_FLOP_PER_TOKEN = HV * (6 * D * D + 2 * C * D + C * C / 3) + HK * 2 * C * D
# The recurrence kernel's share: q, k, v read and o written per token (g and
# beta are read by the prepare stage), and the state-dependent products
# X = K S0^T, Y = Q S0^T, the state update (2 dk dv each) and T R, P Delta
# (C dv each, triangle-exact).
RECUR_BYTES_PER_TOKEN = 2 * HK * D * 2 + HV * D * 2 + HV * D * 4
RECUR_FLOP_PER_TOKEN = HV * (6 * D * D + 2 * C * D)
RECUR_KERNEL = "gdr::chunk_rec_kernel<float>"
COUNTERS = os.path.join(ROOT, "profiles", "chunk_prefill_T32768_counters.json")
KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_amd", "csrc", "kernels", "chunk_bf16.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def long_context_host(n: int = N_CALLS):
    """The n calls' host inputs, generated in parallel threads (numpy releases
    the GIL in the heavy parts)."""
    import concurrent.futures as cf
    from inputs import synth
    workers = max(1, min(n, len(os.sched_getaffinity(0)) // 2))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda i: synth.long_context_call(i, T=T_CALL), range(n)))


def bench_prefill(steps: int, warmup: int, host_calls):
    import torch
    import gated_delta_rule_amd as gdr
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    calls = [(bf(x.q), bf(x.k), bf(x.v), f32(x.g), f32(x.beta)) for x in host_calls]
    state = torch.zeros((1, HV, D, D), device=dev)
    o = torch.empty((1, T_CALL, HV, D), device=dev)
    ws = gdr.chunk_workspace(calls[0][0], calls[0][2])

    # One call = gdr_chunk_fwd_prepare + gdr_chunk_fwd_recurrence on the torch
    # stream (the same kernels gdr_chunk_fwd enqueues), so that events can
    # bracket the recurrence kernel alone.
    def stage(i, name):
        q, k, v, g, beta = calls[i % N_CALLS]
        gdr.chunk_gated_delta_rule(q, k, v, g, beta, state, final_state=state, out=o, workspace=ws, stage=name)

    log(f"prefill: {warmup} warmup + {steps} timed 32K calls over {N_CALLS} distinct pieces")
    for i in range(warmup):
        stage(i, "prepare")
        stage(i, "recurrence")
    torch.cuda.synchronize()
    per = []
    t0 = time.perf_counter()
    start, end = _events()
    start.record()
    for i in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        stage(warmup + i, "prepare")
        e[1].record()
        stage(warmup + i, "recurrence")
        e[2].record()
        per.append(e)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    prep_ms = [e[0].elapsed_time(e[1]) for e in per]
    recur_ms = [e[1].elapsed_time(e[2]) for e in per]
    call_ms = [e[0].elapsed_time(e[2]) for e in per]
    finite = bool(torch.isfinite(state).all() and torch.isfinite(o).all())
    return dict(total_ms=total_ms, wall_s=wall, prep_ms=prep_ms, recur_ms=recur_ms, call_ms=call_ms, finite=finite)


def bench_roofline(reps: int = 10):
    """Achievable rates of this GPU from the roofline probes."""
    import torch
    from gated_delta_rule_amd import roofline
    dev = torch.device("cuda:0")
    nbytes = 2 << 30  # 2 GiB: well past the 256 MB last-level cache
    buf = torch.ones(nbytes // 4, device=dev)
    sums = torch.empty(nbytes // roofline.SLAB, device=dev)

    def timed(fn):
        for _ in range(2):
            fn()
        start, end = _events()
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps

    rmw_nt = 2 * nbytes / (timed(lambda: roofline.rmw(buf, 1.0, True)) * 1e-3) / 1e9
    rmw = 2 * nbytes / (timed(lambda: roofline.rmw(buf, 1.0, False)) * 1e-3) / 1e9
    rd = nbytes / (timed(lambda: roofline.read(buf, sums)) * 1e-3) / 1e9
    del buf, sums
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs, iters = 8 * cus, 4000
    out = torch.empty(wgs * 4, device=dev)
    flop = wgs * 4 * iters * roofline.MFMA_FLOP_PER_WAVE_ITER
    mfma = flop / (timed(lambda: roofline.mfma(out, wgs, iters)) * 1e-3) / 1e12
    valu_iters = 20000
    valu = (wgs * 4 * valu_iters * roofline.VALU_INSTS_PER_WAVE_ITER
            / (timed(lambda: roofline.valu(out, wgs, valu_iters)) * 1e-3) / cus)
    log(f"roofline probes: rmw nt {rmw_nt:.0f} GB/s, rmw {rmw:.0f} GB/s, read {rd:.0f} GB/s, mfma {mfma:.0f} TFLOP/s, "
        f"valu {valu / 1e9:.3f} G wave-instructions/s per CU")
    return {"hbm_rmw_nontemporal_GBps": rmw_nt, "hbm_rmw_GBps": rmw, "hbm_read_GBps": rd,
            "mfma_bf16_TFLOPs": mfma, "valu_wave_insts_per_s_per_cu": valu, "buffer_bytes": nbytes}


def gpu_clocks():
    """Current shader and memory clock levels from the amdgpu driver's sysfs
    files (the lines marked '*' of pp_dpm_sclk / pp_dpm_mclk), or None where
    they cannot be read.  Read as files: no program is started."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
            except OSError:
                continue
            if cur:
                out[f"{os.path.basename(os.path.dirname(dev))}/{name}"] = cur[0]
    return out or None


def bench_decode(steps: int = 256, replicas: int = 1, pool: int = 0, shuffled: bool = True):
    """Decode steps of 64 sequences.  replicas > 1 cycles through that many
    copies of the state set; pool > 0 keeps the states in a pool of that many
    slots (gdr_recurrent_step_indexed) with the rows naming shuffled slots
    (shuffled=True) or slots 0..63 in row order.  frac_hbm counts every
    algorithmic byte (state read and written, q, k, v, gates, o);
    frac_hbm_state_only the state alone."""
    import torch
    import gated_delta_rule_amd as gdr
    from inputs import synth
    dev = torch.device("cuda:0")
    N = 64
    log(f"decode: N={N}, {steps} steps, " + (f"pool of {pool} slots" if pool else f"{replicas} state replica(s)"))
    A_log, dt, s0 = synth.decode_inputs(N=N)
    if pool:
        perm = np.random.default_rng(7).permutation(pool)[:N] if shuffled else np.arange(N)
        slots = torch.zeros((pool, HV, D, D), device=dev)
        slots[torch.as_tensor(perm, device=dev)] = torch.from_numpy(s0).to(dev)
        idx = torch.as_tensor(perm.astype(np.int32), device=dev)
        states = [slots]
    else:
        states = [torch.from_numpy(s0).to(dev) for _ in range(replicas)]
    del s0
    kw = dict(state_indices=idx) if pool else {}
    inputs = []
    for s in range(steps):
        xi = synth.decode_step_inputs(s, N=N)
        inputs.append((torch.from_numpy(xi.q).to(torch.bfloat16).to(dev),
                       torch.from_numpy(xi.k).to(torch.bfloat16).to(dev),
                       torch.from_numpy(xi.v).to(torch.bfloat16).to(dev),
                       torch.from_numpy(xi.g).to(dev), torch.from_numpy(xi.beta).to(dev)))
    o = torch.empty((N, HV, D), device=dev)
    for i in range(8):  # warmup
        gdr.recurrent_step(*inputs[i], states[i % len(states)], out=o, **kw)
    torch.cuda.synchronize()
    start, end = _events()
    start.record()
    for i in range(steps):
        gdr.recurrent_step(*inputs[i], states[i % len(states)], out=o, **kw)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    state_bytes = 2 * N * HV * D * D * 4
    other = N * (2 * HK * D * 2 + HV * D * 2 + 2 * HV * 4 + HV * D * 4)
    return dict(us_per_step=ms * 1e3, state_GBps=state_bytes / (ms * 1e-3) / 1e9,
                total_GBps=(state_bytes + other) / (ms * 1e-3) / 1e9,
                frac_hbm=(state_bytes + other) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                frac_hbm_state_only=state_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                working_set_MiB=replicas * state_bytes / 2 / 2**20)


def bench_decode_layer(steps: int = 128):
    """One decode token of the whole layer path for 64 sequences: the fused
    gdr_decode_layer_step against the same work as three launches
    (gdr_conv_gate_fused on one-token sequences, gdr_recurrent_step,
    gdr_gated_rmsnorm).  Bytes counted: the recurrent state read and written,
    plus x, the conv state (read and written), a, b, z and y; frac_hbm counts
    them all, frac_hbm_state_only the recurrent state alone."""
    import torch
    import gated_delta_rule_amd as gdr
    from inputs import synth
    dev = torch.device("cuda:0")
    N = 64
    C = (2 * HK + HV) * D
    log(f"decode layer: N={N}, {steps} steps, fused vs three launches")
    p0 = synth.pipeline_inputs(seed=7, lengths=[1] * N)
    A_log, dt, s0 = synth.decode_inputs(N=N)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    cw, nw, Al, dtb = bf(p0.conv_w), f32(p0.norm_w), f32(A_log), f32(dt)
    rng = np.random.default_rng(8)
    conv_state = bf(synth.round_bf16(rng.standard_normal((N, C, 3))))
    state = f32(s0)
    del s0
    steps_in = []
    for s in range(steps):
        pi = synth.pipeline_inputs(seed=200 + s, lengths=[1] * N)
        steps_in.append((bf(pi.x), f32(pi.a), f32(pi.b), bf(pi.z)))
    cu = torch.arange(N + 1, device=dev, dtype=torch.int32)

    def fused(i):
        x, a, b, z = steps_in[i % steps]
        gdr.decode_layer_step(x, cw, conv_state, a, b, Al, dtb, state, z, nw, HK, HV)

    cs_out = torch.empty_like(conv_state)

    def unfused(i):
        x, a, b, z = steps_in[i % steps]
        q, k, v, g, beta, _ = gdr.conv_gate_fused(x, cw, cu, a, b, Al, dtb, HK, HV, D, conv_state_in=conv_state,
                                                  output_conv_state=False)
        o = gdr.recurrent_step(q[0], k[0], v[0], g[0], beta[0], state)
        gdr.gated_rmsnorm(o.reshape(1, N, HV, D), z.reshape(1, N, HV * D), nw)

    def timed(fn):
        for i in range(8):
            fn(i)
        torch.cuda.synchronize()
        start, end = _events()
        start.record()
        for i in range(steps):
            fn(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    ms_f = timed(fused)
    ms_u = timed(unfused)
    state_bytes = 2 * N * HV * D * D * 4
    other = N * (C * 2 + 2 * C * 3 * 2 + 2 * HV * 4 + 2 * HV * D * 2)
    return dict(us_per_step=ms_f * 1e3, state_GBps=state_bytes / (ms_f * 1e-3) / 1e9,
                total_GBps=(state_bytes + other) / (ms_f * 1e-3) / 1e9,
                frac_hbm=(state_bytes + other) / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS,
                frac_hbm_state_only=state_bytes / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS,
                three_launches_us_per_step=ms_u * 1e3)


def bench_pipeline(reps: int = 5):
    import torch
    import gated_delta_rule_amd as gdr
    from inputs import synth
    dev = torch.device("cuda:0")
    log("pipeline: generating 8-sequence packed batch (65536 tokens)")
    p = synth.pipeline_inputs()
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    x, w, z = bf(p.x), bf(p.conv_w), bf(p.z)
    a, b, A_log, dt, nw = f32(p.a), f32(p.b), f32(p.A_log), f32(p.dt_bias), f32(p.norm_w)
    cu = torch.from_numpy(p.cu_seqlens).to(dev)
    T = int(p.cu_seqlens[-1])
    del p
    times = {"front": [], "recurrence": [], "norm": []}
    for r in range(reps + 1):
        ev = [_events()[0] for _ in range(4)]
        ev[0].record()
        q, k, v, g, beta, _ = gdr.conv_gate_fused(x, w, cu, a, b, A_log, dt, HK, HV, D)
        ev[1].record()
        o, s = gdr.chunk_gated_delta_rule(q, k, v, g, beta, None, output_final_state=True, cu_seqlens=cu)
        ev[2].record()
        y = gdr.gated_rmsnorm(o, z, nw)
        ev[3].record()
        torch.cuda.synchronize()
        if r > 0:
            for i, key in enumerate(times):
                times[key].append(ev[i].elapsed_time(ev[i + 1]))
    med = {k: float(np.median(v)) for k, v in times.items()}
    total = sum(med.values())
    conv_bytes = T * (2 * (2 * HK + HV) * D * 2 + 2 * HV * 4 * 2)
    norm_bytes = T * (HV * D * 4 + 2 * HV * D * 2)
    return dict(tokens=T, ms=med, tokens_per_s=T / (total * 1e-3),
                front_GBps=conv_bytes / (med["front"] * 1e-3) / 1e9,
                norm_GBps=norm_bytes / (med["norm"] * 1e-3) / 1e9,
                recurrence_tokens_per_s=T / (med["recurrence"] * 1e-3))


def bench_layer(reps: int = 5):
    """One whole delta layer's prefill on a 32768-token sequence with synthetic
    weights (hidden 5120): in-projection GEMM (5120 -> q|k|v 10240, z 6144,
    b 48, a 48), conv front, chunked recurrence, gated RMS norm, out-projection
    GEMM (6144 -> 5120), as gdr_delta_layer_fwd.  Stage times come from the
    same five steps called one by one (HIP events on the launch stream).  The
    projections' rate is set against the bf16 matrix-core peak; torch.matmul
    on the same operands (hipBLASLt) is timed beside them as a reference."""
    import torch
    import gated_delta_rule_amd as gdr
    from inputs import synth
    dev = torch.device("cuda:0")
    T, H = T_CALL, synth.HIDDEN
    Cq, V = (2 * HK + HV) * D, HV * D
    log(f"layer: T={T}, hidden={H}, generating synthetic weights")
    L = synth.layer_inputs(6, lengths=(T,))
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    hid, w_in, w_out, cw = bf(L.hidden), bf(L.w_in), bf(L.w_out), bf(L.conv_w)
    Al, dtb, nw = f32(L.A_log), f32(L.dt_bias), f32(L.norm_w)
    cu = torch.from_numpy(L.cu_seqlens.astype(np.int32)).to(dev)
    del L
    st = torch.zeros((1, HV, D, D), device=dev)
    out = torch.empty((T, H), device=dev, dtype=torch.bfloat16)
    ws = gdr.delta_layer_workspace(T, 1, H, HK, HV, D, device=dev)
    chunk_ws = gdr.chunk_workspace(torch.empty((1, T, HK, D), device=dev, dtype=torch.bfloat16),
                                   torch.empty((1, T, HV, D), device=dev, dtype=torch.bfloat16), cu)

    def layer():
        gdr.delta_layer_fwd(hid, w_in, cw, Al, dtb, nw, w_out, cu, HK, HV, D, initial_state=st,
                            final_state=st, out=out, workspace=ws)

    for _ in range(2):
        layer()
    torch.cuda.synchronize()
    start, end = _events()
    start.record()
    for _ in range(reps):
        layer()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps

    names = ("in_proj", "front", "recurrence", "norm", "out_proj")
    acc = {n: 0.0 for n in names}
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record()
        qkv, z, b, a = gdr.linear(hid, w_in, blocks=[(Cq, torch.bfloat16), (V, torch.bfloat16),
                                                     (HV, torch.float32, True), (HV, torch.float32, True)])
        ev[1].record()
        q, k, v, g, beta, _ = gdr.conv_gate_fused(qkv, cw, cu, a, b, Al, dtb, HK, HV, D)
        ev[2].record()
        o, _ = gdr.chunk_gated_delta_rule(q, k, v, g, beta, st, cu_seqlens=cu, final_state=st, workspace=chunk_ws)
        ev[3].record()
        y = gdr.gated_rmsnorm(o[0], z, nw)
        ev[4].record()
        gdr.linear(y, w_out)
        ev[5].record()
        torch.cuda.synchronize()
        for i, n in enumerate(names):
            acc[n] += ev[i].elapsed_time(ev[i + 1]) / reps
        del qkv, z, b, a, q, k, v, g, beta, o, y

    def mm_ms(x, w):
        wt = w.t()
        for _ in range(2):
            torch.matmul(x, wt)
        torch.cuda.synchronize()
        s0, s1 = _events()
        s0.record()
        for _ in range(reps):
            torch.matmul(x, wt)
        s1.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / reps

    ref_in = mm_ms(hid, w_in)
    y = torch.empty((T, V), device=dev, dtype=torch.bfloat16).normal_()
    ref_out = mm_ms(y, w_out)
    f_in = 2.0 * T * (Cq + V + 2 * HV) * H
    f_out = 2.0 * T * V * H
    tf = lambda f, t: f / (t * 1e-3) / 1e12
    gemm_tf = tf(f_in + f_out, acc["in_proj"] + acc["out_proj"])
    return dict(tokens_per_s=T / (ms * 1e-3), ms=ms, stages_ms=acc,
                gemm={"in_proj_TFLOPs": tf(f_in, acc["in_proj"]), "out_proj_TFLOPs": tf(f_out, acc["out_proj"]),
                      "TFLOPs": gemm_tf, "frac_bf16_peak": gemm_tf / BF16_PEAK_TFLOPS,
                      "hipblaslt_in_proj_TFLOPs": tf(f_in, ref_in), "hipblaslt_out_proj_TFLOPs": tf(f_out, ref_out)},
                config={"T": T, "hidden": H, "num_k_heads": HK, "num_v_heads": HV, "head_dim": D,
                        "weights": "synthetic, N(0, 1/fan_in)"})


def bench_attention(reps: int = 5, dec_steps: int = 20):
    """The global attention layer (24 query / 4 kv heads, d 256): causal
    prefill of one 32768-token sequence (q/k norm + rotary, attention, gate),
    as matrix-core work 4 Hq d T^2 / 2 against the bf16 peak, beside torch's
    scaled_dot_product_attention on the same shapes (no norm, rotary or
    gate); and one decode token for 64 sequences against 32768-slot caches
    filled to 32 000+ tokens, as KV-cache bytes read per step against HBM."""
    import torch
    import gated_delta_rule_amd as gdr
    from inputs import synth
    dev = torch.device("cuda:0")
    Hq, Hk, Da = synth.ATTN_HQ, synth.ATTN_HK, synth.ATTN_D
    T = T_CALL
    log(f"attention: prefill T={T}, decode N=64 x 32768-slot caches")
    gen = torch.Generator(device=dev).manual_seed(52)
    rnd = lambda *sh: torch.randn(sh, device=dev, generator=gen).to(torch.bfloat16)
    q, k, v, g = rnd(T, Hq, Da), rnd(T, Hk, Da), rnd(T, Hk, Da), rnd(T, Hq, Da)
    w = torch.ones(Da, device=dev)
    cu = torch.tensor([0, T], device=dev, dtype=torch.int32)
    out = torch.empty_like(q)
    d = gdr.ops.attn_desc(T, 1, Hq, Hk, Da)
    import ctypes
    nb = ctypes.c_size_t(0)
    gdr.load_library().gdr_attn_prefill_workspace_size(ctypes.byref(d), ctypes.byref(nb))
    ws = torch.empty(nb.value, device=dev, dtype=torch.uint8)

    def timed(fn, n):
        for _ in range(4):  # untimed, until the clocks have settled
            fn()
        torch.cuda.synchronize()
        s0, s1 = _events()
        s0.record()
        for _ in range(n):
            fn()
        s1.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / n

    ms = timed(lambda: gdr.attn_prefill(q, k, v, g, w, w, cu, out=out, workspace=ws), reps)
    flop = 4.0 * Hq * Da * T * T / 2
    qq = q.permute(1, 0, 2).unsqueeze(0)
    kk = k.permute(1, 0, 2).unsqueeze(0).repeat_interleave(Hq // Hk, dim=1)
    vv = v.permute(1, 0, 2).unsqueeze(0).repeat_interleave(Hq // Hk, dim=1)
    try:
        ms_ref = timed(lambda: torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True), reps)
    except Exception:  # a reference only
        ms_ref = None
    del qq, kk, vv, q, k, v, g, out, ws

    N, L = 64, 32768
    kc = torch.randn((N, L, Hk, Da), device=dev, generator=gen).to(torch.bfloat16)
    vc = torch.randn((N, Hk, L // 32, Da, 32), device=dev, generator=gen).to(torch.bfloat16)
    lens = torch.randint(32000, L - dec_steps, (N,), device=dev, generator=gen, dtype=torch.int32)
    qd, kd, vd, gd = rnd(N, Hq, Da), rnd(N, Hk, Da), rnd(N, Hk, Da), rnd(N, Hq, Da)
    od = torch.empty_like(qd)
    dd = gdr.ops.attn_desc(N, N, Hq, Hk, Da, L)
    gdr.load_library().gdr_attn_decode_workspace_size(ctypes.byref(dd), ctypes.byref(nb))
    wsd = torch.empty(nb.value, device=dev, dtype=torch.uint8)
    ms_dec = timed(lambda: gdr.attn_decode(qd, kd, vd, gd, w, w, kc, vc, lens, out=od, workspace=wsd), dec_steps)
    cache_bytes = float((lens.to(torch.int64) + 1).sum().item()) * Hk * Da * 2 * 2
    return dict(prefill={"T": T, "ms": ms, "tokens_per_s": T / (ms * 1e-3),
                         "TFLOPs": flop / (ms * 1e-3) / 1e12,
                         "frac_bf16_peak": flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                         "torch_sdpa_ms": ms_ref},
                decode={"N": N, "cache_len": L, "us_per_step": ms_dec * 1e3,
                        "kv_GBps": cache_bytes / (ms_dec * 1e-3) / 1e9,
                        "frac_hbm": cache_bytes / (ms_dec * 1e-3) / 1e9 / HBM_PEAK_GBS},
                config={"num_q_heads": Hq, "num_kv_heads": Hk, "head_dim": Da, "rotary_dims": 64,
                        "rope_base": 1e7})


def bench_copy(n_bytes: int = 1 << 30, reps: int = 5):
    """Plain device copy of known size: calibration of the HBM byte counters."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(n_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    start, end = _events()
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    return dict(bytes_each_way=n_bytes, ms=ms, GBps=2 * n_bytes / (ms * 1e-3) / 1e9)


def cpu_baseline(host_calls):
    """The fp64 oracle on the first three 32K calls of the same long-context
    workload (state carried from call to call), heads spread over the host's
    cores.  Input generation is not timed."""
    from oracle import gdr as ref
    procs = len(os.sched_getaffinity(0))
    log(f"cpu baseline: fp64 oracle, {len(host_calls)} x {T_CALL} tokens, 48 heads, {procs} processes")
    state, dt, used = None, 0.0, procs
    for x in host_calls:
        t0 = time.perf_counter()
        _, state, used = ref.forward_parallel(x.q, x.k, x.v, x.g, x.beta, state, processes=procs)
        dt += time.perf_counter() - t0
    tokens = len(host_calls) * T_CALL
    return dict(value=tokens / dt, unit="tokens/s", cores=used, kind="oracle",
                sample=f"fp64 token-serial oracle on the first {len(host_calls)} 32768-token calls of the same "
                       f"16/48-head d=128 long-context workload, state carried between calls, heads spread "
                       f"over {used} processes: {tokens} tokens in {dt:.1f} s wall")


def _decode_worker(args):
    from oracle import gdr as ref
    steps, lo, hi, s0 = args
    s = s0
    for xi in steps:
        _, s = ref.decode_step(xi.q[lo:hi], xi.k[lo:hi], xi.v[lo:hi], xi.g[lo:hi], xi.beta[lo:hi], s)
    return s


def cpu_baseline_decode(steps: int = 4, N: int = 64):
    """The fp64 oracle's decode step on the decode workload (64 sequences x 48
    heads, 128x128 state), 4 steps, sequences spread over the host's cores."""
    import multiprocessing as mp
    from inputs import synth
    procs = min(len(os.sched_getaffinity(0)), N)
    _, _, s0 = synth.decode_inputs(N=N)
    xs = [synth.decode_step_inputs(t, N=N) for t in range(steps)]
    bounds = np.linspace(0, N, procs + 1).astype(int)
    jobs = [(xs, int(a), int(b), s0[a:b]) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    log(f"cpu baseline: fp64 oracle decode, {steps} steps of {N}x{HV} states, {len(jobs)} processes")
    with mp.get_context("fork").Pool(len(jobs)) as pool:
        t0 = time.perf_counter()
        pool.map(_decode_worker, jobs)
        dt = time.perf_counter() - t0
    state_bytes = 2 * N * HV * D * D * 4 * steps
    return dict(value=state_bytes / dt / 1e9, unit="GB/s (fp32 state bytes)", cores=len(jobs), kind="oracle",
                sample=f"fp64 oracle decode step, {steps} steps of {N} sequences x {HV} heads (128x128 state), "
                       f"sequences spread over {len(jobs)} processes: {dt:.2f} s wall")


def traffic_from_counters():
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel source."""
    if not os.path.exists(COUNTERS):
        return None, None
    rec = json.load(open(COUNTERS))
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None, "stale"
    return rec.get("hbm_bytes_per_launch"), "ok"


def main():
    global N_CALLS
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=24)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--only", default="all", choices=["all", "prefill", "decode", "decode_layer", "pipeline", "layer",
                                                      "attention", "copy", "roofline"])
    ap.add_argument("--pieces", type=int, default=N_CALLS,
                    help="distinct 32K pieces of the context to cycle through (8 = the whole 262144 tokens)")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    N_CALLS = max(1, min(args.pieces, 8))
    out = {}
    if args.only == "copy":
        print(json.dumps({"copy": bench_copy()}), flush=True)
        return
    if args.only == "roofline":
        print(json.dumps({"achievable": bench_roofline()}), flush=True)
        return
    clocks_before = gpu_clocks()
    host_calls = []
    if args.only in ("all", "prefill"):
        log(f"prefill: generating {N_CALLS} x {T_CALL}-token pieces")
        host_calls = long_context_host(N_CALLS)
        pf = bench_prefill(args.steps, args.warmup, host_calls)
        del host_calls[3:]
        ms_step = pf["total_ms"] / args.steps
        avg_launch_ms = float(np.mean(pf["recur_ms"]))
        bytes_launch = T_CALL * RECUR_BYTES_PER_TOKEN + 2 * STATE_BYTES
        achieved = bytes_launch / (avg_launch_ms * 1e-3) / 1e9
        flops_launch = RECUR_FLOP_PER_TOKEN * T_CALL
        call_bytes = T_CALL * PREFILL_BYTES_PER_TOKEN + 2 * STATE_BYTES
        traffic, tstat = traffic_from_counters()
        tok_s = T_CALL * args.steps / (pf["total_ms"] * 1e-3)
        last_pass = pf["call_ms"][-N_CALLS:] if args.steps >= N_CALLS else None
        out.update({
            "metric": "prefill tokens/s per delta layer (T=32K) + decode state-update HBM GB/s",
            "value": tok_s,
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": ms_step,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"delta-layer chunked prefill of a {N_CALLS * T_CALL}-token context as "
                                   f"{N_CALLS} consecutive 32768-token calls with state resume",
                       "B": 1, "T_per_call": T_CALL, "calls": N_CALLS, "num_k_heads": HK, "num_v_heads": HV, "head_dim": D,
                       "chunk": C, "qkv": "bf16", "gates_state_out": "fp32", "parallelism": "single GPU"},
            # the target is framed against the bf16 matrix-core bound, so the
            # headline roofline is the recurrence kernel's algorithmic MFMA
            # rate; its HBM rate and the whole call's MFMA fraction (prepare
            # included) sit beside it
            "roofline": {"bound": "mfma", "achieved": flops_launch / (avg_launch_ms * 1e-3) / 1e12,
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": flops_launch / (avg_launch_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                         "traffic": traffic,
                         "kernel": RECUR_KERNEL, "avg_launch_ms": avg_launch_ms,
                         "algorithmic_flops_per_launch": flops_launch,
                         "call_mfma_frac": PREFILL_FLOP_PER_TOKEN * T_CALL / (ms_step * 1e-3) / 1e12
                         / BF16_PEAK_TFLOPS,
                         "hbm": {"achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": bytes_launch}},
            "call": {"prepare_ms": float(np.mean(pf["prep_ms"])), "recurrence_ms": avg_launch_ms,
                     "median_ms": float(np.median(pf["call_ms"])),
                     "context_ms": float(np.sum(last_pass)) if last_pass else None,
                     "hbm_frac": call_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "mfma_frac": PREFILL_FLOP_PER_TOKEN * T_CALL / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
            "finite": pf["finite"],
        })
        if tstat == "stale":
            out["roofline"]["traffic_note"] = "counters predate the current kernel source"
    if args.only in ("all", "decode"):
        out["decode"] = bench_decode()
        if args.only == "all":
            out["decode_2_replicas"] = bench_decode(replicas=2)
            out["decode_pool_indexed"] = bench_decode(pool=128)
            out["decode_pool_in_order"] = bench_decode(pool=128, shuffled=False)
            out["decode_layer"] = bench_decode_layer()
    if args.only == "decode_layer":
        out["decode_layer"] = bench_decode_layer()
    if args.only in ("all", "pipeline"):
        out["pipeline"] = bench_pipeline()
    if args.only in ("all", "layer"):
        out["layer"] = bench_layer()
    if args.only in ("all", "attention"):
        out["attention"] = bench_attention()
    if args.only == "all":
        ach = bench_roofline()
        out["achievable"] = ach
        if "roofline" in out:
            out["roofline"]["frac_of_achievable"] = out["roofline"]["achieved"] / ach["mfma_bf16_TFLOPs"]
            out["roofline"]["hbm"]["frac_of_achievable"] = (out["roofline"]["hbm"]["achieved"]
                                                            / ach["hbm_rmw_nontemporal_GBps"])
        for key in ("decode", "decode_2_replicas", "decode_pool_indexed", "decode_pool_in_order", "decode_layer"):
            if key in out:
                out[key]["frac_of_achievable"] = out[key]["state_GBps"] / ach["hbm_rmw_nontemporal_GBps"]
    out["clocks"] = {"before": clocks_before, "after": gpu_clocks()}
    if args.only == "all" and not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(host_calls[:3] if host_calls else long_context_host(3))
        out["cpu_baseline_decode"] = cpu_baseline_decode()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
