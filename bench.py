#!/usr/bin/env python3
"""Throughput of the gated delta rule path on one MI355X.

A step is one 32768-token chunked-prefill call of one delta layer
(16 key / 48 value heads, d = 128, bf16 q/k/v, fp32 gates, state and output,
chunk 64) that resumes from the previous call's final state -- the shape of
one call of a 262144-token context processed in 32K pieces.  ``value`` is the
prefill rate in tokens/s over the K timed steps.  The same JSON line also
reports, measured in the same run:

  decode    -- 64 sequences x 48 heads of 128x128 fp32 state, one token per
               step, state updated in place, 256 steps: state GB/s
  pipeline  -- the whole layer path over a packed batch of 8 sequences
               (65536 tokens): conv+SiLU+gates, recurrence, gated RMSNorm
  roofline  -- the dominant kernel of the call, the state-carrying
               recurrence (gdr_chunk_fwd_recurrence): its algorithmic HBM bytes
               per launch (q, k, v read, o written, state in and out) over its
               average launch time (HIP events on the launch stream, around
               each recurrence launch inside the timed loop), against the
               8 TB/s HBM peak; plus its MFMA fraction and the HBM bytes the
               committed rocprofv3 counters measured for it
  cpu_baseline -- the fp64 CPU oracle timed on the host cores on a bounded
               sample of the same workload (the first three 32K-token calls)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only prefill|decode|pipeline|copy|all]
                       [--no-cpu]
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


def bench_prefill(steps: int, warmup: int):
    import torch
    import gated_delta_rule_amd as gdr
    from gated_delta_rule_amd import synth
    dev = torch.device("cuda:0")
    log(f"prefill: generating T={T_CALL} inputs")
    x = synth.long_context_call(0, T=T_CALL)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    q, k, v = bf(x.q), bf(x.k), bf(x.v)
    g, beta = f32(x.g), f32(x.beta)
    state = torch.zeros((1, HV, D, D), device=dev)
    o = torch.empty((1, T_CALL, HV, D), device=dev)
    ws = gdr.chunk_workspace(q, v)
    del x

    # One call = gdr_chunk_fwd_prepare + gdr_chunk_fwd_recurrence on the torch
    # stream (the same kernels gdr_chunk_fwd enqueues), so that events can
    # bracket the recurrence kernel alone.
    def stage(name):
        gdr.chunk_gated_delta_rule(q, k, v, g, beta, state, final_state=state, out=o, workspace=ws, stage=name)

    log(f"prefill: {warmup} warmup + {steps} timed 32K calls")
    for _ in range(warmup):
        stage("prepare")
        stage("recurrence")
    torch.cuda.synchronize()
    per = []
    t0 = time.perf_counter()
    start, end = _events()
    start.record()
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        stage("prepare")
        e[1].record()
        stage("recurrence")
        e[2].record()
        per.append(e)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    prep_ms = [e[0].elapsed_time(e[1]) for e in per]
    recur_ms = [e[1].elapsed_time(e[2]) for e in per]
    finite = bool(torch.isfinite(state).all() and torch.isfinite(o).all())
    return dict(total_ms=total_ms, wall_s=wall, prep_ms=prep_ms, recur_ms=recur_ms, finite=finite)


def bench_decode(steps: int = 256, replicas: int = 1):
    import torch
    import gated_delta_rule_amd as gdr
    from gated_delta_rule_amd import synth
    dev = torch.device("cuda:0")
    N = 64
    log(f"decode: N={N}, {steps} steps, {replicas} state replica(s)")
    A_log, dt, s0 = synth.decode_inputs(N=N)
    states = [torch.from_numpy(s0).to(dev) for _ in range(replicas)]
    del s0
    inputs = []
    for s in range(steps):
        xi = synth.decode_step_inputs(s, N=N)
        inputs.append((torch.from_numpy(xi.q).to(torch.bfloat16).to(dev),
                       torch.from_numpy(xi.k).to(torch.bfloat16).to(dev),
                       torch.from_numpy(xi.v).to(torch.bfloat16).to(dev),
                       torch.from_numpy(xi.g).to(dev), torch.from_numpy(xi.beta).to(dev)))
    o = torch.empty((N, HV, D), device=dev)
    for i in range(8):  # warmup
        gdr.recurrent_step(*inputs[i], states[i % replicas], out=o)
    torch.cuda.synchronize()
    start, end = _events()
    start.record()
    for i in range(steps):
        gdr.recurrent_step(*inputs[i], states[i % replicas], out=o)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    state_bytes = 2 * N * HV * D * D * 4
    other = N * (2 * HK * D * 2 + HV * D * 2 + 2 * HV * 4 + HV * D * 4)
    return dict(us_per_step=ms * 1e3, state_GBps=state_bytes / (ms * 1e-3) / 1e9,
                total_GBps=(state_bytes + other) / (ms * 1e-3) / 1e9,
                frac_hbm=state_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, working_set_MiB=replicas * state_bytes / 2 / 2**20)


def bench_pipeline(reps: int = 5):
    import torch
    import gated_delta_rule_amd as gdr
    from gated_delta_rule_amd import synth
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


def cpu_baseline(calls: int = 3):
    """The fp64 oracle on the first ``calls`` 32K-token calls of the same
    long-context workload (state carried from call to call), heads spread over
    the host's cores.  Input generation is not timed."""
    from gated_delta_rule_amd import synth
    from oracle import gdr as ref
    procs = len(os.sched_getaffinity(0))
    log(f"cpu baseline: fp64 oracle, {calls} x {T_CALL} tokens, 48 heads, {procs} processes")
    state, dt, used = None, 0.0, procs
    for i in range(calls):
        x = synth.long_context_call(i, T=T_CALL)
        t0 = time.perf_counter()
        _, state, used = ref.forward_parallel(x.q, x.k, x.v, x.g, x.beta, state, processes=procs)
        dt += time.perf_counter() - t0
        del x
    tokens = calls * T_CALL
    return dict(value=tokens / dt, unit="tokens/s", cores=used, kind="oracle",
                sample=f"fp64 token-serial oracle on the first {calls} 32768-token calls of the same "
                       f"16/48-head d=128 long-context workload, state carried between calls, heads spread "
                       f"over {used} processes: {tokens} tokens in {dt:.1f} s wall")


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
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default="all", choices=["all", "prefill", "decode", "pipeline", "copy"])
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
    out = {}
    if args.only == "copy":
        print(json.dumps({"copy": bench_copy()}), flush=True)
        return
    if args.only in ("all", "prefill"):
        pf = bench_prefill(args.steps, args.warmup)
        ms_step = pf["total_ms"] / args.steps
        avg_launch_ms = float(np.mean(pf["recur_ms"]))
        bytes_launch = T_CALL * RECUR_BYTES_PER_TOKEN + 2 * STATE_BYTES
        achieved = bytes_launch / (avg_launch_ms * 1e-3) / 1e9
        call_bytes = T_CALL * PREFILL_BYTES_PER_TOKEN + 2 * STATE_BYTES
        traffic, tstat = traffic_from_counters()
        tok_s = T_CALL * args.steps / (pf["total_ms"] * 1e-3)
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
            "config": {"workload": "delta-layer chunked prefill, 32768-token calls with state resume",
                       "B": 1, "T_per_call": T_CALL, "num_k_heads": HK, "num_v_heads": HV, "head_dim": D,
                       "chunk": C, "qkv": "bf16", "gates_state_out": "fp32", "parallelism": "single GPU"},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                         "kernel": RECUR_KERNEL, "avg_launch_ms": avg_launch_ms,
                         "algorithmic_bytes_per_launch": bytes_launch,
                         "mfma_frac": RECUR_FLOP_PER_TOKEN * T_CALL / (avg_launch_ms * 1e-3) / 1e12
                         / BF16_PEAK_TFLOPS},
            "call": {"prepare_ms": float(np.mean(pf["prep_ms"])), "recurrence_ms": avg_launch_ms,
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
    if args.only in ("all", "pipeline"):
        out["pipeline"] = bench_pipeline()
    if args.only == "all" and not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
