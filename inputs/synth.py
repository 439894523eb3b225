"""Seeded synthetic inputs for the gated delta rule path.

Every array the tests, the benchmark and the smoke check feed to either the
HIP library or the CPU oracle comes from here, so both sides see bit-identical
values.  This module holds no step of the method: it only draws random numbers
and shapes their distributions the way the workload recipe states them
(unit-norm q/k, logistic-normal beta, softplus-shaped log-decay g).  The gate
*step* of the path (beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias),
computed from raw projections) lives in the conv-front kernel and in the
oracle; for that path the generator hands out the raw draws a and b.

Recipe (per value head: A_log ~ U(0, ln 16), dt_bias ~ U(-1, 1); per token:
q, k ~ N(0, 1) then L2-normalised, v ~ N(0, 1), beta = sigmoid(N(0, 1)),
g = -exp(A_log) * softplus(N(0, 1) + dt_bias)).  The head geometry (16 key
heads, 48 value heads, head dim 128, chunk 64) is the delta-rule layer shape
given on the Agnes-3.0-Flash pages ("architecture" section of the model-card
write-up).

Values destined for bf16 are drawn in float64, rounded to float32 and then
rounded to nearest-even bf16; they are returned as float32 arrays that hold
exactly representable bf16 values, so ``torch.from_numpy(a).to(bfloat16)`` is
exact.  numpy's PCG64 generator is used throughout; the draw order inside each
function is fixed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "rng",
    "round_bf16",
    "GDRInputs",
    "gdr_inputs",
    "tiny_config",
    "layer_prefill",
    "long_context_call",
    "decode_inputs",
    "decode_step_inputs",
    "varlen_lengths",
    "pipeline_inputs",
    "matmul_inputs",
    "LayerInputs",
    "layer_inputs",
    "HIDDEN",
    "AttnInputs",
    "attn_inputs",
    "HK",
    "HV",
    "D",
]

HK, HV, D = 16, 48, 128


def rng(*seed: int) -> np.random.Generator:
    """PCG64 generator for a tuple of integer seeds."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to float32, then to nearest-even bf16; returned as float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).reshape(f.shape)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


@dataclass
class GDRInputs:
    """Inputs of one chunked-prefill or decode call (numpy, host side)."""

    q: np.ndarray  # [B, T, Hk, dk]   (decode: [N, Hk, dk])
    k: np.ndarray
    v: np.ndarray  # [B, T, Hv, dv]   (decode: [N, Hv, dv])
    g: np.ndarray  # [B, T, Hv] float32 log-decay (<= 0)
    beta: np.ndarray  # [B, T, Hv] float32 in (0, 1)
    A_log: np.ndarray  # [Hv]
    dt_bias: np.ndarray  # [Hv]
    dtype: str  # "bf16" or "f32": storage type of q, k, v
    chunk_size: int = 64
    initial_state: Optional[np.ndarray] = None  # [N, Hv, dv, dk] float32
    cu_seqlens: Optional[np.ndarray] = None  # [N+1] int32
    meta: dict = field(default_factory=dict)

    @property
    def num_k_heads(self) -> int:
        return self.q.shape[-2]

    @property
    def num_v_heads(self) -> int:
        return self.v.shape[-2]


def _head_params(g: np.random.Generator, hv: int):
    A_log = g.uniform(0.0, math.log(16.0), size=hv)
    dt_bias = g.uniform(-1.0, 1.0, size=hv)
    return A_log.astype(np.float32), dt_bias.astype(np.float32)


def _token_draws(gen, lead, hk, hv, dk, dv, dtype, A_log, dt_bias):
    q = _cast(_unit(gen.standard_normal(lead + (hk, dk))), dtype)
    k = _cast(_unit(gen.standard_normal(lead + (hk, dk))), dtype)
    v = _cast(gen.standard_normal(lead + (hv, dv)), dtype)
    b_raw = gen.standard_normal(lead + (hv,))
    a_raw = gen.standard_normal(lead + (hv,))
    beta = (1.0 / (1.0 + np.exp(-b_raw))).astype(np.float32)
    g = (-np.exp(A_log.astype(np.float64)) * _softplus(a_raw + dt_bias.astype(np.float64))).astype(np.float32)
    return q, k, v, g, beta


def gdr_inputs(
    seed: int,
    *,
    B: int = 1,
    T: int,
    hk: int = HK,
    hv: int = HV,
    d: int = D,
    dtype: str = "bf16",
    chunk_size: int = 64,
    initial_state_std: Optional[float] = None,
    head_seed: Optional[int] = None,
) -> GDRInputs:
    """Prefill inputs [B, T, heads, d] drawn by the workload recipe.

    ``head_seed`` selects the stream of the per-head parameters (A_log,
    dt_bias) so that several calls of one long sequence can share them.
    """
    hgen = rng(seed if head_seed is None else head_seed, 0)
    A_log, dt_bias = _head_params(hgen, hv)
    gen = rng(seed, 1)
    q, k, v, g, beta = _token_draws(gen, (B, T), hk, hv, d, d, dtype, A_log, dt_bias)
    s0 = None
    if initial_state_std is not None:
        s0 = (initial_state_std * rng(seed, 2).standard_normal((B, hv, d, d))).astype(np.float32)
    return GDRInputs(q, k, v, g, beta, A_log, dt_bias, dtype, chunk_size, s0)


def tiny_config() -> GDRInputs:
    """B=1, T=128, 2 key / 6 value heads, d=32, chunk 32, all fp32, zero state."""
    return gdr_inputs(1, B=1, T=128, hk=2, hv=6, d=32, dtype="f32", chunk_size=32)


def layer_prefill(T: int = 4096, seed: int = 2) -> GDRInputs:
    """One delta layer's prefill, 16/48 heads, d=128, bf16 q/k/v, zero state."""
    return gdr_inputs(seed, B=1, T=T, dtype="bf16", chunk_size=64)


def long_context_call(i: int, T: int = 32768) -> GDRInputs:
    """Call ``i`` of a long sequence processed as consecutive T-token calls.

    Call i draws its tokens from seed 4*1000 + i; the per-head gate parameters
    are shared by all calls (seed 4).
    """
    return gdr_inputs(4 * 1000 + i, B=1, T=T, dtype="bf16", chunk_size=64, head_seed=4)


def decode_inputs(N: int = 64, hk: int = HK, hv: int = HV, d: int = D, dtype: str = "bf16",
                  state_std: float = 0.05, seed: int = 3):
    """Per-head gate parameters and the seeded fp32 initial state [N, Hv, d, d]."""
    A_log, dt_bias = _head_params(rng(seed, 0), hv)
    s0 = (state_std * rng(seed, 2).standard_normal((N, hv, d, d))).astype(np.float32)
    return A_log, dt_bias, s0


def decode_step_inputs(step: int, N: int = 64, hk: int = HK, hv: int = HV, d: int = D,
                       dtype: str = "bf16", seed: int = 3) -> GDRInputs:
    """Fresh single-token inputs of decode step ``step`` (q, k: [N, Hk, d])."""
    A_log, dt_bias = _head_params(rng(seed, 0), hv)
    gen = rng(seed, 100 + step)
    q, k, v, g, beta = _token_draws(gen, (N,), hk, hv, d, d, dtype, A_log, dt_bias)
    return GDRInputs(q, k, v, g, beta, A_log, dt_bias, dtype, 1)


def varlen_lengths(seed: int = 5, n: int = 8, total: int = 65536, floor: int = 1024,
                   cap: int = 32768) -> np.ndarray:
    """Sequence lengths >= floor and <= cap summing to ``total``.

    n-1 sorted uniform integer cut points split total - n*floor; each gap is
    added to the floor.  Redrawn until every length is <= cap.
    """
    gen = rng(seed, 3)
    span = total - n * floor
    while True:
        cuts = np.sort(gen.integers(0, span + 1, size=n - 1))
        gaps = np.diff(np.concatenate([[0], cuts, [span]]))
        lens = floor + gaps
        if lens.max() <= cap:
            return lens.astype(np.int64)


def cu_seqlens_of(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


@dataclass
class PipelineInputs:
    """Inputs of the full delta-layer path (conv front, recurrence, norm)."""

    x: np.ndarray  # [T, Cq+Ck+Cv] bf16-valued float32 (q | k | v channel blocks)
    conv_w: np.ndarray  # [C, 4] bf16-valued float32; tap 3 multiplies the current token
    a: np.ndarray  # [T, Hv] float32 raw decay projection
    b: np.ndarray  # [T, Hv] float32 raw write-strength projection
    A_log: np.ndarray  # [Hv] float32
    dt_bias: np.ndarray  # [Hv] float32
    z: np.ndarray  # [T, Hv*dv] bf16-valued float32 gate of the output norm
    norm_w: np.ndarray  # [dv] float32
    cu_seqlens: np.ndarray  # [N+1] int32
    hk: int
    hv: int
    d: int


def pipeline_inputs(seed: int = 5, *, lengths=None, hk: int = HK, hv: int = HV, d: int = D,
                    n: int = 8, total: int = 65536) -> PipelineInputs:
    """Packed varlen batch for the whole delta-layer path.

    Default: 8 sequences, lengths in [1024, 32768], 65536 tokens in total,
    10240 conv channels (2*16*128 + 48*128) and 6144 gated-norm channels.
    """
    if lengths is None:
        lengths = varlen_lengths(seed, n=n, total=total)
    cu = cu_seqlens_of(lengths)
    T = int(cu[-1])
    C = 2 * hk * d + hv * d
    hgen = rng(seed, 0)
    A_log, dt_bias = _head_params(hgen, hv)
    gen = rng(seed, 1)
    x = round_bf16(gen.standard_normal((T, C), dtype=np.float32))
    conv_w = round_bf16(gen.uniform(-0.5, 0.5, size=(C, 4)))
    a = gen.standard_normal((T, hv), dtype=np.float32)
    b = gen.standard_normal((T, hv), dtype=np.float32)
    z = round_bf16(gen.standard_normal((T, hv * d), dtype=np.float32))
    norm_w = (1.0 + 0.1 * gen.standard_normal(d)).astype(np.float32)
    return PipelineInputs(x, conv_w, a, b, A_log, dt_bias, z, norm_w, cu, hk, hv, d)


HIDDEN = 5120  # model width of the pages' layer


def matmul_inputs(seed: int, M: int, N: int, K: int):
    """x [M, K] ~ N(0, 1) and w [N, K] ~ N(0, 1/K), both bf16 values (float32 arrays)."""
    gen = rng(seed, 20)
    x = round_bf16(gen.standard_normal((M, K), dtype=np.float32))
    w = round_bf16(gen.standard_normal((N, K), dtype=np.float32) / np.float32(math.sqrt(K)))
    return x, w


@dataclass
class LayerInputs:
    hidden: np.ndarray   # [T, H] bf16 values
    w_in: np.ndarray     # [C + V + 2 hv, H] bf16 values: rows q|k|v, z, b, a
    conv_w: np.ndarray   # [C, 4] bf16 values
    A_log: np.ndarray    # [hv]
    dt_bias: np.ndarray  # [hv]
    norm_w: np.ndarray   # [d]
    w_out: np.ndarray    # [H, V] bf16 values
    cu_seqlens: np.ndarray
    hk: int
    hv: int
    d: int


def layer_inputs(seed: int = 6, *, lengths=(4096,), hk: int = HK, hv: int = HV, d: int = D,
                 hidden: int = HIDDEN) -> LayerInputs:
    """Synthetic weights and activations of one whole delta layer.

    hidden ~ N(0, 1); projection weights ~ N(0, 1/fan_in), so every projection
    output is about N(0, 1) like the activations the path recipe draws; conv
    weights ~ U(-0.5, 0.5), per-head A_log / dt_bias as in the path recipe,
    norm weight 1 + 0.1 N(0, 1).  No trained values are involved.
    """
    cu = cu_seqlens_of(list(lengths))
    T = int(cu[-1])
    C, V = (2 * hk + hv) * d, hv * d
    A_log, dt_bias = _head_params(rng(seed, 0), hv)
    gen = rng(seed, 21)
    x = round_bf16(gen.standard_normal((T, hidden), dtype=np.float32))
    w_in = round_bf16(gen.standard_normal((C + V + 2 * hv, hidden), dtype=np.float32)
                      / np.float32(math.sqrt(hidden)))
    conv_w = round_bf16(gen.uniform(-0.5, 0.5, size=(C, 4)))
    norm_w = (1.0 + 0.1 * gen.standard_normal(d)).astype(np.float32)
    w_out = round_bf16(gen.standard_normal((hidden, V), dtype=np.float32) / np.float32(math.sqrt(V)))
    return LayerInputs(x, w_in, conv_w, A_log, dt_bias, norm_w, w_out, cu, hk, hv, d)


ATTN_HQ, ATTN_HK, ATTN_D = 24, 4, 256  # the global attention layer's heads


@dataclass
class AttnInputs:
    q: np.ndarray       # [T, Hq, D] bf16 values
    k: np.ndarray       # [T, Hk, D]
    v: np.ndarray       # [T, Hk, D]
    gate: np.ndarray    # [T, Hq, D]
    q_norm_w: np.ndarray  # [D]
    k_norm_w: np.ndarray  # [D]
    cu_seqlens: np.ndarray


def attn_inputs(seed: int = 40, *, lengths=(4096,), hq: int = ATTN_HQ, hk: int = ATTN_HK,
                d: int = ATTN_D) -> AttnInputs:
    """Activations of the global attention layer: q, k, v and gate ~ N(0, 1)
    (the outputs of its projections), norm weights 1 + 0.1 N(0, 1)."""
    cu = cu_seqlens_of(list(lengths))
    T = int(cu[-1])
    gen = rng(seed, 30)
    q = round_bf16(gen.standard_normal((T, hq, d), dtype=np.float32))
    k = round_bf16(gen.standard_normal((T, hk, d), dtype=np.float32))
    v = round_bf16(gen.standard_normal((T, hk, d), dtype=np.float32))
    gate = round_bf16(gen.standard_normal((T, hq, d), dtype=np.float32))
    qw = (1.0 + 0.1 * gen.standard_normal(d)).astype(np.float32)
    kw = (1.0 + 0.1 * gen.standard_normal(d)).astype(np.float32)
    return AttnInputs(q, k, v, gate, qw, kw, cu)
