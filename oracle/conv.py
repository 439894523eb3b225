"""Oracle of the layer front and back around the recurrence -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module; the HIP library never does.

Follows the Agnes-3.0-Flash pages: the delta-rule layer has a kernel-4 causal
convolution in front and a gated RMS norm behind (deepmagic page,
"architecture" section; linear_conv_kernel_dim 4 in the config field list on
the mhpq page, section 2.1); the gates are beta = sigmoid(b) and
g = -exp(A_log) * softplus(a + dt_bias), computed in fp32 (yfxerp page,
section 1.2); z is 6144 wide and b, a are one value per value head (yfxerp
page, parameter ledger in section 2).

Readings where the pages are silent:
  * the conv is depthwise over all q|k|v channels, without bias; tap 3
    multiplies the current token, taps 0..2 the three previous tokens of the
    same sequence (zero, or the carried conv state, before its start);
    SiLU(x) = x * sigmoid(x) follows it on every channel;
  * the gated norm is per (token, value head) over d_v:
    y = o / sqrt(mean(o^2) + eps) * w * SiLU(z), eps = 1e-6, w shared by heads.

Two conv evaluations are given.  ``conv_silu`` is the definition in float64.
``conv_silu_fp32`` fixes the float32 evaluation that the bf16 output is
required to reproduce bit for bit: products w*x (exact for bf16 operands),
summed oldest tap first, ((p0 + p1) + p2) + p3, each add rounded to float32;
SiLU as v / (1 + exp32(-v)) with every operation a single IEEE float32
operation (no fused multiply-add) and ``exp32`` below; round to nearest even
bf16.  The tests hold ``conv_silu_fp32`` to within one bf16 ulp of
``conv_silu``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_bf16",
    "exp32",
    "silu32",
    "conv_silu",
    "conv_silu_fp32",
    "conv_state_out",
    "gates",
    "gated_rmsnorm",
]

_F = np.float32


def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 result."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    out = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = out.astype(np.uint32).view(np.float32).reshape(f.shape)
    return np.where(nan, np.float32(np.nan), out)


# Cody and Waite's argument reduction (x = n ln 2 + r, |r| <= ln2/2, with ln 2
# split as C1 + C2 so that n*C1 is exact for |n| < 2^15) followed by the Taylor
# polynomial of exp(r) to degree 7 in Horner form, scaled by 2^n.
_LOG2E = _F(1.4426950408889634)
_C1 = _F(0.693359375)  # 355/512
_C2 = _F(-2.12194440e-4)  # ln 2 - C1, rounded to float32
_TAYLOR = [_F(1.0 / f) for f in (5040.0, 720.0, 120.0, 24.0, 6.0, 2.0, 1.0, 1.0)]
_EXP_HI = _F(88.72283935546875)  # largest x with finite exp32(x)
_EXP_LO = _F(-103.97208)  # below ln(2^-150): exp32 is 0


def exp32(x) -> np.ndarray:
    """exp in float32: Cody-Waite reduction + degree-7 Taylor, one IEEE op at a time."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        n = np.rint(x * _LOG2E).astype(np.float32)
        r = (x - n * _C1) - n * _C2
        p = np.full_like(x, _TAYLOR[0])
        for c in _TAYLOR[1:]:
            p = p * r + c
        n_int = np.clip(n, -200, 200).astype(np.int32)
        y = np.ldexp(p, n_int).astype(np.float32)
    y = np.where(x > _EXP_HI, np.float32(np.inf), y)
    y = np.where(x < _EXP_LO, np.float32(0.0), y)
    return np.where(np.isnan(x), x, y).astype(np.float32)


def silu32(v) -> np.ndarray:
    """SiLU in float32: v / (1 + exp32(-v)), each op rounded to float32."""
    v = np.asarray(v, dtype=np.float32)
    with np.errstate(over="ignore"):
        return (v / (np.float32(1.0) + exp32(-v))).astype(np.float32)


def _histories(x, cu_seqlens, conv_state):
    """Yield (n, t0, t1, extended input [3 + L, C]) per sequence."""
    x = np.asarray(x)
    C = x.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for n in range(len(cu) - 1):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        hist = np.zeros((3, C), dtype=x.dtype) if conv_state is None else \
            np.asarray(conv_state[n], dtype=x.dtype).T
        yield n, t0, t1, np.concatenate([hist, x[t0:t1]], axis=0)


def conv_silu(x, w, cu_seqlens, conv_state=None) -> np.ndarray:
    """Definition in float64: y[t, c] = SiLU(sum_j w[c, j] x[t - 3 + j, c]).

    x: [T, C]; w: [C, 4]; conv_state: [N, C, 3] history, oldest first, or None.
    Returns y [T, C] float64 (not rounded).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = np.zeros_like(x)
    for _, t0, t1, xe in _histories(x, cu_seqlens, conv_state):
        L = t1 - t0
        pre = sum(w[:, j] * xe[j:j + L] for j in range(4))
        y[t0:t1] = pre / (1.0 + np.exp(-pre))
    return y


def conv_silu_fp32(x, w, cu_seqlens, conv_state=None) -> np.ndarray:
    """Fixed-order float32 evaluation, rounded to bf16 (returned as float32).

    The bit pattern of this result is the conv front's required output.
    """
    x = np.asarray(x, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    y = np.zeros_like(x)
    for _, t0, t1, xe in _histories(x, cu_seqlens, conv_state):
        L = t1 - t0
        acc = w[:, 0] * xe[0:L]
        for j in range(1, 4):
            acc = (acc + w[:, j] * xe[j:j + L]).astype(np.float32)
        y[t0:t1] = silu32(acc)
    return round_bf16(y)


def conv_state_out(x, cu_seqlens, conv_state=None) -> np.ndarray:
    """Last three inputs of every sequence (history included): [N, C, 3], oldest first."""
    out = []
    for _, _, _, xe in _histories(np.asarray(x), cu_seqlens, conv_state):
        out.append(xe[-3:].T)
    return np.stack(out) if out else np.zeros((0, np.shape(x)[1], 3), dtype=np.asarray(x).dtype)


def gates(a, b, A_log, dt_bias):
    """beta = sigmoid(b); g = -exp(A_log) * softplus(a + dt_bias), in float64.

    softplus(x) = max(x, 0) + log1p(exp(-|x|)).  a, b: [T, Hv]; A_log, dt_bias: [Hv].
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    x = a + np.asarray(dt_bias, dtype=np.float64)
    sp = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    g = -np.exp(np.asarray(A_log, dtype=np.float64)) * sp
    beta = 1.0 / (1.0 + np.exp(-b))
    return g, beta


def gated_rmsnorm(o, z, w, eps: float = 1e-6) -> np.ndarray:
    """y = o / sqrt(mean(o^2) + eps) * w * z * sigmoid(z) over the last axis, float64.

    o, z: [..., d]; w: [d].
    """
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * w * (z / (1.0 + np.exp(-z)))
