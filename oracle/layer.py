"""fp64 oracle of the whole delta layer -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module; the HIP library never does.

The layer as the Agnes-3.0-Flash pages describe it: an input projection from
the hidden width (5120, deepmagic page, architecture section) to the q|k|v
channels, a 6144-wide z and one b and one a per value head (yfxerp page,
parameter ledger in section 2); the kernel-4 causal conv + SiLU and the gates
in front of the recurrence, the gated RMS norm behind it (deepmagic page,
architecture section) and an output projection from 6144 back to the hidden
width (the same ledger).  The stages are the ones ``oracle.conv`` and
``oracle.gdr`` define; this module strings them together with plain float64
matrix products.

Readings where the pages are silent:
  * the model runs in bf16, so every projection output (q|k|v, z, b, a and
    the layer output) is rounded to bf16, nearest even; the gates then take
    b and a as those bf16 values, widened;
  * the input projection's rows are ordered q|k|v channels, then z, then b,
    then a (the order the ledger lists them in);
  * q|k|v channels are blocked q (Hk heads), k (Hk heads), v (Hv heads), head
    major, as in the conv front;
  * the recurrence runs with q/k L2 normalisation, scale 1 and chunk 64, and
    its output o goes into the norm unrounded; the norm output y is rounded
    to bf16 before the output projection.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from oracle import conv as cv
from oracle import gdr

__all__ = ["linear", "delta_layer_forward"]


def linear(x, w) -> np.ndarray:
    """x W^T in float64: x [M, K], w [N, K] -> [M, N] (a linear layer's product)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def delta_layer_forward(hidden, w_in, conv_w, A_log, dt_bias, norm_w, w_out, cu_seqlens, hk: int, hv: int, *,
                        conv_state=None, initial_state=None, heads: Optional[Sequence[int]] = None,
                        eps: float = 1e-6, norm_eps: float = 1e-6) -> dict:
    """The layer's prefill over a packed batch.

    hidden [T, H]; w_in [C + V + 2 hv, H]; conv_w [C, 4]; A_log, dt_bias [hv];
    norm_w [d]; w_out [H, V]; cu_seqlens [N+1]; C = (2 hk + hv) d, V = hv d.
    ``heads`` restricts the recurrence to some value heads; the others' o is
    zero, so y and out are then only partial (use it for stage checks).
    Returns a dict of every stage: qkv, z, b, a (bf16 values, float32), the
    conv outputs q, k, v (bf16 values), g, beta, o, final_state, y (bf16
    values) and out (bf16 values).
    """
    hidden = np.asarray(hidden, dtype=np.float32)
    T, H = hidden.shape
    V = np.shape(w_out)[1]
    d = V // hv
    C = (2 * hk + hv) * d
    proj = linear(hidden, w_in)
    qkv = cv.round_bf16(proj[:, :C])
    z = cv.round_bf16(proj[:, C:C + V])
    b = cv.round_bf16(proj[:, C + V:C + V + hv])
    a = cv.round_bf16(proj[:, C + V + hv:C + V + 2 * hv])
    xc = cv.conv_silu_fp32(qkv, conv_w, cu_seqlens, conv_state)
    q = xc[:, :hk * d].reshape(1, T, hk, d)
    k = xc[:, hk * d:2 * hk * d].reshape(1, T, hk, d)
    v = xc[:, 2 * hk * d:].reshape(1, T, hv, d)
    g, beta = cv.gates(a, b, A_log, dt_bias)
    o, final = gdr.forward(q, k, v, g[None], beta[None], initial_state, cu_seqlens, use_qk_l2norm=True, eps=eps,
                           heads=heads)
    y = cv.round_bf16(cv.gated_rmsnorm(o[0], z.reshape(T, hv, d), norm_w, norm_eps).reshape(T, V))
    out = cv.round_bf16(linear(y, w_out))
    return dict(qkv=qkv, z=z, b=b, a=a, q=q, k=k, v=v, g=g, beta=beta, o=o, final_state=final, y=y, out=out,
                conv_state=cv.conv_state_out(qkv, cu_seqlens, conv_state))
