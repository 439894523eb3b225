"""fp64 oracle of the global attention layer -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module; the HIP library never does.

What the Agnes-3.0-Flash pages say of the layer that takes every fourth
place in the decoder (deepmagic page, architecture section; kongchang page,
attention details; mhpq page, section 2 table and config fields):
grouped-query attention with 24 query heads and 4 key/value heads (6:1),
head dim 256, an RMS norm on q and on k, a sigmoid gate on the output, a q
projection twice as wide (q and its gate); rotary position encoding over
three axes (text / height / width, mrope sections 11:11:10, base 1e7) on the
first 25 % of each head (64 dims).

Readings where the pages are silent (each listed in the design notes):
  * text tokens carry the same position on all three rotary axes, so the
    three-axis encoding is ordinary rotary encoding over the 32 frequency
    pairs base^(-2j/64), j = 0..31, whichever axis each pair belongs to;
  * the rotated dims are paired as (j, j + 32) inside the first 64 dims
    (rotate-half), the remaining 192 dims pass through;
  * the RMS norm is per head over the 256 dims, x / sqrt(mean(x^2) + eps) * w
    with eps = 1e-6 and one weight vector for q and one for k, applied
    before the rotation;
  * scores are q.k / sqrt(256), causal within each sequence; query head h
    reads key/value head floor(h / 6);
  * the gate is elementwise over the head's 256 outputs:
    out = softmax(q k^T / 16) v * sigmoid(gate);
  * positions count from 0 at each sequence start; a decode token sits at
    the position equal to the number of tokens already cached.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

__all__ = ["rms_norm", "rope", "rope_angles", "positions", "prep", "core_prefill", "prefill", "core_decode",
           "decode"]

ROT_DIMS = 64
ROPE_BASE = 1.0e7


def rms_norm(x, w, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, dtype=np.float64)


def rope_angles(pos, rot: int = ROT_DIMS, base: float = ROPE_BASE) -> np.ndarray:
    """Rotation angles pos * base^(-2j/rot), j = 0 .. rot/2 - 1: [len(pos), rot/2]."""
    j = np.arange(rot // 2, dtype=np.float64)
    inv = base ** (-2.0 * j / rot)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope(x, pos, rot: int = ROT_DIMS, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate dims (j, j + rot/2) of x[t, ..., :rot] by angle pos[t] * base^(-2j/rot)."""
    x = np.array(x, dtype=np.float64, copy=True)
    ang = rope_angles(pos, rot, base)
    extra = (slice(None),) + (None,) * (x.ndim - 2) + (slice(None),)
    c, s = np.cos(ang)[extra], np.sin(ang)[extra]
    h = rot // 2
    x1, x2 = x[..., :h].copy(), x[..., h:rot].copy()
    x[..., :h] = x1 * c - x2 * s
    x[..., h:rot] = x2 * c + x1 * s
    return x


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def _attend(qh, k, v, scale):
    """softmax(qh k^T * scale) and its product with v, for one query over keys k, v (float64)."""
    s = (qh @ k.T) * scale
    s -= np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    p /= np.sum(p, axis=-1, keepdims=True)
    return p @ v, p


def positions(cu_seqlens, T: int) -> np.ndarray:
    """Position of every packed token inside its sequence (0 at each start)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pos = np.zeros(T, dtype=np.int64)
    for n in range(len(cu) - 1):
        pos[cu[n]:cu[n + 1]] = np.arange(cu[n + 1] - cu[n])
    return pos


def prep(q, k, pos, q_norm_w, k_norm_w, eps: float = 1e-6):
    """The normed, rotated q [T, Hq, D] and k [T, Hk, D] at positions pos [T]."""
    return rope(rms_norm(q, q_norm_w, eps), pos), rope(rms_norm(k, k_norm_w, eps), pos)


def core_prefill(q_rot, k_rot, v, gate, cu_seqlens, *, heads: Optional[Sequence[int]] = None,
                 rows: Optional[Sequence[int]] = None) -> dict:
    """Causal GQA attention of already normed and rotated q, k, gated.

    Returns dict(out [T, Hq, D], mass [T, Hq, D]); mass = sum_j p_j |v_j| *
    sigmoid(gate), the scale of the output's rounding error budget.  Rows
    and heads not asked for are zero.
    """
    q_rot = np.asarray(q_rot, dtype=np.float64)
    k_rot = np.asarray(k_rot, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, D = q_rot.shape
    grp = Hq // k_rot.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    start = np.zeros(T, dtype=np.int64)
    for n in range(len(cu) - 1):
        start[cu[n]:cu[n + 1]] = cu[n]
    out = np.zeros_like(q_rot)
    mass = np.zeros_like(q_rot)
    scale = 1.0 / np.sqrt(D)
    for t in (range(T) if rows is None else rows):
        t0 = start[t]
        for h in (range(Hq) if heads is None else heads):
            kh = h // grp
            o, p = _attend(q_rot[t, h][None], k_rot[t0:t + 1, kh], v[t0:t + 1, kh], scale)
            sg = _sigmoid(gate[t, h])
            out[t, h] = o[0] * sg
            mass[t, h] = (p @ np.abs(v[t0:t + 1, kh]))[0] * sg
    return dict(out=out, mass=mass)


def prefill(q, k, v, gate, q_norm_w, k_norm_w, cu_seqlens, *, eps: float = 1e-6,
            heads: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None) -> dict:
    """Causal GQA attention over a packed batch.

    q, gate [T, Hq, D]; k, v [T, Hk, D]; cu_seqlens [N+1].  ``heads`` and
    ``rows`` restrict which query heads and tokens are computed (others are
    zero).  Returns dict(out, mass, q_rot, k_rot) in float64: the gated
    attention output, its error scale (see core_prefill) and the normed,
    rotated q and k.
    """
    T = np.shape(q)[0]
    q_rot, k_rot = prep(q, k, positions(cu_seqlens, T), q_norm_w, k_norm_w, eps)
    r = core_prefill(q_rot, k_rot, v, gate, cu_seqlens, heads=heads, rows=rows)
    return dict(out=r["out"], mass=r["mass"], q_rot=q_rot, k_rot=k_rot)


def core_decode(q_rot, gate, k_cache, v_cache, lengths) -> dict:
    """One query per sequence against positions 0 .. lengths[n] - 1 of its
    cache: dict(out [N, Hq, D], mass [N, Hq, D]) as in core_prefill."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    N, Hq, D = q_rot.shape
    grp = Hq // np.shape(k_cache)[2]
    out = np.zeros_like(q_rot)
    mass = np.zeros_like(q_rot)
    scale = 1.0 / np.sqrt(D)
    for n in range(N):
        L = int(lengths[n])
        kc = np.asarray(k_cache[n, :L], dtype=np.float64)
        vc = np.asarray(v_cache[n, :L], dtype=np.float64)
        for h in range(Hq):
            o, p = _attend(q_rot[n, h][None], kc[:, h // grp], vc[:, h // grp], scale)
            sg = _sigmoid(gate[n, h])
            out[n, h] = o[0] * sg
            mass[n, h] = (p @ np.abs(vc[:, h // grp]))[0] * sg
    return dict(out=out, mass=mass)


def decode(q, k, v, gate, q_norm_w, k_norm_w, k_cache, v_cache, cache_lens, *, eps: float = 1e-6) -> dict:
    """One new token per sequence against its cache.

    q, gate [N, Hq, D]; k, v [N, Hk, D]; k_cache, v_cache [N, L, Hk, D] holding
    the cached (normed, rotated) keys and values at positions 0 ..
    cache_lens[n] - 1.  The token sits at position cache_lens[n]: its k is
    normed and rotated, both are appended, and its query attends to positions
    0 .. cache_lens[n].  Returns dict(out, mass, q_rot, k_rot, k_cache,
    v_cache) with the caches updated (float64 copies).
    """
    lens = np.asarray(cache_lens, dtype=np.int64)
    q_rot, k_rot = prep(q, k, lens, q_norm_w, k_norm_w, eps)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    for n in range(len(lens)):
        kc[n, lens[n]] = k_rot[n]
        vc[n, lens[n]] = np.asarray(v[n], dtype=np.float64)
    r = core_decode(q_rot, gate, kc, vc, lens + 1)
    return dict(out=r["out"], mass=r["mass"], q_rot=q_rot, k_rot=k_rot, k_cache=kc, v_cache=vc)
