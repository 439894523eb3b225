"""fp64 oracle of the gated delta rule recurrence -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module; the HIP library never does.

The definition followed (Agnes-3.0-Flash pages: gpts24 page, paragraph on the
delta rule -- new state = old state times (I - beta k k^T) plus beta v k^T,
beta a learned per-token write strength; same page, next paragraph -- the gated
variant adds a forget gate; yfxerp page, section 1.2 -- beta = sigmoid(b),
g = -exp(A_log) * softplus(a + dt_bias), q/k L2-normalised inside the kernel):

    S_t = S_{t-1} * exp(g_t) * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = scale * S_t q_t

per (sequence, value head), with S in R^{d_v x d_k}.  ``recurrence`` evaluates
it token by token in the distributed form

    S <- alpha_t S;  u = S k_t;  delta = beta_t (v_t - u);  S <- S + delta k_t^T

which is the same expression multiplied out (alpha_t S_{t-1} (I - beta k k^T)
= alpha_t S_{t-1} - beta (alpha_t S_{t-1} k) k^T).  The unexpanded product of
matrices is checked against it exactly, in rational arithmetic, by the tests.

Readings where the pages are silent (each listed in the design notes):
  * value head h reads key head floor(h * Hk / Hv) (contiguous groups of 3);
  * L2 normalisation is x / sqrt(sum(x^2) + eps), eps = 1e-6, per token and
    key head, applied to q and k when ``use_qk_l2norm`` is set;
  * query scale defaults to 1 (o_t = S_t q_t as written);
  * with ``cu_seqlens`` the batch is one packed row and sequence n is tokens
    [cu[n], cu[n+1]); every sequence starts from its own initial state.

``chunked`` is the chunk-parallel rewrite of the same recurrence (the pages:
prefill takes a block-parallel path with chunk_size 64, decode a single-step
recurrence, and both are numerically interchangeable).  It exists only to pin
that equivalence; parity tests compare the GPU against ``forward``.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "l2_normalise",
    "head_map",
    "recurrence",
    "sequences",
    "forward",
    "forward_parallel",
    "decode_step",
    "decode_step_pool",
    "decode_layer_step",
    "chunked",
]


def l2_normalise(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def head_map(num_k_heads: int, num_v_heads: int) -> np.ndarray:
    """Key head read by each value head: floor(h * Hk / Hv)."""
    if num_v_heads % num_k_heads:
        raise ValueError("value heads must be a multiple of key heads")
    return np.arange(num_v_heads) // (num_v_heads // num_k_heads)


def recurrence(S, alpha, beta, k, v, q, scale=1.0):
    """Token-serial gated delta rule over a batch of independent chains.

    S: [H, dv, dk] start state (not modified); alpha, beta: [T, H];
    k, q: [T, H, dk]; v: [T, H, dv].  Works on float64 arrays and on object
    arrays of ``fractions.Fraction`` (exact arithmetic).
    Returns (o [T, H, dv], S_T [H, dv, dk]).
    """
    S = S.copy()
    T = len(alpha)
    o = np.zeros((T,) + S.shape[:2], dtype=S.dtype)
    for t in range(T):
        S *= alpha[t][:, None, None]
        u = np.matmul(S, k[t][:, :, None])[..., 0]
        delta = beta[t][:, None] * (v[t] - u)
        S += delta[:, :, None] * k[t][:, None, :]
        o[t] = scale * np.matmul(S, q[t][:, :, None])[..., 0]
    return o, S


def sequences(B: int, T: int, cu_seqlens: Optional[np.ndarray]):
    """(row, start, end) of every sequence: batch rows, or packed cu_seqlens."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    if B != 1:
        raise ValueError("cu_seqlens needs a single packed row")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to T")
    return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def forward(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *,
            use_qk_l2norm: bool = True, eps: float = 1e-6, scale: float = 1.0,
            heads: Optional[Sequence[int]] = None, token_limit: Optional[int] = None):
    """Reference prefill for q, k [B, T, Hk, dk], v [B, T, Hv, dv], g, beta [B, T, Hv].

    initial_state: [N, Hv, dv, dk] or None (zero).  ``heads`` restricts the
    computation to a subset of value heads (others stay zero);
    ``token_limit`` stops every sequence after that many of its tokens.
    Returns (o [B, T, Hv, dv] float64, final_state [N, Hv, dv, dk] float64).
    """
    B, T, hk, dk = np.shape(q)
    hv, dv = np.shape(v)[2], np.shape(v)[3]
    kmap = head_map(hk, hv)
    hs = np.arange(hv) if heads is None else np.asarray(heads, dtype=np.int64)
    # only the value heads asked for, and the key heads they read, are upcast
    kh = kmap[hs]
    q = np.asarray(np.asarray(q)[:, :, kh], dtype=np.float64)
    k = np.asarray(np.asarray(k)[:, :, kh], dtype=np.float64)
    v = np.asarray(np.asarray(v)[:, :, hs], dtype=np.float64)
    g = np.asarray(np.asarray(g)[:, :, hs], dtype=np.float64)
    beta = np.asarray(np.asarray(beta)[:, :, hs], dtype=np.float64)
    if use_qk_l2norm:
        q = l2_normalise(q, eps)
        k = l2_normalise(k, eps)
    seqs = sequences(B, T, cu_seqlens)
    o = np.zeros((B, T, hv, dv))
    final = np.zeros((len(seqs), hv, dv, dk))
    for n, (b, t0, t1) in enumerate(seqs):
        if token_limit is not None:
            t1 = min(t1, t0 + token_limit)
        S0 = np.zeros((len(hs), dv, dk)) if initial_state is None else \
            np.asarray(initial_state[n], dtype=np.float64)[hs]
        sl = slice(t0, t1)
        o_seq, S = recurrence(S0, np.exp(g[b, sl]), beta[b, sl], k[b, sl], v[b, sl], q[b, sl], scale)
        o[b, sl][:, hs] = o_seq
        final[n, hs] = S
    return o, final


_POOL_ARGS = None


def _pool_worker(heads):
    args, kwargs = _POOL_ARGS
    o, s = forward(*args, heads=heads, **kwargs)
    return heads, o[:, :, heads], s[:, heads]


def forward_parallel(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *,
                     processes: Optional[int] = None, **kwargs):
    """``forward`` with value heads spread over a fork-based process pool.

    Chains of different value heads are independent, so the result is the same
    as ``forward``'s.  Returns (o, final_state, processes used).
    """
    global _POOL_ARGS
    hv = np.asarray(v).shape[2]
    if processes is None:
        processes = len(os.sched_getaffinity(0))
    processes = max(1, min(processes, hv))
    groups = [list(range(i, hv, processes)) for i in range(processes)]
    _POOL_ARGS = ((q, k, v, g, beta, initial_state, cu_seqlens), kwargs)
    try:
        if processes == 1:
            parts = [_pool_worker(groups[0])]
        else:
            with mp.get_context("fork").Pool(processes) as pool:
                parts = pool.map(_pool_worker, groups)
    finally:
        _POOL_ARGS = None
    B, T = np.asarray(q).shape[:2]
    dk, dv = np.asarray(q).shape[3], np.asarray(v).shape[3]
    n = B if cu_seqlens is None else len(cu_seqlens) - 1
    o = np.zeros((B, T, hv, dv))
    final = np.zeros((n, hv, dv, dk))
    for heads, o_part, s_part in parts:
        o[:, :, heads] = o_part
        final[:, heads] = s_part
    return o, final, processes


def decode_step(q, k, v, g, beta, state, *, use_qk_l2norm: bool = True,
                eps: float = 1e-6, scale: float = 1.0):
    """One decode token for N independent sequences.

    q, k: [N, Hk, dk]; v: [N, Hv, dv]; g, beta: [N, Hv]; state [N, Hv, dv, dk].
    Returns (o [N, Hv, dv], new_state [N, Hv, dv, dk]), both float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    kmap = head_map(hk, hv)
    if use_qk_l2norm:
        q = l2_normalise(q, eps)
        k = l2_normalise(k, eps)
    S0 = np.asarray(state, dtype=np.float64).reshape(N * hv, dv, dk)
    flat = lambda x: np.asarray(x, dtype=np.float64).reshape(1, N * hv, *np.shape(x)[2:])
    o, S = recurrence(S0, np.exp(flat(g)), flat(beta), flat(k[:, kmap]), flat(v),
                      flat(q[:, kmap]), scale)
    return o.reshape(N, hv, dv), S.reshape(N, hv, dv, dk)


def decode_step_pool(q, k, v, g, beta, pool, state_indices, *, use_qk_l2norm: bool = True,
                     eps: float = 1e-6, scale: float = 1.0):
    """decode_step on states kept in a pool (yfxerp page, section 1.2: the
    delta-rule layers keep their recurrent state in a cache layer of their
    own).  Row n updates pool[state_indices[n]]; an index outside
    [0, len(pool)) marks a padding row, whose o is zero and which touches no
    slot.  Valid indices must be distinct.

    Returns (o [N, Hv, dv], new_pool), both float64; slots no row names keep
    their values.
    """
    idx = np.asarray(state_indices, dtype=np.int64)
    pool = np.asarray(pool, dtype=np.float64)
    live = (idx >= 0) & (idx < len(pool))
    if len(np.unique(idx[live])) != int(live.sum()):
        raise ValueError("state_indices name a slot twice")
    N, hv, dv = len(idx), np.shape(v)[1], np.shape(v)[2]
    o = np.zeros((N, hv, dv))
    new_pool = pool.copy()
    if live.any():
        rows = np.flatnonzero(live)
        sel = lambda x: np.asarray(x)[rows]
        o_live, s_live = decode_step(sel(q), sel(k), sel(v), sel(g), sel(beta), pool[idx[rows]],
                                     use_qk_l2norm=use_qk_l2norm, eps=eps, scale=scale)
        o[rows] = o_live
        new_pool[idx[rows]] = s_live
    return o, new_pool


def decode_layer_step(x, conv_w, conv_state, a, b, A_log, dt_bias, state, z, norm_w, hk, hv, *,
                      state_indices=None, use_qk_l2norm: bool = True, eps: float = 1e-6, scale: float = 1.0,
                      norm_eps: float = 1e-6):
    """One decode token of the layer path: the conv front against each row's
    conv state (the fp32 bit-exact definition), the gates, decode_step_pool,
    and the gated RMS norm (deepmagic page, architecture section; yfxerp page,
    section 1.2: the decode path keeps a conv state beside the recurrent state).

    x: [N, C] (C = (2 hk + hv) d, blocks q | k | v); conv_state: [P, C, 3];
    state: [P, hv, d, d]; a, b: [N, hv]; z: [N, hv d].  Rows name slots of both
    pools through state_indices (default: row n -> slot n); padding rows
    (index outside [0, P)) give zero outputs and touch no slot.
    Returns (y [N, hv d], o [N, hv, d], qkv [N, C] (bf16 values), new conv
    pool, new state pool); y and o float64.
    """
    from oracle import conv as cv
    x = np.asarray(x, dtype=np.float32)
    N, C = x.shape
    d = C // (2 * hk + hv)
    P = len(state)
    idx = np.arange(N) if state_indices is None else np.asarray(state_indices, dtype=np.int64)
    live = np.flatnonzero((idx >= 0) & (idx < P))
    conv_pool = np.array(conv_state, dtype=np.float32, copy=True)
    qkv = np.zeros((N, C), dtype=np.float32)
    if len(live):
        cu = np.arange(len(live) + 1)
        cs = conv_pool[idx[live]]
        qkv[live] = cv.conv_silu_fp32(x[live], conv_w, cu, cs)
        conv_pool[idx[live]] = cv.conv_state_out(x[live], cu, cs)
    q = qkv[:, :hk * d].reshape(N, hk, d)
    k = qkv[:, hk * d:2 * hk * d].reshape(N, hk, d)
    v = qkv[:, 2 * hk * d:].reshape(N, hv, d)
    g, beta = cv.gates(a, b, A_log, dt_bias)
    o, new_state = decode_step_pool(q, k, v, g, beta, state, idx, use_qk_l2norm=use_qk_l2norm, eps=eps,
                                    scale=scale)
    y = np.zeros((N, hv * d))
    if len(live):
        zz = np.asarray(z, dtype=np.float64).reshape(N, hv, d)
        y[live] = cv.gated_rmsnorm(o[live], zz[live], norm_w, norm_eps).reshape(len(live), hv * d)
    return y, o, qkv, conv_pool, new_state


def chunked(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *, chunk_size: int = 64,
            use_qk_l2norm: bool = True, eps: float = 1e-6, scale: float = 1.0,
            heads: Optional[Sequence[int]] = None):
    """Chunk-form evaluation of the same recurrence, in float64.

    For a chunk of L tokens with start state S0, local cumulative log-decay
    G_i = sum_{m<=i} g_m and Gamma_ij = exp(G_i - G_j) for j <= i (else 0):
      A     = strictly-lower(diag(beta) (Gamma * K K^T))
      Delta = (I + A)^{-1} (diag(beta) V - diag(beta exp(G)) K S0^T)
      O     = scale (diag(exp(G)) Q S0^T + (Gamma * Q K^T) Delta)
      S_L   = exp(G_L) S0 + (diag(Gamma_{L,:}) Delta)^T K
    Chunks restart at every sequence start; the last one may be partial.
    Used only to pin chunked-vs-stepwise equivalence.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, hk, dk = q.shape
    hv, dv = v.shape[2], v.shape[3]
    kmap = head_map(hk, hv)
    hs = range(hv) if heads is None else heads
    if use_qk_l2norm:
        q = l2_normalise(q, eps)
        k = l2_normalise(k, eps)
    seqs = sequences(B, T, cu_seqlens)
    o = np.zeros((B, T, hv, dv))
    final = np.zeros((len(seqs), hv, dv, dk))
    for n, (b, t0, t1) in enumerate(seqs):
        for h in hs:
            S = np.zeros((dv, dk)) if initial_state is None else \
                np.asarray(initial_state[n, h], dtype=np.float64).copy()
            for c0 in range(t0, t1, chunk_size):
                c1 = min(c0 + chunk_size, t1)
                K = k[b, c0:c1, kmap[h]]
                Q = q[b, c0:c1, kmap[h]]
                V = v[b, c0:c1, h]
                bt = beta[b, c0:c1, h]
                G = np.cumsum(g[b, c0:c1, h])
                L = c1 - c0
                diff = G[:, None] - G[None, :]
                lower = np.tril(np.ones((L, L), dtype=bool))
                Gam = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
                A = np.tril(bt[:, None] * Gam * (K @ K.T), -1)
                R = bt[:, None] * V - (bt * np.exp(G))[:, None] * (K @ S.T)
                Dlt = np.linalg.solve(np.eye(L) + A, R)
                o[b, c0:c1, h] = scale * (np.exp(G)[:, None] * (Q @ S.T) + (Gam * (Q @ K.T)) @ Dlt)
                S = np.exp(G[-1]) * S + (Gam[-1][:, None] * Dlt).T @ K
            final[n, h] = S
    return o, final
