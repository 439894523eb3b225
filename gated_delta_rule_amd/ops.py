"""Torch-facing wrappers of the libgdr entry points.

Each function checks tensor placement, dtype and contiguity, allocates its
outputs with torch, and passes raw device pointers and the current HIP stream
to the C ABI.  Every step of the computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

_DT = {torch.float32: _lib.GDR_F32, torch.bfloat16: _lib.GDR_BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtypes, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_desc(B, T, N, Hk, Hv, D, chunk_size, qkv_dtype, out_dtype, use_qk_l2norm, scale, eps):
    d = _lib.GdrDesc()
    d.struct_size = ctypes.sizeof(_lib.GdrDesc)
    d.batch, d.seq_len, d.num_seqs = B, T, N
    d.num_k_heads, d.num_v_heads = Hk, Hv
    d.head_dim_k = d.head_dim_v = D
    d.chunk_size = chunk_size
    d.qkv_dtype = _DT[qkv_dtype]
    d.out_dtype = _DT[out_dtype]
    d.use_qk_l2norm = int(bool(use_qk_l2norm))
    d.scale = scale
    d.l2norm_eps = eps
    return d


def chunk_gated_delta_rule(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                           beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                           output_final_state: bool = False, cu_seqlens: Optional[torch.Tensor] = None,
                           use_qk_l2norm_in_kernel: bool = True, scale: float = 1.0,
                           chunk_size: int = 64, out_dtype: torch.dtype = torch.float32,
                           final_state: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None,
                           stage: str = "all") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill (gdr_chunk_fwd).

    q, k: [B, T, Hk, d]; v: [B, T, Hv, d] (bf16 or fp32, same dtype);
    g, beta: [B, T, Hv] fp32; initial_state: [N, Hv, d, d] fp32 or None;
    cu_seqlens: int32 [N+1] (then B must be 1).  ``final_state`` may be given
    as a preallocated output (it may be ``initial_state`` itself); ``workspace``
    (uint8, device) is used if large enough, else one is allocated.
    ``stage``: "all" (gdr_chunk_fwd), or "prepare" / "recurrence" for the two
    stages alone (gdr_chunk_fwd_prepare / gdr_chunk_fwd_recurrence; pass the
    same ``workspace``, ``out`` and ``final_state`` to both).
    Returns (o [B, T, Hv, d] out_dtype, final_state or None).
    """
    entry = {"all": "gdr_chunk_fwd", "prepare": "gdr_chunk_fwd_prepare",
             "recurrence": "gdr_chunk_fwd_recurrence"}.get(stage)
    if entry is None:
        raise ValueError(f"unknown stage {stage!r}")
    dev = q.device
    qd = q.dtype
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, (qd,), dev)
    if qd not in _DT:
        raise TypeError(f"q/k/v dtype {qd} unsupported")
    _need(g, "g", (torch.float32,), dev)
    _need(beta, "beta", (torch.float32,), dev)
    B, T, Hk, D = q.shape
    Hv = v.shape[2]
    if k.shape != q.shape or v.shape != (B, T, Hv, D) or g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (torch.int32,), dev)
        N = cu_seqlens.numel() - 1
        if B != 1:
            raise ValueError("cu_seqlens needs B == 1")
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", (torch.float32,), dev)
        if initial_state.shape != (N, Hv, D, D):
            raise ValueError(f"initial_state must be {(N, Hv, D, D)}")
    if final_state is None and output_final_state:
        final_state = torch.empty((N, Hv, D, D), device=dev, dtype=torch.float32)
    if final_state is not None:
        _need(final_state, "final_state", (torch.float32,), dev)
        if final_state.shape != (N, Hv, D, D):
            raise ValueError(f"final_state must be {(N, Hv, D, D)}")
    if out is None:
        out = torch.empty((B, T, Hv, D), device=dev, dtype=out_dtype)
    else:
        _need(out, "out", (out_dtype,), dev)
    desc = make_desc(B, T, N, Hk, Hv, D, chunk_size, qd, out_dtype, use_qk_l2norm_in_kernel, scale, 1e-6)
    lib = _lib.load()
    nbytes = ctypes.c_size_t(0)
    _lib.check("gdr_chunk_fwd_workspace_size", lib.gdr_chunk_fwd_workspace_size(ctypes.byref(desc),
                                                                                ctypes.byref(nbytes)))
    if workspace is None or workspace.numel() < nbytes.value:
        if stage != "all" and nbytes.value:
            raise ValueError(f"stage {stage!r} needs a workspace of {nbytes.value} bytes")
        workspace = torch.empty(nbytes.value, device=dev, dtype=torch.uint8) if nbytes.value else None
    st = getattr(lib, entry)(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), _ptr(out),
                             _ptr(workspace), nbytes.value, _stream(dev))
    _lib.check(entry, st)
    return out, final_state


def chunk_workspace(q: torch.Tensor, v: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                    chunk_size: int = 64, out_dtype: torch.dtype = torch.float32) -> Optional[torch.Tensor]:
    """A device workspace (uint8) of the size gdr_chunk_fwd needs for these
    shapes (gdr_chunk_fwd_workspace_size), or None if it needs none."""
    B, T, Hk, D = q.shape
    N = cu_seqlens.numel() - 1 if cu_seqlens is not None else B
    desc = make_desc(B, T, N, Hk, v.shape[2], D, chunk_size, q.dtype, out_dtype, True, 1.0, 1e-6)
    nbytes = ctypes.c_size_t(0)
    _lib.check("gdr_chunk_fwd_workspace_size",
               _lib.load().gdr_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes)))
    return torch.empty(nbytes.value, device=q.device, dtype=torch.uint8) if nbytes.value else None


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                   state: torch.Tensor, use_qk_l2norm_in_kernel: bool = True, scale: float = 1.0,
                   out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                   state_indices: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode token (gdr_recurrent_step); the states are updated in place.

    q, k: [N, Hk, d]; v: [N, Hv, d]; g, beta: [N, Hv] fp32.  Returns o [N, Hv, d].
    Without ``state_indices``, ``state`` is [N, Hv, d, d].  With it (int32 [N],
    gdr_recurrent_step_indexed), ``state`` is a pool [P, Hv, d, d] and sequence
    n updates slot state_indices[n]; an index outside [0, P) marks a padding
    row (o = 0, no slot touched).
    """
    dev = q.device
    qd = q.dtype
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, (qd,), dev)
    if qd not in _DT:
        raise TypeError(f"q/k/v dtype {qd} unsupported")
    _need(g, "g", (torch.float32,), dev)
    _need(beta, "beta", (torch.float32,), dev)
    _need(state, "state", (torch.float32,), dev)
    N, Hk, D = q.shape
    Hv = v.shape[1]
    if k.shape != q.shape or v.shape != (N, Hv, D) or g.shape != (N, Hv) or beta.shape != (N, Hv):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    if state_indices is None:
        if state.shape != (N, Hv, D, D):
            raise ValueError(f"state must be {(N, Hv, D, D)}")
    else:
        _need(state_indices, "state_indices", (torch.int32,), dev)
        if state_indices.shape != (N,) or state.dim() != 4 or state.shape[1:] != (Hv, D, D):
            raise ValueError(f"state_indices must be [{N}] and state a pool [P, {Hv}, {D}, {D}]")
    if out is None:
        out = torch.empty((N, Hv, D), device=dev, dtype=out_dtype)
    else:
        _need(out, "out", (out_dtype,), dev)
    desc = make_desc(N, 1, N, Hk, Hv, D, 64, qd, out_dtype, use_qk_l2norm_in_kernel, scale, 1e-6)
    lib = _lib.load()
    if state_indices is None:
        st = lib.gdr_recurrent_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(state), _ptr(out), _stream(dev))
        _lib.check("gdr_recurrent_step", st)
    else:
        st = lib.gdr_recurrent_step_indexed(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                            _ptr(state) if state.numel() else None, state.shape[0],
                                            _ptr(state_indices), _ptr(out), _stream(dev))
        _lib.check("gdr_recurrent_step_indexed", st)
    return out


def decode_layer_step(x: torch.Tensor, conv_w: torch.Tensor, conv_state: torch.Tensor, a: torch.Tensor,
                      b: torch.Tensor, A_log: torch.Tensor, dt_bias: torch.Tensor, state: torch.Tensor,
                      z: torch.Tensor, norm_w: torch.Tensor, num_k_heads: int, num_v_heads: int,
                      state_indices: Optional[torch.Tensor] = None, use_qk_l2norm_in_kernel: bool = True,
                      scale: float = 1.0, norm_eps: float = 1e-6, return_intermediates: bool = False):
    """One decode token of the layer path in one launch (gdr_decode_layer_step):
    conv front against the rolling ``conv_state``, gates, recurrent step, gated
    RMS norm.  Both states are updated in place.

    x: [N, C] bf16 (C = (2*Hk + Hv)*128, blocks q | k | v); conv_w: [C, 4] bf16;
    conv_state: [P, C, 3] bf16; a, b: [N, Hv] fp32; A_log, dt_bias: [Hv] fp32;
    state: [P, Hv, 128, 128] fp32; z: [N, Hv*128] bf16; norm_w: [128] fp32.
    Without ``state_indices`` P = N and row n uses slot n; with it (int32 [N])
    row n uses slot state_indices[n] of both pools, and an index outside [0, P)
    marks a padding row (zero outputs, no slot touched).
    Returns y [N, Hv*128] bf16, or (y, o [N, Hv, 128] fp32, qkv [N, C] bf16)
    with ``return_intermediates``.
    """
    dev = x.device
    Hk, Hv, D = num_k_heads, num_v_heads, 128
    N, C = x.shape
    if C != (2 * Hk + Hv) * D:
        raise ValueError(f"x must be [N, {(2 * Hk + Hv) * D}]")
    _need(x, "x", (torch.bfloat16,), dev)
    _need(conv_w, "conv_w", (torch.bfloat16,), dev)
    _need(conv_state, "conv_state", (torch.bfloat16,), dev)
    _need(z, "z", (torch.bfloat16,), dev)
    for t, name in ((a, "a"), (b, "b"), (A_log, "A_log"), (dt_bias, "dt_bias"), (state, "state"),
                    (norm_w, "norm_w")):
        _need(t, name, (torch.float32,), dev)
    P = state.shape[0]
    if conv_w.shape != (C, 4) or conv_state.shape != (P, C, 3) or state.shape != (P, Hv, D, D) \
            or a.shape != (N, Hv) or b.shape != (N, Hv) or z.shape != (N, Hv * D) or norm_w.shape != (D,):
        raise ValueError("shape mismatch among the decode-layer arguments")
    if state_indices is None:
        if P != N:
            raise ValueError("without state_indices the pools hold one slot per row")
    else:
        _need(state_indices, "state_indices", (torch.int32,), dev)
        if state_indices.shape != (N,):
            raise ValueError(f"state_indices must be [{N}]")
    y = torch.empty((N, Hv * D), device=dev, dtype=torch.bfloat16)
    o = torch.empty((N, Hv, D), device=dev, dtype=torch.float32) if return_intermediates else None
    qkv = torch.empty((N, C), device=dev, dtype=torch.bfloat16) if return_intermediates else None
    desc = make_desc(N, 1, N, Hk, Hv, D, 64, torch.bfloat16, torch.float32, use_qk_l2norm_in_kernel, scale, 1e-6)
    st = _lib.load().gdr_decode_layer_step(
        ctypes.byref(desc), _ptr(x), _ptr(conv_w), _ptr(conv_state) if conv_state.numel() else None, _ptr(a),
        _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(state) if state.numel() else None, P, _ptr(state_indices),
        _ptr(z), _ptr(norm_w), norm_eps, _ptr(y), _ptr(o), _ptr(qkv), _stream(dev))
    _lib.check("gdr_decode_layer_step", st)
    return (y, o, qkv) if return_intermediates else y


def conv_gate_fused(x: torch.Tensor, conv_w: torch.Tensor, cu_seqlens: torch.Tensor, a: torch.Tensor,
                    b: torch.Tensor, A_log: torch.Tensor, dt_bias: torch.Tensor, num_k_heads: int,
                    num_v_heads: int, head_dim: int, conv_state_in: Optional[torch.Tensor] = None,
                    output_conv_state: bool = False):
    """Conv + SiLU + gates front (gdr_conv_gate_fused).

    x: [T, C] bf16 with C = 2*Hk*d + Hv*d; conv_w: [C, 4] bf16; cu_seqlens int32 [N+1];
    a, b: [T, Hv] fp32; A_log, dt_bias: [Hv] fp32.
    Returns (q [1, T, Hk, d], k [1, T, Hk, d], v [1, T, Hv, d], g [1, T, Hv], beta [1, T, Hv],
    conv_state_out [N, C, 3] or None).
    """
    dev = x.device
    Hk, Hv, D = num_k_heads, num_v_heads, head_dim
    T, C = x.shape
    if C != (2 * Hk + Hv) * D:
        raise ValueError("x width must be 2*Hk*d + Hv*d")
    _need(x, "x", (torch.bfloat16,), dev)
    _need(conv_w, "conv_w", (torch.bfloat16,), dev)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,), dev)
    for t, name in ((a, "a"), (b, "b"), (A_log, "A_log"), (dt_bias, "dt_bias")):
        _need(t, name, (torch.float32,), dev)
    if conv_w.shape != (C, 4) or a.shape != (T, Hv) or b.shape != (T, Hv) or A_log.shape != (Hv,) \
            or dt_bias.shape != (Hv,):
        raise ValueError("shape mismatch in conv front inputs")
    N = cu_seqlens.numel() - 1
    if conv_state_in is not None:
        _need(conv_state_in, "conv_state_in", (torch.bfloat16,), dev)
        if conv_state_in.shape != (N, C, 3):
            raise ValueError(f"conv_state_in must be {(N, C, 3)}")
    q = torch.empty((1, T, Hk, D), device=dev, dtype=torch.bfloat16)
    k = torch.empty((1, T, Hk, D), device=dev, dtype=torch.bfloat16)
    v = torch.empty((1, T, Hv, D), device=dev, dtype=torch.bfloat16)
    g = torch.empty((1, T, Hv), device=dev, dtype=torch.float32)
    beta = torch.empty((1, T, Hv), device=dev, dtype=torch.float32)
    state_out = torch.empty((N, C, 3), device=dev, dtype=torch.bfloat16) if output_conv_state else None
    desc = _lib.GdrConvDesc()
    desc.struct_size = ctypes.sizeof(_lib.GdrConvDesc)
    desc.num_tokens, desc.num_seqs = T, N
    desc.num_k_heads, desc.num_v_heads, desc.head_dim = Hk, Hv, D
    st = _lib.load().gdr_conv_gate_fused(ctypes.byref(desc), _ptr(x), _ptr(conv_w), _ptr(cu_seqlens),
                                         _ptr(conv_state_in), _ptr(state_out), _ptr(a), _ptr(b), _ptr(A_log),
                                         _ptr(dt_bias), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         _stream(dev))
    _lib.check("gdr_conv_gate_fused", st)
    return q, k, v, g, beta, state_out


def gated_rmsnorm(o: torch.Tensor, z: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gated RMSNorm back (gdr_gated_rmsnorm).

    o: [..., Hv, d] fp32 or bf16; z: [..., Hv*d] bf16 (same leading size);
    w: [d] fp32.  Returns y [..., Hv*d] bf16.
    """
    dev = o.device
    _need(o, "o", (torch.float32, torch.bfloat16), dev)
    _need(z, "z", (torch.bfloat16,), dev)
    _need(w, "w", (torch.float32,), dev)
    Hv, D = o.shape[-2], o.shape[-1]
    T = o.numel() // (Hv * D)
    if z.numel() != T * Hv * D or w.shape != (D,):
        raise ValueError("shape mismatch among o, z, w")
    if out is None:
        out = torch.empty(z.shape, device=dev, dtype=torch.bfloat16)
    desc = _lib.GdrNormDesc()
    desc.struct_size = ctypes.sizeof(_lib.GdrNormDesc)
    desc.num_tokens, desc.num_heads, desc.head_dim = T, Hv, D
    desc.o_dtype = _DT[o.dtype]
    desc.eps = eps
    st = _lib.load().gdr_gated_rmsnorm(ctypes.byref(desc), _ptr(o), _ptr(z), _ptr(w), _ptr(out), _stream(dev))
    _lib.check("gdr_gated_rmsnorm", st)
    return out


def linear(x: torch.Tensor, w: torch.Tensor, blocks=None, out_dtype: torch.dtype = torch.bfloat16):
    """Dense projection y = x W^T (gdr_linear): bf16 operands, fp32 accumulation.

    x: [M, K] bf16, w: [N, K] bf16 (K a multiple of 32).  Without ``blocks``
    returns one [M, N] tensor of ``out_dtype`` (bf16 or fp32).  ``blocks`` is a
    list of (width, dtype) or (width, dtype, round_bf16) splitting the N output
    columns into separate tensors, returned as a list.
    """
    dev = x.device
    _need(x, "x", (torch.bfloat16,), dev)
    _need(w, "w", (torch.bfloat16,), dev)
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [M, K] and w [N, K]")
    M, K = x.shape
    N = w.shape[0]
    single = blocks is None
    if single:
        blocks = [(N, out_dtype)]
    if not 1 <= len(blocks) <= 4:
        raise ValueError("1..4 output blocks")
    outs = (_lib.GdrLinearOut * len(blocks))()
    tensors = []
    for i, blk in enumerate(blocks):
        width, dt = blk[0], blk[1]
        rnd = bool(blk[2]) if len(blk) > 2 else False
        t = torch.empty((M, width), device=dev, dtype=dt)
        tensors.append(t)
        outs[i].ptr = t.data_ptr() if t.numel() else None
        outs[i].ld = width
        outs[i].cols = width
        outs[i].dtype = _DT[dt]
        outs[i].round_bf16 = int(rnd)
        outs[i].reserved = 0
    st = _lib.load().gdr_linear(M, N, K, _ptr(x), K, _ptr(w), K, outs, len(blocks), _stream(dev))
    _lib.check("gdr_linear", st)
    return tensors[0] if single else tensors


def layer_desc(T, N, hidden, Hk, Hv, D, l2norm_eps=1e-6, norm_eps=1e-6):
    d = _lib.GdrLayerDesc()
    d.struct_size = ctypes.sizeof(_lib.GdrLayerDesc)
    d.num_tokens, d.num_seqs, d.hidden = T, N, hidden
    d.num_k_heads, d.num_v_heads, d.head_dim = Hk, Hv, D
    d.l2norm_eps, d.norm_eps = l2norm_eps, norm_eps
    return d


def delta_layer_workspace(T: int, N: int, hidden: int, num_k_heads: int, num_v_heads: int, head_dim: int = 128,
                          device=None) -> torch.Tensor:
    """A device workspace large enough for delta_layer_fwd on these sizes."""
    d = layer_desc(T, N, hidden, num_k_heads, num_v_heads, head_dim)
    n = ctypes.c_size_t(0)
    _lib.check("gdr_delta_layer_workspace_size", _lib.load().gdr_delta_layer_workspace_size(ctypes.byref(d),
                                                                                           ctypes.byref(n)))
    return torch.empty(max(n.value, 1), device=device, dtype=torch.uint8)


def delta_layer_fwd(hidden: torch.Tensor, w_in: torch.Tensor, conv_w: torch.Tensor, A_log: torch.Tensor,
                    dt_bias: torch.Tensor, norm_w: torch.Tensor, w_out: torch.Tensor, cu_seqlens: torch.Tensor,
                    num_k_heads: int, num_v_heads: int, head_dim: int = 128,
                    conv_state_in: Optional[torch.Tensor] = None, output_conv_state: bool = False,
                    initial_state: Optional[torch.Tensor] = None, output_final_state: bool = False,
                    final_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, l2norm_eps: float = 1e-6, norm_eps: float = 1e-6):
    """Prefill of one whole delta layer (gdr_delta_layer_fwd).

    hidden: [T, H] bf16; w_in: [C + V + 2*Hv, H] bf16 (rows q|k|v, z, b, a);
    conv_w: [C, 4] bf16; A_log, dt_bias: [Hv] fp32; norm_w: [d] fp32;
    w_out: [H, V] bf16; cu_seqlens: int32 [N+1].
    Returns (out [T, H] bf16, final_state or None, conv_state_out or None).
    """
    dev = hidden.device
    Hk, Hv, D = num_k_heads, num_v_heads, head_dim
    T, H = hidden.shape
    C, V = (2 * Hk + Hv) * D, Hv * D
    _need(hidden, "hidden", (torch.bfloat16,), dev)
    _need(w_in, "w_in", (torch.bfloat16,), dev)
    _need(conv_w, "conv_w", (torch.bfloat16,), dev)
    _need(w_out, "w_out", (torch.bfloat16,), dev)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,), dev)
    for t, name in ((A_log, "A_log"), (dt_bias, "dt_bias"), (norm_w, "norm_w")):
        _need(t, name, (torch.float32,), dev)
    N = cu_seqlens.numel() - 1
    if w_in.shape != (C + V + 2 * Hv, H) or w_out.shape != (H, V) or conv_w.shape != (C, 4) \
            or A_log.shape != (Hv,) or dt_bias.shape != (Hv,) or norm_w.shape != (D,):
        raise ValueError("shape mismatch in delta layer weights")
    if conv_state_in is not None:
        _need(conv_state_in, "conv_state_in", (torch.bfloat16,), dev)
        if conv_state_in.shape != (N, C, 3):
            raise ValueError(f"conv_state_in must be {(N, C, 3)}")
    if initial_state is not None:
        _need(initial_state, "initial_state", (torch.float32,), dev)
        if initial_state.shape != (N, Hv, D, D):
            raise ValueError(f"initial_state must be {(N, Hv, D, D)}")
    if output_final_state and final_state is None:
        final_state = torch.empty((N, Hv, D, D), device=dev, dtype=torch.float32)
    conv_state_out = torch.empty((N, C, 3), device=dev, dtype=torch.bfloat16) if output_conv_state else None
    if out is None:
        out = torch.empty((T, H), device=dev, dtype=torch.bfloat16)
    d = layer_desc(T, N, H, Hk, Hv, D, l2norm_eps, norm_eps)
    if workspace is None:
        workspace = delta_layer_workspace(T, N, H, Hk, Hv, D, device=dev)
    st = _lib.load().gdr_delta_layer_fwd(ctypes.byref(d), _ptr(hidden), _ptr(w_in), _ptr(conv_w), _ptr(A_log),
                                         _ptr(dt_bias), _ptr(norm_w), _ptr(w_out), _ptr(cu_seqlens),
                                         _ptr(conv_state_in), _ptr(conv_state_out), _ptr(initial_state),
                                         _ptr(final_state), _ptr(out), _ptr(workspace), workspace.numel(),
                                         _stream(dev))
    _lib.check("gdr_delta_layer_fwd", st)
    return out, final_state, conv_state_out


def attn_desc(T, N, Hq, Hk, D=256, cache_len=0, eps=1e-6, rope_base=1.0e7):
    d = _lib.GdrAttnDesc()
    d.struct_size = ctypes.sizeof(_lib.GdrAttnDesc)
    d.num_tokens, d.num_seqs, d.num_q_heads, d.num_kv_heads, d.head_dim = T, N, Hq, Hk, D
    d.cache_len, d.norm_eps, d.rope_base = cache_len, eps, rope_base
    return d


def attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor, q_norm_w: torch.Tensor,
                 k_norm_w: torch.Tensor, cu_seqlens: torch.Tensor, k_cache: Optional[torch.Tensor] = None,
                 v_cache: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, eps: float = 1e-6, rope_base: float = 1.0e7):
    """Causal global attention prefill (gdr_attn_prefill).

    q, gate: [T, Hq, 256] bf16; k, v: [T, Hk, 256] bf16; norm weights [256]
    fp32; cu_seqlens int32 [N+1]; optional k_cache [N, L, Hk, 256] and
    v_cache [N, Hk, L / 32, 256, 32] bf16 (L a multiple of 64; the blocked
    layout include/gdr.h defines) receive the rotated keys and the values.
    Returns out [T, Hq, 256] bf16.
    """
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate")):
        _need(t, name, (torch.bfloat16,), dev)
    _need(q_norm_w, "q_norm_w", (torch.float32,), dev)
    _need(k_norm_w, "k_norm_w", (torch.float32,), dev)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,), dev)
    T, Hq, D = q.shape
    Hk = k.shape[1]
    if k.shape != (T, Hk, D) or v.shape != (T, Hk, D) or gate.shape != (T, Hq, D):
        raise ValueError("shape mismatch among q, k, v, gate")
    N = cu_seqlens.numel() - 1
    cache_len = 0
    if k_cache is not None:
        _need(k_cache, "k_cache", (torch.bfloat16,), dev)
        _need(v_cache, "v_cache", (torch.bfloat16,), dev)
        cache_len = k_cache.shape[1]
        if k_cache.shape != (N, cache_len, Hk, D) or v_cache.shape != (N, Hk, cache_len // 32, D, 32):
            raise ValueError(f"caches must be [N, L, {Hk}, {D}] and [N, {Hk}, L / 32, {D}, 32]")
    d = attn_desc(T, N, Hq, Hk, D, cache_len, eps, rope_base)
    if workspace is None:
        nb = ctypes.c_size_t(0)
        _lib.check("gdr_attn_prefill_workspace_size",
                   _lib.load().gdr_attn_prefill_workspace_size(ctypes.byref(d), ctypes.byref(nb)))
        workspace = torch.empty(max(nb.value, 1), device=dev, dtype=torch.uint8)
    if out is None:
        out = torch.empty((T, Hq, D), device=dev, dtype=torch.bfloat16)
    st = _lib.load().gdr_attn_prefill(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w),
                                      _ptr(k_norm_w), _ptr(cu_seqlens), _ptr(out), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check("gdr_attn_prefill", st)
    return out


def attn_qk_norm_rope(q: torch.Tensor, k: torch.Tensor, q_norm_w: torch.Tensor, k_norm_w: torch.Tensor,
                      cu_seqlens: torch.Tensor, eps: float = 1e-6, rope_base: float = 1.0e7):
    """q' and k' (RMS norm + rotary) of a packed batch (gdr_attn_qk_norm_rope)."""
    dev = q.device
    _need(q, "q", (torch.bfloat16,), dev)
    _need(k, "k", (torch.bfloat16,), dev)
    _need(q_norm_w, "q_norm_w", (torch.float32,), dev)
    _need(k_norm_w, "k_norm_w", (torch.float32,), dev)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,), dev)
    T, Hq, D = q.shape
    Hk = k.shape[1]
    q_out, k_out = torch.empty_like(q), torch.empty_like(k)
    d = attn_desc(T, cu_seqlens.numel() - 1, Hq, Hk, D, 0, eps, rope_base)
    st = _lib.load().gdr_attn_qk_norm_rope(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(q_norm_w), _ptr(k_norm_w),
                                           _ptr(cu_seqlens), _ptr(q_out), _ptr(k_out), _stream(dev))
    _lib.check("gdr_attn_qk_norm_rope", st)
    return q_out, k_out


def attn_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor, q_norm_w: torch.Tensor,
                k_norm_w: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, cache_lens: torch.Tensor,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, eps: float = 1e-6,
                rope_base: float = 1.0e7):
    """One decode token per sequence (gdr_attn_decode).

    q, gate: [N, Hq, 256]; k, v: [N, Hk, 256] bf16; k_cache [N, L, Hk, 256],
    v_cache [N, Hk, L / 32, 256, 32] bf16 updated in place at cache_lens[n];
    cache_lens int32 [N] (not advanced).  Returns out [N, Hq, 256] bf16.
    """
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, name, (torch.bfloat16,), dev)
    _need(q_norm_w, "q_norm_w", (torch.float32,), dev)
    _need(k_norm_w, "k_norm_w", (torch.float32,), dev)
    _need(cache_lens, "cache_lens", (torch.int32,), dev)
    N, Hq, D = q.shape
    Hk = k.shape[1]
    L = k_cache.shape[1]
    if k.shape != (N, Hk, D) or v.shape != (N, Hk, D) or gate.shape != (N, Hq, D) \
            or k_cache.shape != (N, L, Hk, D) or v_cache.shape != (N, Hk, L // 32, D, 32) \
            or cache_lens.shape != (N,):
        raise ValueError("shape mismatch in attention decode inputs")
    d = attn_desc(N, N, Hq, Hk, D, L, eps, rope_base)
    if workspace is None:
        nb = ctypes.c_size_t(0)
        _lib.check("gdr_attn_decode_workspace_size",
                   _lib.load().gdr_attn_decode_workspace_size(ctypes.byref(d), ctypes.byref(nb)))
        workspace = torch.empty(max(nb.value, 1), device=dev, dtype=torch.uint8)
    if out is None:
        out = torch.empty((N, Hq, D), device=dev, dtype=torch.bfloat16)
    st = _lib.load().gdr_attn_decode(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w),
                                     _ptr(k_norm_w), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens), _ptr(out),
                                     _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check("gdr_attn_decode", st)
    return out
