"""ctypes view of libgdr.so (include/gdr.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_OK, GDR_ERR_INVALID_ARG, GDR_ERR_UNSUPPORTED, GDR_ERR_HIP = 0, -1, -2, -3
GDR_F32, GDR_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20  # GDR_NOALLOC_SCRATCH_BYTES

EXPORTED = (
    "gdr_abi_version",
    "gdr_status_string",
    "gdr_last_error",
    "gdr_chunk_fwd_workspace_size",
    "gdr_chunk_fwd",
    "gdr_chunk_fwd_prepare",
    "gdr_chunk_fwd_recurrence",
    "gdr_chunk_fwd_noalloc",
    "gdr_recurrent_step",
    "gdr_recurrent_step_indexed",
    "gdr_decode_layer_step",
    "gdr_conv_gate_fused",
    "gdr_gated_rmsnorm",
    "gdr_linear",
    "gdr_delta_layer_workspace_size",
    "gdr_delta_layer_fwd",
    "gdr_attn_qk_norm_rope",
    "gdr_attn_prefill_workspace_size",
    "gdr_attn_prefill",
    "gdr_attn_decode_workspace_size",
    "gdr_attn_decode",
)


class GdrDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_dim_k", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("use_qk_l2norm", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("l2norm_eps", ctypes.c_float),
    ]


class GdrConvDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_tokens", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


class GdrNormDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("o_dtype", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


class GdrLinearOut(ctypes.Structure):
    _fields_ = [
        ("ptr", ctypes.c_void_p),
        ("ld", ctypes.c_int64),
        ("cols", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("round_bf16", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class GdrLayerDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_tokens", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("l2norm_eps", ctypes.c_float),
        ("norm_eps", ctypes.c_float),
    ]


class GdrAttnDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_tokens", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("cache_len", ctypes.c_int32),
        ("norm_eps", ctypes.c_float),
        ("rope_base", ctypes.c_double),
    ]


class GDRError(RuntimeError):
    """A libgdr entry point returned a negative status."""

    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func} failed with {status_string(status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libgdr.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_amd.build` "
            "(hipcc, gfx950). There is no non-HIP implementation of this library.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gdr_abi_version.restype = I32
    lib.gdr_abi_version.argtypes = []
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_status_string.argtypes = [I32]
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_last_error.argtypes = []
    lib.gdr_chunk_fwd_workspace_size.restype = I32
    lib.gdr_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(GdrDesc), ctypes.POINTER(SZ)]
    for name in ("gdr_chunk_fwd", "gdr_chunk_fwd_prepare", "gdr_chunk_fwd_recurrence"):
        fn = getattr(lib, name)
        fn.restype = I32
        fn.argtypes = [ctypes.POINTER(GdrDesc), P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.gdr_chunk_fwd_noalloc.restype = I32
    lib.gdr_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(GdrDesc), P, P, P, P, P, P, P, P, P, P]
    lib.gdr_recurrent_step.restype = I32
    lib.gdr_recurrent_step.argtypes = [ctypes.POINTER(GdrDesc), P, P, P, P, P, P, P, P]
    lib.gdr_recurrent_step_indexed.restype = I32
    lib.gdr_recurrent_step_indexed.argtypes = [ctypes.POINTER(GdrDesc), P, P, P, P, P, P, ctypes.c_int32, P, P, P]
    lib.gdr_decode_layer_step.restype = I32
    lib.gdr_decode_layer_step.argtypes = ([ctypes.POINTER(GdrDesc)] + [P] * 8 + [ctypes.c_int32, P, P, P, F]
                                          + [P] * 4)
    lib.gdr_conv_gate_fused.restype = I32
    lib.gdr_conv_gate_fused.argtypes = [ctypes.POINTER(GdrConvDesc)] + [P] * 15
    lib.gdr_gated_rmsnorm.restype = I32
    lib.gdr_gated_rmsnorm.argtypes = [ctypes.POINTER(GdrNormDesc), P, P, P, P, P]
    I64 = ctypes.c_int64
    lib.gdr_linear.restype = I32
    lib.gdr_linear.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, I64, P, I64,
                               ctypes.POINTER(GdrLinearOut), ctypes.c_int32, P]
    lib.gdr_delta_layer_workspace_size.restype = I32
    lib.gdr_delta_layer_workspace_size.argtypes = [ctypes.POINTER(GdrLayerDesc), ctypes.POINTER(SZ)]
    lib.gdr_delta_layer_fwd.restype = I32
    lib.gdr_delta_layer_fwd.argtypes = [ctypes.POINTER(GdrLayerDesc)] + [P] * 14 + [SZ, P]
    lib.gdr_attn_qk_norm_rope.restype = I32
    lib.gdr_attn_qk_norm_rope.argtypes = [ctypes.POINTER(GdrAttnDesc)] + [P] * 8
    lib.gdr_attn_prefill_workspace_size.restype = I32
    lib.gdr_attn_prefill_workspace_size.argtypes = [ctypes.POINTER(GdrAttnDesc), ctypes.POINTER(SZ)]
    lib.gdr_attn_prefill.restype = I32
    lib.gdr_attn_prefill.argtypes = [ctypes.POINTER(GdrAttnDesc)] + [P] * 11 + [SZ, P]
    lib.gdr_attn_decode_workspace_size.restype = I32
    lib.gdr_attn_decode_workspace_size.argtypes = [ctypes.POINTER(GdrAttnDesc), ctypes.POINTER(SZ)]
    lib.gdr_attn_decode.restype = I32
    lib.gdr_attn_decode.argtypes = [ctypes.POINTER(GdrAttnDesc)] + [P] * 11 + [SZ, P]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gdr_status_string(status).decode()


def check(func: str, status: int) -> None:
    if status != GDR_OK:
        raise GDRError(func, status, load().gdr_last_error().decode())
