"""Gated delta rule for AMD MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in libgdr.so (include/gdr.h); this package is a thin torch
binding over it.  Importing the ops loads the library and raises ImportError
if it has not been built (``python -m gated_delta_rule_amd.build``).
"""
from ._lib import GDRError, load as load_library  # noqa: F401
from .ops import (  # noqa: F401
    attn_decode,
    attn_prefill,
    attn_qk_norm_rope,
    chunk_gated_delta_rule,
    chunk_workspace,
    conv_gate_fused,
    decode_layer_step,
    delta_layer_fwd,
    delta_layer_workspace,
    gated_rmsnorm,
    linear,
    recurrent_step,
)

__all__ = [
    "GDRError",
    "load_library",
    "chunk_gated_delta_rule",
    "chunk_workspace",
    "recurrent_step",
    "decode_layer_step",
    "conv_gate_fused",
    "gated_rmsnorm",
    "linear",
    "delta_layer_fwd",
    "delta_layer_workspace",
    "attn_prefill",
    "attn_qk_norm_rope",
    "attn_decode",
]
