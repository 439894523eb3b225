"""Shared test utilities: tensor transfer and the parity metrics."""
from __future__ import annotations

import sys

import numpy as np

BF16_TOL = 2e-3  # max |gpu - ref| / RMS(ref), bf16 q/k/v with fp32 state
F32_TOL = 1e-5   # same metric, all-fp32 inputs


def say(*msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(*msg, file=sys.stderr, flush=True)


def gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, dtype: str, dev):
    """Host float32 array (bf16-representable if dtype == 'bf16') -> device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f32":
        t = t.to(torch.float32)
    elif dtype == "i32":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32))
    else:
        raise ValueError(dtype)
    return t.to(dev)


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_err(x, ref) -> float:
    """max |x - ref| / RMS(ref)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0:
        return float(np.max(np.abs(x - ref)))
    return float(np.max(np.abs(x - ref)) / rms)


def bf16_ulp(x) -> np.ndarray:
    e = np.floor(np.log2(np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def bits_equal(a, b) -> bool:
    """Bit-identical tensors (NaN payloads included)."""
    import torch
    a = a.detach().contiguous()
    b = b.detach().contiguous()
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    iv = {torch.float32: torch.int32, torch.bfloat16: torch.int16}[a.dtype]
    return bool(torch.equal(a.view(iv), b.view(iv)))


# The decode V cache is blocked by 32 positions (include/gdr.h): position
# 32 b + i of dim d sits at [n][h][b][d][VC_POS[i]]; VC_KEY is the inverse.
VC_POS = [8 * ((i % 16) // 4) + 4 * (i // 16) + i % 4 for i in range(32)]
VC_KEY = [VC_POS.index(p) for p in range(32)]


def _tp(x, dims):
    return x.permute(*dims) if hasattr(x, "permute") else np.transpose(x, dims)


def _contig(x):
    return x.contiguous() if hasattr(x, "contiguous") else np.ascontiguousarray(x)


def v_cache_blocked(vnat):
    """Natural values [N, L, Hk, D] -> the decode V cache [N, Hk, L / 32, D, 32]
    (numpy or torch)."""
    N, L, Hk, D = vnat.shape
    x = vnat.reshape(N, L // 32, 32, Hk, D)[:, :, VC_KEY]  # [N, b, position, Hk, D]
    return _contig(_tp(x, (0, 3, 1, 4, 2)))


def v_cache_natural(vb):
    """The decode V cache [N, Hk, L / 32, D, 32] -> natural values [N, L, Hk, D]."""
    N, Hk, B, D, _ = vb.shape
    x = _tp(vb, (0, 2, 4, 1, 3))[:, :, VC_POS]  # [N, b, key, Hk, D]
    return _contig(x.reshape(N, B * 32, Hk, D))
