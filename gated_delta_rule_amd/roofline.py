"""ctypes view of libgdr_roofline.so (include/gdr_roofline.h): launch-only
probes of the achievable HBM streaming rate and bf16 matrix-core rate, which
the benchmark times with events beside the path's own kernels."""
import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdr_roofline.so")
EXPORTED = ("gdr_roofline_rmw", "gdr_roofline_read", "gdr_roofline_mfma", "gdr_roofline_valu",
            "gdr_probe_silu_mid", "gdr_probe_bf16_rne")
SLAB = 65536  # bytes per workgroup of the streaming probes
MFMA_FLOP_PER_WAVE_ITER = 8 * 16 * 16 * 32 * 2
VALU_INSTS_PER_WAVE_ITER = 16

_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libgdr_roofline.so (once); raises ImportError if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (python -m gated_delta_rule_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        P, Z = ctypes.c_void_p, ctypes.c_size_t
        lib.gdr_roofline_rmw.argtypes = [P, Z, ctypes.c_float, ctypes.c_int, P]
        lib.gdr_roofline_read.argtypes = [P, Z, P, P]
        lib.gdr_roofline_mfma.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
        lib.gdr_roofline_valu.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
        for name in ("gdr_probe_silu_mid", "gdr_probe_bf16_rne"):
            getattr(lib, name).argtypes = [ctypes.c_uint32, ctypes.c_ulonglong, P, P, P]
        for name in EXPORTED:
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(name: str, status: int) -> None:
    if status != 0:
        raise RuntimeError(f"{name} returned {status}")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def rmw(buf: torch.Tensor, scale: float = 1.0, nontemporal: bool = False) -> None:
    """In place buf *= scale, 64 KiB per workgroup (fp32, numel*4 a multiple of 65536)."""
    _check("gdr_roofline_rmw", load().gdr_roofline_rmw(buf.data_ptr(), buf.numel() * 4, scale, int(nontemporal),
                                                       _stream(buf)))


def read(buf: torch.Tensor, sums: torch.Tensor) -> None:
    """sums[i] = sum of the i-th 64 KiB slab of buf (fp32)."""
    _check("gdr_roofline_read", load().gdr_roofline_read(buf.data_ptr(), buf.numel() * 4, sums.data_ptr(),
                                                         _stream(buf)))


def mfma(out: torch.Tensor, workgroups: int, iters: int) -> None:
    """workgroups x 4 waves, each iters x 8 bf16 16x16x32 matrix-core ops."""
    _check("gdr_roofline_mfma", load().gdr_roofline_mfma(out.data_ptr(), workgroups, iters, _stream(out)))


def valu(out: torch.Tensor, workgroups: int, iters: int) -> None:
    """workgroups x 4 waves, each iters x 16 independent fp32 VALU instructions."""
    _check("gdr_roofline_valu", load().gdr_roofline_valu(out.data_ptr(), workgroups, iters, _stream(out)))


def contract_probe(name: str, first_bits: int, count: int, device) -> tuple:
    """Run gdr_probe_<name> over count fp32 patterns from first_bits; returns
    (mismatches, smallest failing pattern or None)."""
    bad = torch.zeros(1, device=device, dtype=torch.int64)
    first = torch.full((1,), -1, device=device, dtype=torch.int32)  # 0xffffffff
    fn = getattr(load(), f"gdr_probe_{name}")
    _check(f"gdr_probe_{name}", fn(first_bits, count, bad.data_ptr(), first.data_ptr(), _stream(bad)))
    torch.cuda.synchronize(device)
    n = int(bad.item())
    f = int(first.item()) & 0xFFFFFFFF
    return n, (None if n == 0 else f)
