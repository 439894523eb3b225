"""The roofline probe library: exports what include/gdr_roofline.h declares,
rejects bad arguments before launching (CPU), and computes what it says (GPU)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from gated_delta_rule_amd import roofline
from helpers import gpu, say

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_match_header():
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "gdr_roofline.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(gdr_[a-z0-9_]+)\s*\(", text)))
    assert declared == sorted(roofline.EXPORTED)
    roofline.load()
    out = subprocess.run(["nm", "-D", "--defined-only", roofline.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared) <= exported


def test_bad_arguments_rejected_before_launch():
    lib = roofline.load()
    fake = ctypes.c_void_p(1 << 20)
    assert lib.gdr_roofline_rmw(None, 65536, 1.0, 0, None) == -1
    assert lib.gdr_roofline_rmw(fake, 65536 + 16, 1.0, 0, None) == -1
    assert lib.gdr_roofline_rmw(fake, 0, 1.0, 1, None) == -1
    assert lib.gdr_roofline_read(fake, 65536, None, None) == -1
    assert lib.gdr_roofline_read(fake, 1000, fake, None) == -1
    assert lib.gdr_roofline_mfma(fake, 0, 10, None) == -1
    assert lib.gdr_roofline_mfma(None, 4, 10, None) == -1
    assert lib.gdr_roofline_valu(fake, 4, 0, None) == -1
    assert lib.gdr_roofline_valu(None, 4, 10, None) == -1


@pytest.mark.gpu
def test_probes_compute_what_they_say():
    import torch
    dev = gpu()
    say("roofline probes: rmw, read, mfma, valu")
    n = 4 * 65536 // 4
    x = torch.arange(n, device=dev, dtype=torch.float32) % 1000
    ref = x.clone()
    roofline.rmw(x, 2.0)
    roofline.rmw(x, 0.5, nontemporal=True)
    torch.cuda.synchronize()
    assert torch.equal(x, ref)
    roofline.rmw(x, 3.0, nontemporal=True)
    torch.cuda.synchronize()
    assert torch.equal(x, ref * 3.0)
    sums = torch.empty(4, device=dev)
    roofline.read(ref, sums)
    torch.cuda.synchronize()
    expect = ref.view(4, -1).double().sum(1).cpu().numpy()
    assert np.allclose(sums.cpu().numpy(), expect, rtol=1e-6)
    out = torch.full((8 * 4,), float("nan"), device=dev)
    roofline.mfma(out, 8, 3)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    # the VALU probe's lane 0 runs a <- a * 0.999f (c = 0) on a = 1..8, in
    # fp32 with the multiply rounded on its own, and writes the chains' sum
    out = torch.full((8 * 4,), float("nan"), device=dev)
    roofline.valu(out, 8, 5)
    torch.cuda.synchronize()
    m = np.float32(0.999)
    acc = [np.float32(u + 1) for u in range(8)]
    for _ in range(5):
        acc = [np.float32(a * m) + np.float32(0) for a in acc]
    r = np.float32(0)
    for a in acc:
        r = np.float32(r + a)
    assert np.all(out.cpu().numpy() == r)


def test_contract_probes_reject_bad_arguments():
    lib = roofline.load()
    fake = ctypes.c_void_p(1 << 20)
    for name in ("gdr_probe_silu_mid", "gdr_probe_bf16_rne"):
        fn = getattr(lib, name)
        assert fn(0, 0, fake, fake, None) == -1
        assert fn(0, (1 << 32) + 1, fake, fake, None) == -1
        assert fn(0, 16, None, fake, None) == -1


@pytest.mark.gpu
def test_conv_silu_shortcut_equals_ieee_division_on_all_of_minus80_to_80():
    """The conv kernel's SiLU for |v| <= 80 (rcp plus one residual
    correction) gives the contract's IEEE-division SiLU bit for bit on every
    fp32 value in [-80, 80] (about 2.2e9 patterns)."""
    dev = gpu()
    say("contract probe: silu32_mid vs silu32 on [-80, 80]")
    top = 0x42A00000  # 80.0
    for lo in (0x00000000, 0x80000000):
        n, first = roofline.contract_probe("silu_mid", lo, top + 1, dev)
        assert n == 0, f"{n} mismatches, first at pattern {first:#010x}"


@pytest.mark.gpu
def test_hardware_bf16_conversion_is_round_to_nearest_even():
    """The fp32 -> bf16 conversion the kernels use rounds to nearest even on
    every one of the 2^32 fp32 patterns (NaN to a quiet NaN of its sign)."""
    dev = gpu()
    say("contract probe: fp32 -> bf16 on all 2^32 patterns")
    n, first = roofline.contract_probe("bf16_rne", 0, 1 << 32, dev)
    assert n == 0, f"{n} mismatches, first at pattern {first:#010x}"
