"""The C ABI on the CPU: the library loads, exports what include/gdr.h declares,
and rejects bad arguments synchronously, before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from gated_delta_rule_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header():
    lib = _lib.load()
    declared = _declared()
    assert declared == sorted(_lib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)
    assert lib.gdr_abi_version() == 1


def test_status_strings():
    assert _lib.status_string(0) == "GDR_OK"
    assert _lib.status_string(-1) == "GDR_ERR_INVALID_ARG"
    assert _lib.status_string(-2) == "GDR_ERR_UNSUPPORTED"
    assert _lib.status_string(-3) == "GDR_ERR_HIP"
    assert _lib.status_string(7) == "GDR_UNKNOWN_STATUS"


def _desc(**kw):
    d = _lib.GdrDesc()
    d.struct_size = ctypes.sizeof(_lib.GdrDesc)
    base = dict(batch=1, seq_len=128, num_seqs=1, num_k_heads=16, num_v_heads=48, head_dim_k=128,
                head_dim_v=128, chunk_size=64, qkv_dtype=1, out_dtype=0, use_qk_l2norm=1, scale=1.0,
                l2norm_eps=1e-6)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


FAKE = 0x7F0000000000  # never dereferenced: every case below fails validation first


CHUNK_ENTRIES = ("gdr_chunk_fwd", "gdr_chunk_fwd_prepare", "gdr_chunk_fwd_recurrence")


def _chunk(d, q=FAKE, cu=None, o=FAKE, init=None, fin=None, entry="gdr_chunk_fwd"):
    lib = _lib.load()
    return getattr(lib, entry)(ctypes.byref(d) if d is not None else None, q, FAKE, FAKE, FAKE, FAKE, init, fin,
                               cu, o, None, 0, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(num_v_heads=40), -1, "multiple"),
    (dict(head_dim_k=96, head_dim_v=96), -2, "head dims"),
    (dict(head_dim_k=128, head_dim_v=64), -2, "head dims"),
    (dict(chunk_size=48), -2, "chunk_size"),
    (dict(qkv_dtype=5), -1, "dtype"),
    (dict(batch=2, num_seqs=3), -1, "num_seqs"),
    (dict(seq_len=-1), -1, "negative"),
    (dict(num_k_heads=0), -1, "positive"),
    (dict(l2norm_eps=-1.0), -1, "eps"),
    (dict(struct_size=8), -1, "struct_size"),
    (dict(num_k_heads=1, num_v_heads=65), -2, "value heads per key head"),
])
@pytest.mark.parametrize("entry", CHUNK_ENTRIES)
def test_chunk_fwd_rejects_bad_descriptors(kw, status, msg, entry):
    assert _chunk(_desc(**kw), entry=entry) == status
    assert msg in _lib.load().gdr_last_error().decode()


@pytest.mark.parametrize("entry", CHUNK_ENTRIES)
def test_chunk_fwd_rejects_null_and_misaligned(entry):
    lib = _lib.load()
    assert _chunk(None, entry=entry) == -1
    assert _chunk(_desc(), q=None, entry=entry) == -1 and "required" in lib.gdr_last_error().decode()
    assert _chunk(_desc(), q=FAKE + 2, entry=entry) == -1 and "aligned" in lib.gdr_last_error().decode()
    assert _chunk(_desc(), fin=FAKE + 4, entry=entry) == -1
    assert _chunk(_desc(batch=2, num_seqs=2), cu=FAKE, entry=entry) == -1  # packed batch needs batch == 1
    # a bf16 d=128 call needs the workspace in either stage
    assert _chunk(_desc(), entry=entry) == -1 and "workspace" in lib.gdr_last_error().decode()


def test_workspace_size():
    lib = _lib.load()
    n = ctypes.c_size_t(123)
    rec, table = 25728, 256
    # bf16, d = 128, chunk 64: chunk table + one record per (chunk, value head)
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(_desc()), ctypes.byref(n)) == 0
    assert n.value == table + (2 + 1) * 48 * rec  # T = 128: 2 chunks, + 1 for a packed batch
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(_desc(batch=1, num_seqs=8, seq_len=1000)),
                                            ctypes.byref(n)) == 0
    assert n.value == table + (16 + 8) * 48 * rec
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(_desc(batch=3, num_seqs=3)), ctypes.byref(n)) == 0
    assert n.value == table + 3 * 2 * 48 * rec
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(_desc(qkv_dtype=0)), ctypes.byref(n)) == 0 and n.value == 0
    # a call that needs a workspace and gets none fails before any launch
    assert _chunk(_desc()) == -1 and "workspace" in lib.gdr_last_error().decode()
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(_desc(chunk_size=16)), ctypes.byref(n)) == -2
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(_desc()), None) == -1


def test_recurrent_step_validation():
    lib = _lib.load()
    d = _desc(batch=4, num_seqs=4, seq_len=1)
    args = [FAKE] * 5
    assert lib.gdr_recurrent_step(ctypes.byref(_desc(batch=4, num_seqs=4, seq_len=2)), *args, FAKE, FAKE, None) == -1
    assert lib.gdr_recurrent_step(ctypes.byref(d), *args, None, FAKE, None) == -1
    assert lib.gdr_recurrent_step(ctypes.byref(d), *args, FAKE + 8, FAKE, None) == -1
    assert "aligned" in lib.gdr_last_error().decode()
    ix = lib.gdr_recurrent_step_indexed
    assert ix(ctypes.byref(d), *args, FAKE, -1, FAKE, FAKE, None) == -1 and "pool_size" in lib.gdr_last_error().decode()
    assert ix(ctypes.byref(d), *args, FAKE, 8, None, FAKE, None) == -1 and "state_indices" in lib.gdr_last_error().decode()
    assert ix(ctypes.byref(d), *args, None, 8, FAKE, FAKE, None) == -1  # a NULL pool only when it is empty
    assert ix(ctypes.byref(d), *args, FAKE + 8, 8, FAKE, FAKE, None) == -1
    assert ix(ctypes.byref(_desc(batch=4, num_seqs=4, seq_len=2)), *args, FAKE, 8, FAKE, FAKE, None) == -1


def test_decode_layer_step_validation():
    lib = _lib.load()
    f = lib.gdr_decode_layer_step
    d = _desc(batch=4, num_seqs=4, seq_len=1)

    def call(desc, state=FAKE, pool=8, x=FAKE, conv_w=FAKE):
        return f(ctypes.byref(desc), x, conv_w, FAKE, FAKE, FAKE, FAKE, FAKE, state, pool, FAKE, FAKE, FAKE, 1e-6,
                 FAKE, None, None, None)

    assert call(_desc(batch=4, num_seqs=4, seq_len=2)) == -1
    assert call(_desc(batch=4, num_seqs=4, seq_len=1, head_dim_k=64, head_dim_v=64)) == -2
    assert call(_desc(batch=4, num_seqs=4, seq_len=1, num_k_heads=1, num_v_heads=5)) == -2
    assert call(_desc(batch=4, num_seqs=4, seq_len=1, qkv_dtype=0)) == -2
    assert call(d, pool=-1) == -1 and "pool_size" in lib.gdr_last_error().decode()
    assert call(d, x=None) == -1
    assert call(d, state=FAKE + 4) == -1 and "aligned" in lib.gdr_last_error().decode()
    assert call(d, conv_w=FAKE + 2) == -1
    assert call(_desc(batch=0, num_seqs=0, seq_len=1)) == 0  # nothing to do


def test_conv_and_norm_validation():
    lib = _lib.load()
    c = _lib.GdrConvDesc()
    c.struct_size = ctypes.sizeof(_lib.GdrConvDesc)
    c.num_tokens, c.num_seqs, c.num_k_heads, c.num_v_heads, c.head_dim = 16, 1, 16, 48, 128
    ptrs = [FAKE] * 14
    assert lib.gdr_conv_gate_fused(ctypes.byref(c), FAKE, FAKE, None, *ptrs[3:], None) == -1  # no cu_seqlens
    # conv_state_out aliasing conv_state_in
    assert lib.gdr_conv_gate_fused(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, *ptrs[5:], None) == -1
    assert "alias" in lib.gdr_last_error().decode()
    c.head_dim = 100
    assert lib.gdr_conv_gate_fused(ctypes.byref(c), *([FAKE] * 15)) == -2
    n = _lib.GdrNormDesc()
    n.struct_size = ctypes.sizeof(_lib.GdrNormDesc)
    n.num_tokens, n.num_heads, n.head_dim, n.o_dtype, n.eps = 4, 48, 96, 0, 1e-6
    assert lib.gdr_gated_rmsnorm(ctypes.byref(n), FAKE, FAKE, FAKE, FAKE, None) == -2
    n.head_dim = 128
    assert lib.gdr_gated_rmsnorm(ctypes.byref(n), FAKE, FAKE, FAKE, FAKE + 2, None) == -1
    assert lib.gdr_gated_rmsnorm(None, FAKE, FAKE, FAKE, FAKE, None) == -1


def _blocks(*specs):
    arr = (_lib.GdrLinearOut * len(specs))()
    for i, (ptr, ld, cols, dt, rnd) in enumerate(specs):
        arr[i].ptr, arr[i].ld, arr[i].cols, arr[i].dtype, arr[i].round_bf16 = ptr, ld, cols, dt, rnd
    return arr


def test_linear_validation():
    lib = _lib.load()
    ok = _blocks((FAKE, 256, 256, 1, 0))
    assert lib.gdr_linear(4, 256, 200, FAKE, 200, FAKE, 200, ok, 1, None) == -1  # K not a multiple of 32
    assert "multiple of 32" in lib.gdr_last_error().decode()
    assert lib.gdr_linear(4, 256, 256, FAKE, 200, FAKE, 256, ok, 1, None) == -1  # ldx not a multiple of 8
    assert lib.gdr_linear(4, 256, 256, FAKE, 128, FAKE, 256, ok, 1, None) == -1  # ldx < K
    assert lib.gdr_linear(4, 256, 256, FAKE + 8, 256, FAKE, 256, ok, 1, None) == -1  # x misaligned
    assert lib.gdr_linear(4, 256, 256, FAKE, 256, FAKE, 256, ok, 0, None) == -1  # no blocks
    assert lib.gdr_linear(4, 256, 256, FAKE, 256, FAKE, 256, ok, 5, None) == -1  # too many
    assert lib.gdr_linear(4, 260, 256, FAKE, 256, FAKE, 256, ok, 1, None) == -1  # widths != N
    assert "sum" in lib.gdr_last_error().decode()
    assert lib.gdr_linear(4, 8, 256, FAKE, 256, FAKE, 256, _blocks((FAKE + 2, 8, 8, 0, 0)), 1, None) == -1
    assert lib.gdr_linear(4, 8, 256, FAKE, 256, FAKE, 256, _blocks((FAKE + 1, 8, 8, 1, 0)), 1, None) == -1
    assert lib.gdr_linear(4, 8, 256, FAKE, 256, FAKE, 256, _blocks((FAKE, 8, -1, 1, 0), (FAKE, 8, 9, 1, 0)),
                          2, None) == -1
    assert lib.gdr_linear(4, 8, 256, FAKE, 256, FAKE, 256, _blocks((None, 8, 8, 1, 0)), 1, None) == -1
    assert lib.gdr_linear(4, 8, 256, FAKE, 256, FAKE, 256, _blocks((FAKE, 4, 8, 1, 0)), 1, None) == -1  # ld<w
    assert lib.gdr_linear(4, 8, 256, FAKE, 256, FAKE, 256, _blocks((FAKE, 8, 8, 7, 0)), 1, None) == -1  # dtype
    assert lib.gdr_linear(-1, 8, 256, FAKE, 256, FAKE, 256, ok, 1, None) == -1
    # nothing to compute: accepted without a launch
    assert lib.gdr_linear(0, 256, 256, None, 256, None, 256, _blocks((None, 256, 256, 1, 0)), 1, None) == 0


def test_delta_layer_validation_and_workspace():
    lib = _lib.load()
    d = _lib.GdrLayerDesc()
    d.struct_size = ctypes.sizeof(_lib.GdrLayerDesc)
    d.num_tokens, d.num_seqs, d.hidden = 32768, 1, 5120
    d.num_k_heads, d.num_v_heads, d.head_dim = 16, 48, 128
    d.l2norm_eps = d.norm_eps = 1e-6
    n = ctypes.c_size_t(0)
    assert lib.gdr_delta_layer_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    T, C, V = 32768, 10240, 6144
    inter = T * (2 * C + 2 * V + 4 * 48 * 4 + 2 * C) + T * V * 4
    assert inter <= n.value < inter + 700 * 2 ** 20  # plus the recurrence's per-chunk records
    d.head_dim = 64
    assert lib.gdr_delta_layer_workspace_size(ctypes.byref(d), ctypes.byref(n)) == -2
    d.head_dim, d.hidden = 128, 5000
    assert lib.gdr_delta_layer_workspace_size(ctypes.byref(d), ctypes.byref(n)) == -1
    d.hidden = 5120
    args = [FAKE] * 14
    assert lib.gdr_delta_layer_fwd(ctypes.byref(d), *args, 10, None) == -1  # short workspace
    assert "workspace" in lib.gdr_last_error().decode()
    args[7] = None  # no cu_seqlens
    assert lib.gdr_delta_layer_fwd(ctypes.byref(d), *args, 1 << 40, None) == -1
    assert lib.gdr_delta_layer_fwd(None, *([FAKE] * 14), 1 << 40, None) == -1


def _attn_desc(T=64, N=1, hq=24, hk=4, d=256, L=0):
    a = _lib.GdrAttnDesc()
    a.struct_size = ctypes.sizeof(_lib.GdrAttnDesc)
    a.num_tokens, a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim = T, N, hq, hk, d
    a.cache_len, a.norm_eps, a.rope_base = L, 1e-6, 1e7
    return a


def test_attention_validation_and_workspace():
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    d = _attn_desc(T=32768)
    assert lib.gdr_attn_prefill_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    q_rot = 32768 * 24 * 256 * 2
    assert q_rot < n.value < q_rot + 2 * (32768 + 128) * 4 * 256 * 2 + 4096
    assert lib.gdr_attn_prefill_workspace_size(ctypes.byref(_attn_desc(d=128)), ctypes.byref(n)) == -2
    assert lib.gdr_attn_prefill_workspace_size(ctypes.byref(_attn_desc(hq=10)), ctypes.byref(n)) == -2
    assert lib.gdr_attn_prefill_workspace_size(ctypes.byref(_attn_desc(N=0)), ctypes.byref(n)) == -1
    P = [FAKE] * 11
    d = _attn_desc()
    assert lib.gdr_attn_prefill(ctypes.byref(d), *P, 16, None) == -1  # short workspace
    args = list(P)
    args[9] = None  # k_cache without v_cache
    assert lib.gdr_attn_prefill(ctypes.byref(d), *args, 1 << 40, None) == -1
    assert "both" in lib.gdr_last_error().decode()
    d = _attn_desc(L=100)  # cache_len not a multiple of 64
    assert lib.gdr_attn_prefill(ctypes.byref(d), *P, 1 << 40, None) == -1
    args = list(P)
    args[6] = None  # no cu_seqlens
    assert lib.gdr_attn_prefill(ctypes.byref(_attn_desc()), *args, 1 << 40, None) == -1
    # decode
    dd = _attn_desc(T=64, N=64, L=32768)
    assert lib.gdr_attn_decode_workspace_size(ctypes.byref(dd), ctypes.byref(n)) == 0
    assert n.value >= 64 * 24 * 256 * 2
    assert lib.gdr_attn_decode_workspace_size(ctypes.byref(_attn_desc(T=64, N=64, L=0)), ctypes.byref(n)) == -1
    assert lib.gdr_attn_decode_workspace_size(ctypes.byref(_attn_desc(T=3, N=64, L=64)), ctypes.byref(n)) == -1
    assert lib.gdr_attn_decode(ctypes.byref(dd), *P, 16, None) == -1  # short workspace
    args = list(P)
    args[8] = None  # no cache_lens
    assert lib.gdr_attn_decode(ctypes.byref(dd), *args, 1 << 40, None) == -1
    assert lib.gdr_attn_decode(ctypes.byref(dd), *[FAKE + 8] + P[1:], 1 << 40, None) == -1  # misaligned q
    assert lib.gdr_attn_qk_norm_rope(ctypes.byref(_attn_desc()), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                     None) == -1


def test_no_oracle_in_product_path():
    """The library and its binding never import the oracle."""
    pkg = os.path.join(ROOT, "gated_delta_rule_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", src, flags=re.M), f
                assert "oracle/" not in src and "oracle." not in src, f


def test_chunk_fwd_noalloc_rejects_calls_beyond_the_scratch():
    """A call whose workspace exceeds the static scratch fails before any
    HIP call (no device is touched on this CPU-only host)."""
    lib = _lib.load()
    d = _desc(seq_len=1 << 20)
    nbytes = ctypes.c_size_t(0)
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(d), ctypes.byref(nbytes)) == 0
    assert nbytes.value > _lib.NOALLOC_SCRATCH_BYTES
    st = lib.gdr_chunk_fwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None)
    assert st == -1
    assert "static scratch" in lib.gdr_last_error().decode()
    # bad descriptors are rejected as gdr_chunk_fwd rejects them
    st = lib.gdr_chunk_fwd_noalloc(ctypes.byref(_desc(num_v_heads=40)), FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                   None, FAKE, None)
    assert st == -1 and "multiple" in lib.gdr_last_error().decode()
