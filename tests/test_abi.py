"""The C-ABI library loads without a GPU, exports every declared symbol, and
rejects every invalid argument with its status code before any HIP call.
No test here launches a kernel: all pointers are fake addresses that the
validation must reject before they could be used."""

import ctypes
import os
import re
import subprocess

import pytest

from transformer_attention_06_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE, DEVICE = 0, 1, 2, 3, 4
F32, BF16 = native.NC_F32, native.NC_BF16
A = 0x100000  # aligned fake device address (never dereferenced)


def _gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="module")
def L():
    return native.lib()


def msg(L):
    return L.nc_last_error_message().decode()


def test_header_declares_exactly_the_exports():
    with open(os.path.join(ROOT, "include", "ncattn.h")) as f:
        src = f.read()
    declared = set(re.findall(r"\b(nc_[a-z0-9_]+)\s*\(", src))
    assert declared == set(native.EXPORTS)


def test_library_exports_every_symbol(L):
    for name in native.EXPORTS:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", native.LIB_PATH], capture_output=True, text=True).stdout
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in native.EXPORTS:
        assert name in syms, name


def test_version_and_status_strings(L):
    assert L.nc_abi_version() == 1
    assert L.nc_status_string(0) == b"ok"
    for s in range(1, 6):
        assert L.nc_status_string(s) not in (b"ok", b"unknown status")
    assert L.nc_status_string(99) == b"unknown status"


def fwd(L, dt=BF16, B=1, T=64, H=2, Hkv=1, D=64, q=A, k=A, v=A, w=0, scale=0.125, out=A, lse=A):
    return L.nc_attn_fwd(dt, B, T, H, Hkv, D, q, k, v, w, scale, out, lse, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q=None), INVALID, "q is NULL"),
    (dict(v=None), INVALID, "v is NULL"),
    (dict(out=None), INVALID, "out"),
    (dict(lse=None), INVALID, "lse"),
    (dict(B=0), INVALID, "sizes"),
    (dict(T=-1), INVALID, "sizes"),
    (dict(H=3, Hkv=2), INVALID, "multiple"),
    (dict(D=48), UNSUPPORTED, "head dim"),
    (dict(D=256), UNSUPPORTED, "head dim"),
    (dict(dt=7), INVALID, "dtype"),
    (dict(k=A + 8), INVALID, "aligned"),
    (dict(scale=0.0), INVALID, "scale"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(scale=float("inf")), INVALID, "scale"),
    (dict(B=4096, T=4096, H=2, D=128), UNSUPPORTED, "exceeds"),
])
def test_fwd_validation(L, kw, code, needle):
    assert fwd(L, **kw) == code
    assert needle in msg(L)


@pytest.mark.skipif(_gpu(), reason="with a GPU present a fully valid call would launch on fake pointers")
def test_valid_call_without_gpu_reports_device(L):
    assert fwd(L) == DEVICE
    assert msg(L)


def test_bwd_workspace_query_is_pure(L):
    B, T, H, Hkv, D = 2, 100, 4, 2, 64
    stats = -(-(B * H * T * 4) // 256) * 256
    assert L.nc_attn_bwd_workspace_bytes(BF16, B, T, H, Hkv, D) == 2 * stats
    assert L.nc_attn_bwd_workspace_bytes(F32, B, T, H, Hkv, D) == 2 * stats
    assert L.nc_attn_bwd_workspace_bytes(BF16, B, T, 3, 2, D) == 0
    assert L.nc_attn_bwd_workspace_bytes(BF16, B, T, H, Hkv, 40) == 0


def bwd(L, ws=A, wsb=1 << 30, dq=A, dout=A, dt=BF16, D=64, H=2, Hkv=1, w=0, scale=0.1):
    return L.nc_attn_bwd(dt, 1, 64, H, Hkv, D, A, A, A, A, A, dout, w, scale, dq, A, A, ws, wsb, None)


def test_bwd_validation(L):
    assert bwd(L, dq=None) == INVALID
    assert bwd(L, dout=A + 4) == INVALID
    assert bwd(L, ws=None) == WORKSPACE
    need = L.nc_attn_bwd_workspace_bytes(BF16, 1, 64, 2, 1, 64)
    assert bwd(L, wsb=need - 1) == WORKSPACE
    assert "workspace" in msg(L)
    assert bwd(L, ws=A + 8) == WORKSPACE
    assert bwd(L, D=96) == UNSUPPORTED
    assert bwd(L, H=3, Hkv=2) == INVALID


def test_decode_workspace_query_is_pure(L):
    # one partial of D + 2 floats per (row, query head, chunk); a chunk is
    # (64 / (D/8)) lane groups x 16, 8 or 4 positions for G <= 2, <= 4, <= 8
    assert L.nc_attn_decode_workspace_bytes(BF16, 64, 10, 10, 128, 2048) == 64 * 10 * 32 * 130 * 4
    assert L.nc_attn_decode_workspace_bytes(BF16, 3, 4, 2, 32, 257) == 3 * 4 * 2 * 34 * 4
    assert L.nc_attn_decode_workspace_bytes(BF16, 3, 8, 2, 64, 100) == 3 * 8 * 2 * 66 * 4
    assert L.nc_attn_decode_workspace_bytes(BF16, 3, 4, 3, 32, 257) == 0


def dec(L, H=4, Hkv=2, D=64, T_max=100, seqlens=A, ws=A, wsb=1 << 30, lse=A, out=A, scale=0.1):
    return L.nc_attn_decode(BF16, 2, H, Hkv, D, T_max, A, A, A, seqlens, 0, scale, out, lse, ws, wsb, None)


def test_decode_validation(L):
    assert dec(L, H=5, Hkv=1) == UNSUPPORTED  # group of 5 not built
    assert "group" in msg(L)
    assert dec(L, seqlens=None) == INVALID
    assert dec(L, seqlens=A + 2) == INVALID
    assert dec(L, lse=None) == INVALID
    assert dec(L, out=A + 4) == INVALID
    assert dec(L, ws=None) == WORKSPACE
    assert dec(L, wsb=10) == WORKSPACE
    assert dec(L, T_max=0) == INVALID
    assert dec(L, scale=-1.0) == INVALID


def test_rope_table_validation(L):
    assert L.nc_rope_table(0, 64, 1e5, A, A, None) == INVALID
    assert L.nc_rope_table(16, 63, 1e5, A, A, None) == INVALID
    assert L.nc_rope_table(16, 64, 1.0, A, A, None) == INVALID
    assert L.nc_rope_table(16, 64, 1e5, None, A, None) == INVALID
    assert L.nc_rope_table(16, 64, 1e5, A + 2, A, None) == INVALID


def test_prologue_validation(L):
    f = L.nc_qk_prologue_fwd
    assert f(BF16, 1, 64, 2, 1, 64, A, A, None, A, A, 32, 1e-6, A, A, None) == INVALID  # T > T_rope
    assert "table" in msg(L)
    assert f(BF16, 1, 16, 2, 1, 64, A, A, None, A, A, 32, -1.0, A, A, None) == INVALID  # eps
    assert f(BF16, 1, 16, 2, 1, 64, A, A, A + 2, A, A, 32, 1e-6, A, A, None) == INVALID  # pos_offset
    assert f(BF16, 1, 16, 2, 1, 64, A, A, None, A, A, 32, 1e-6, None, A, None) == INVALID
    assert f(BF16, 1, 16, 2, 1, 80, A, A, None, A, A, 32, 1e-6, A, A, None) == UNSUPPORTED
    g = L.nc_qk_prologue_bwd
    assert g(BF16, 1, 16, 2, 1, 64, A, A, None, A, A, 32, 1e-6, None, A, A, A, None) == INVALID
    assert g(BF16, 1, 16, 2, 1, 64, A, A, None, A, A, 32, 1e-6, A, A, A, None, None) == INVALID


def test_profile_hook_validation(L):
    assert L.nc_profile_bwd_main(A, None, None) == INVALID  # dq_begin, dkdv_begin, end
    assert L.nc_profile_bwd_main(A, A, None) == INVALID
    assert L.nc_profile_bwd_main(None, None, None) == OK


def test_fp8_forward_validation(L):
    f = L.nc_attn_fwd_fp8
    assert f(1, 16, 2, 1, 32, A, A, A, 1.0, 1.0, 1.0, 0, 0.1, A, A, None) == UNSUPPORTED  # D = 32
    assert "D=32" in msg(L)
    assert f(1, 16, 2, 1, 128, A, A, A, 0.0, 1.0, 1.0, 0, 0.1, A, A, None) == INVALID  # descale 0
    assert f(1, 16, 2, 1, 128, A, A, A, 1.0, float("nan"), 1.0, 0, 0.1, A, A, None) == INVALID
    assert f(1, 16, 2, 1, 128, A, A, A, 1.0, 1.0, float("inf"), 0, 0.1, A, A, None) == INVALID
    assert "descale" in msg(L)
    assert f(1, 16, 2, 1, 128, None, A, A, 1.0, 1.0, 1.0, 0, 0.1, A, A, None) == INVALID
    assert f(1, 16, 3, 2, 128, A, A, A, 1.0, 1.0, 1.0, 0, 0.1, A, A, None) == INVALID  # H % Hkv
    assert f(1, 16, 2, 1, 128, A, A, A, 1e30, 1e30, 1.0, 0, 0.1, A, A, None) == INVALID  # scale overflow


def test_grid_limits(L):
    # float32 attention: heads and rows on the second and third grid axes
    assert fwd(L, dt=F32, B=70000, T=1, H=1, Hkv=1, D=32) == UNSUPPORTED
    assert "65535" in msg(L)
    assert fwd(L, dt=F32, B=1, T=1, H=70000, Hkv=1, D=32) == UNSUPPORTED
    # decode: rows and cache chunks (64 positions per chunk at D = 128, group 1)
    d = L.nc_attn_decode
    assert d(BF16, 70000, 1, 1, 128, 1, A, A, A, A, 0, 0.1, A, A, A, 1 << 40, None) == UNSUPPORTED
    assert d(BF16, 1, 1, 1, 128, 65535 * 64 + 1, A, A, A, A, 0, 0.1, A, A, A, 1 << 40, None) == UNSUPPORTED
    assert "T_max" in msg(L)


def test_clock_probe_validation(L):
    assert L.nc_measure_shader_clock(None, 10, None) == INVALID
    assert "out" in msg(L)
    assert L.nc_measure_shader_clock(A, 0, None) == INVALID
    assert L.nc_measure_shader_clock(A, 10001, None) == INVALID
    assert "milliseconds" in msg(L)


def test_error_message_is_per_thread(L):
    import threading
    assert fwd(L, q=None) == INVALID
    seen = []

    def other():
        seen.append(msg(L))

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen == [""]
    assert "q is NULL" in msg(L)


def bwdp(L, q_raw=A, k_raw=A, pos=None, T=64, T_rope=128, eps=1e-6, ws=A, wsb=1 << 30, dk=A, D=64):
    return L.nc_attn_bwd_prologue(BF16, 1, T, 2, 1, D, A, A, A, A, A, A, 0, 0.1, q_raw, k_raw, pos, A, A,
                                  T_rope, eps, A, dk, A, ws, wsb, None)


def test_bwd_prologue_validation(L):
    assert bwdp(L, q_raw=None) == INVALID
    assert bwdp(L, k_raw=A + 4) == INVALID
    assert bwdp(L, T_rope=32) == INVALID  # T > T_rope without offsets
    assert "table" in msg(L)
    assert bwdp(L, eps=-1.0) == INVALID
    assert bwdp(L, pos=A + 2) == INVALID
    assert bwdp(L, dk=None) == INVALID
    assert bwdp(L, ws=None) == WORKSPACE
    assert bwdp(L, wsb=16) == WORKSPACE
    assert bwdp(L, D=80) == UNSUPPORTED


def test_decode_step_workspace_query_is_pure(L):
    for dt in (BF16, F32):  # the split-K partials, as for nc_attn_decode
        assert L.nc_attn_decode_step_workspace_bytes(dt, 64, 10, 10, 128, 2048) == \
            L.nc_attn_decode_workspace_bytes(dt, 64, 10, 10, 128, 2048) == 64 * 10 * 32 * 130 * 4
    assert L.nc_attn_decode_step_workspace_bytes(BF16, 3, 4, 3, 32, 257) == 0


def dstep(L, q=A, k_new=A, v_new=A, kc=A, vc=A, lens=A, cos=A, T_rope=128, eps=1e-6, lse=A, ws=A, wsb=1 << 30,
          H=4, Hkv=2, D=64, scale=0.1):
    return L.nc_attn_decode_step(BF16, 2, H, Hkv, D, 100, q, k_new, v_new, kc, vc, lens, cos, A, T_rope, eps, 0,
                                 scale, A, lse, ws, wsb, None)


def test_decode_step_validation(L):
    assert dstep(L, H=5, Hkv=1) == UNSUPPORTED
    assert dstep(L, D=96) == UNSUPPORTED
    assert dstep(L, k_new=None) == INVALID
    assert "k_new" in msg(L)
    assert dstep(L, v_new=A + 8) == INVALID
    assert dstep(L, kc=None) == INVALID
    assert dstep(L, lens=None) == INVALID
    assert dstep(L, lens=A + 2) == INVALID
    assert dstep(L, cos=None) == INVALID
    assert dstep(L, T_rope=0) == INVALID
    assert dstep(L, eps=float("nan")) == INVALID
    assert dstep(L, lse=A + 2) == INVALID
    assert dstep(L, scale=0.0) == INVALID
    assert dstep(L, ws=None) == WORKSPACE
    assert dstep(L, wsb=100) == WORKSPACE


def dstep_noalloc(L, B=2, H=4, Hkv=2, D=64, T_max=100, k_new=A, lens=A, eps=1e-6, scale=0.1):
    return L.nc_attn_decode_step_noalloc(BF16, B, H, Hkv, D, T_max, A, k_new, A, A, A, lens, A, A, 128, eps, 0,
                                         scale, A, A, None)


def test_decode_step_noalloc_validation(L):
    # the same checks as nc_attn_decode_step, and a size limit instead of a workspace
    assert dstep_noalloc(L, H=5, Hkv=1) == UNSUPPORTED
    assert dstep_noalloc(L, k_new=None) == INVALID
    assert dstep_noalloc(L, lens=A + 2) == INVALID
    assert dstep_noalloc(L, eps=float("nan")) == INVALID
    assert dstep_noalloc(L, scale=0.0) == INVALID
    need = L.nc_attn_decode_step_workspace_bytes(BF16, 64, 32, 4, 128, 4096)
    assert need > native.NC_NOALLOC_SCRATCH_BYTES
    assert dstep_noalloc(L, B=64, H=32, Hkv=4, D=128, T_max=4096) == UNSUPPORTED
    assert "scratch" in msg(L)
    # the decode workload's partials fit
    assert L.nc_attn_decode_step_workspace_bytes(BF16, 64, 10, 10, 128, 2048) <= native.NC_NOALLOC_SCRATCH_BYTES
    if not _gpu():
        assert dstep_noalloc(L, B=64, H=10, Hkv=10, D=128, T_max=2048) == DEVICE


def test_kv_cache_replicate_validation(L):
    f = L.nc_kv_cache_replicate
    assert f(BF16, 4, 100, 2, 64, 0, A, A, None) == INVALID  # n_tokens < 1
    assert f(BF16, 4, 100, 2, 64, 101, A, A, None) == INVALID  # n_tokens > T_max
    assert "n_tokens" in msg(L)
    assert f(BF16, 4, 100, 2, 64, 10, None, A, None) == INVALID
    assert f(BF16, 4, 100, 2, 64, 10, A, A + 4, None) == INVALID
    assert f(BF16, 0, 100, 2, 64, 10, A, A, None) == INVALID
    assert f(BF16, 4, 100, 2, 48, 10, A, A, None) == UNSUPPORTED


def fcache(L, q=A, kc=A, lens=A, out=A, lse=A, Tq=8, T_max=64, H=4, Hkv=2, D=64, scale=0.1):
    return L.nc_attn_fwd_cache(BF16, 2, Tq, H, Hkv, D, T_max, q, kc, A, lens, 0, scale, out, lse, None)


def test_fwd_cache_validation(L):
    assert fcache(L, T_max=7) == INVALID
    assert "T_max" in msg(L)
    assert fcache(L, H=3) == INVALID
    assert fcache(L, D=96) == UNSUPPORTED
    assert fcache(L, q=None) == INVALID
    assert fcache(L, kc=A + 2) == INVALID
    assert fcache(L, lens=None) == INVALID
    assert fcache(L, lens=A + 1) == INVALID
    assert fcache(L, out=None) == INVALID
    assert fcache(L, lse=None) == INVALID
    assert fcache(L, scale=-1.0) == INVALID


def test_kv_cache_append_validation(L):
    f = L.nc_kv_cache_append
    assert f(BF16, 2, 8, 2, 64, 7, A, A, A, A, A, None) == INVALID  # T_max < Tq
    assert f(BF16, 2, 8, 2, 64, 64, None, A, A, A, A, None) == INVALID
    assert f(BF16, 2, 8, 2, 64, 64, A, A, A, A + 8, A, None) == INVALID
    assert f(BF16, 2, 8, 2, 64, 64, A, A, A, A, None, None) == INVALID
    assert f(BF16, 2, 8, 2, 64, 64, A, A, A, A, A + 2, None) == INVALID
    assert f(BF16, 2, 0, 2, 64, 64, A, A, A, A, A, None) == INVALID
    assert f(BF16, 2, 8, 2, 40, 64, A, A, A, A, A, None) == UNSUPPORTED


def test_fwd_prologue_validation(L):
    f = L.nc_attn_fwd_prologue

    def call(q=A, k=A, v=A, pos=None, T=64, T_rope=128, eps=1e-6, qo=A, ko=A, out=A, lse=A, D=64, scale=0.1):
        return f(BF16, 1, T, 2, 1, D, q, k, v, pos, A, A, T_rope, eps, 0, scale, qo, ko, out, lse, None)

    assert call(q=None) == INVALID
    assert call(v=None) == INVALID
    assert call(T_rope=32) == INVALID
    assert "table" in msg(L)
    assert call(pos=A + 2) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call(qo=None) == INVALID
    assert call(ko=A + 4) == INVALID
    assert call(out=None) == INVALID
    assert call(lse=None) == INVALID
    assert call(scale=float("inf")) == INVALID
    assert call(D=80) == UNSUPPORTED
    assert L.nc_profile_fwd_prologue(A, None, A) == INVALID
    assert L.nc_profile_fwd_prologue(None, None, None) == OK
