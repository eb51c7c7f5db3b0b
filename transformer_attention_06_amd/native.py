"""ctypes binding of libncattn.so (argument marshalling only).

The functions below carry the names of the C entry points declared in
include/ncattn.h. They take torch tensors for device memory and the current
torch stream, pass raw pointers and sizes to the library, and raise
``NcError`` on a non-zero status. Every step of the computation runs in the
library's HIP kernels; there is no fallback: if the library is missing or
cannot be loaded, the first call raises.
"""

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("NCATTN_LIB") or os.path.join(HERE, "libncattn.so")

NC_F32, NC_BF16 = 0, 1
STATUS = {0: "NC_OK", 1: "NC_ERR_INVALID_ARG", 2: "NC_ERR_UNSUPPORTED", 3: "NC_ERR_WORKSPACE",
          4: "NC_ERR_DEVICE", 5: "NC_ERR_LAUNCH"}

# every symbol include/ncattn.h declares
EXPORTS = (
    "nc_abi_version", "nc_status_string", "nc_last_error_message",
    "nc_attn_fwd", "nc_attn_fwd_cache", "nc_kv_cache_append", "nc_attn_bwd_workspace_bytes", "nc_attn_bwd", "nc_attn_bwd_prologue",
    "nc_profile_bwd_main",
    "nc_attn_decode_workspace_bytes", "nc_attn_decode",
    "nc_attn_decode_step_workspace_bytes", "nc_attn_decode_step", "nc_attn_decode_step_noalloc",
    "nc_kv_cache_replicate",
    "nc_rope_table", "nc_qk_prologue_fwd", "nc_qk_prologue_bwd", "nc_attn_fwd_prologue",
    "nc_profile_fwd_prologue", "nc_measure_shader_clock", "nc_attn_fwd_fp8",
)


class NcError(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name}: {STATUS.get(status, status)}: {msg}")
        self.status = status


_lock = threading.Lock()
_lib = None

_i, _p, _f, _d, _sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_double, ctypes.c_size_t

_SIGS = {
    "nc_abi_version": ([], _i),
    "nc_status_string": ([_i], ctypes.c_char_p),
    "nc_last_error_message": ([], ctypes.c_char_p),
    "nc_attn_fwd": ([_i] * 6 + [_p, _p, _p, _i, _f, _p, _p, _p], _i),
    "nc_attn_fwd_cache": ([_i] * 7 + [_p] * 4 + [_i, _f, _p, _p, _p], _i),
    "nc_kv_cache_append": ([_i] * 6 + [_p] * 5 + [_p], _i),
    "nc_attn_bwd_workspace_bytes": ([_i] * 6, _sz),
    "nc_attn_bwd": ([_i] * 6 + [_p] * 6 + [_i, _f] + [_p] * 3 + [_p, _sz, _p], _i),
    "nc_attn_bwd_prologue": ([_i] * 6 + [_p] * 6 + [_i, _f] + [_p] * 5 + [_i, _f] + [_p] * 3
                             + [_p, _sz, _p], _i),
    "nc_profile_bwd_main": ([_p, _p, _p], _i),
    "nc_profile_fwd_prologue": ([_p, _p, _p], _i),
    "nc_attn_decode_workspace_bytes": ([_i] * 6, _sz),
    "nc_attn_decode": ([_i] * 6 + [_p] * 4 + [_i, _f, _p, _p, _p, _sz, _p], _i),
    "nc_attn_decode_step_workspace_bytes": ([_i] * 6, _sz),
    "nc_attn_decode_step": ([_i] * 6 + [_p] * 8 + [_i, _f, _i, _f, _p, _p, _p, _sz, _p], _i),
    "nc_attn_decode_step_noalloc": ([_i] * 6 + [_p] * 8 + [_i, _f, _i, _f, _p, _p, _p], _i),
    "nc_kv_cache_replicate": ([_i] * 6 + [_p, _p, _p], _i),
    "nc_rope_table": ([_i, _i, _d, _p, _p, _p], _i),
    "nc_qk_prologue_fwd": ([_i] * 6 + [_p] * 5 + [_i, _f, _p, _p, _p], _i),
    "nc_attn_fwd_prologue": ([_i] * 6 + [_p] * 6 + [_i, _f, _i, _f] + [_p] * 4 + [_p], _i),
    "nc_qk_prologue_bwd": ([_i] * 6 + [_p] * 5 + [_i, _f, _p, _p, _p, _p, _p], _i),
    "nc_measure_shader_clock": ([_p, _i, _p], _i),
    "nc_attn_fwd_fp8": ([_i] * 5 + [_p] * 3 + [_f] * 3 + [_i, _f, _p, _p, _p], _i),
}


def lib():
    """Load libncattn.so once and declare its signatures."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise OSError(f"{LIB_PATH} not found: build it with "
                              "`python -m transformer_attention_06_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in _SIGS.items():
                fn = getattr(L, name)
                fn.argtypes = args
                fn.restype = res
            _lib = L
        return _lib


def _raise_on(name, status):
    if status != 0:
        raise NcError(name, status, lib().nc_last_error_message().decode())


def _dt(t):
    import torch
    if t.dtype == torch.bfloat16:
        return NC_BF16
    if t.dtype == torch.float32:
        return NC_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libncattn must be contiguous")
    return t.data_ptr()


def _arg(t, name, shape, dtypes, device, optional=False):
    """Pointer of tensor t after checking what the C ABI cannot see: t is on
    `device` (a GPU), has exactly `shape` (None: any) and one of `dtypes`
    (None: any), and is contiguous. The library trusts these, so a tensor
    that fails here would otherwise be read or written out of bounds."""
    import torch
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return _ptr(t)


def _gpu(t, name):
    """The device of the leading tensor argument, which must be a GPU."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    return t.device


def _dims(t, name, n):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _empty(shape, like, dtype=None):
    import torch
    return torch.empty(shape, dtype=dtype or like.dtype, device=like.device)


def _rope_args(cos, sin, D, dev):
    """cos/sin float32 [T_rope, D/2] on dev -> (cos ptr, sin ptr, T_rope)."""
    import torch
    if not isinstance(cos, torch.Tensor) or cos.dim() != 2:
        raise ValueError("cos must be a float32 tensor [T_rope, D/2]")
    T_rope = cos.shape[0]
    f32 = (torch.float32,)
    return (_arg(cos, "cos", (T_rope, D // 2), f32, dev), _arg(sin, "sin", (T_rope, D // 2), f32, dev), T_rope)


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)


def nc_abi_version():
    return lib().nc_abi_version()


def nc_attn_fwd(q, k, v, window, scale, out=None, lse=None, stream=None):
    """q [B,T,H,D], k/v [B,T,Hkv,D] -> (out [B,T,H,D], lse [B,H,T] float32)."""
    import torch
    dev = _gpu(q, "q")
    B, T, H, D = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[2]
    dt = (q.dtype,)
    out = _empty(q.shape, q) if out is None else out
    lse = _empty((B, H, T), q, torch.float32) if lse is None else lse
    st = lib().nc_attn_fwd(_dt(q), B, T, H, Hkv, D, _arg(q, "q", None, None, dev),
                           _arg(k, "k", (B, T, Hkv, D), dt, dev), _arg(v, "v", (B, T, Hkv, D), dt, dev),
                           int(window), float(scale), _arg(out, "out", (B, T, H, D), dt, dev),
                           _arg(lse, "lse", (B, H, T), (torch.float32,), dev), _stream(stream))
    _raise_on("nc_attn_fwd", st)
    return out, lse


def nc_attn_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, window, scale, out=None, lse=None,
                    stream=None):
    """float8 e4m3 q8 [B,T,H,D], k8/v8 [B,T,Hkv,D] (torch.float8_e4m3fn or uint8 codes) with one
    descale per tensor -> (out [B,T,H,D] bf16, lse [B,H,T] float32)."""
    import torch
    dev = _gpu(q8, "q8")
    B, T, H, D = _dims(q8, "q8", 4)
    Hkv = _dims(k8, "k8", 4)[2]
    codes = (torch.float8_e4m3fn, torch.uint8)
    out = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev) if lse is None else lse
    st = lib().nc_attn_fwd_fp8(B, T, H, Hkv, D, _arg(q8, "q8", None, codes, dev),
                               _arg(k8, "k8", (B, T, Hkv, D), codes, dev), _arg(v8, "v8", (B, T, Hkv, D), codes, dev),
                               float(q_descale), float(k_descale), float(v_descale), int(window), float(scale),
                               _arg(out, "out", (B, T, H, D), (torch.bfloat16,), dev),
                               _arg(lse, "lse", (B, H, T), (torch.float32,), dev), _stream(stream))
    _raise_on("nc_attn_fwd_fp8", st)
    return out, lse


def nc_attn_bwd_workspace_bytes(dtype_code, B, T, H, Hkv, D):
    return lib().nc_attn_bwd_workspace_bytes(dtype_code, B, T, H, Hkv, D)


def _bwd_args(q, k, v, out, lse, dout, dq, dk, dv, workspace, dev):
    """Checked pointers of the attention backward's tensors (allocating the
    outputs and the workspace when not given)."""
    import torch
    B, T, H, D = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[2]
    dt = (q.dtype,)
    dq = _empty(q.shape, q) if dq is None else dq
    dk = _empty(k.shape, k) if dk is None else dk
    dv = _empty(k.shape, k) if dv is None else dv
    if workspace is None:
        need = nc_attn_bwd_workspace_bytes(_dt(q), B, T, H, Hkv, D)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    qs, ks = (B, T, H, D), (B, T, Hkv, D)
    ptrs = [_arg(q, "q", None, None, dev), _arg(k, "k", ks, dt, dev), _arg(v, "v", ks, dt, dev),
            _arg(out, "out", qs, dt, dev), _arg(lse, "lse", (B, H, T), (torch.float32,), dev),
            _arg(dout, "dout", qs, dt, dev), _arg(dq, "dq", qs, dt, dev), _arg(dk, "dk", ks, dt, dev),
            _arg(dv, "dv", ks, dt, dev), _arg(workspace, "workspace", None, None, dev)]
    return (B, T, H, Hkv, D), ptrs, (dq, dk, dv), _nbytes(workspace)


def nc_attn_bwd(q, k, v, out, lse, dout, window, scale, dq=None, dk=None, dv=None,
                workspace=None, stream=None):
    """Gradients (dq, dk, dv) of sum(out * dout); dk/dv summed over each query group."""
    dev = _gpu(q, "q")
    (B, T, H, Hkv, D), P, grads, wsb = _bwd_args(q, k, v, out, lse, dout, dq, dk, dv, workspace, dev)
    st = lib().nc_attn_bwd(_dt(q), B, T, H, Hkv, D, P[0], P[1], P[2], P[3], P[4], P[5], int(window), float(scale),
                           P[6], P[7], P[8], P[9], wsb, _stream(stream))
    _raise_on("nc_attn_bwd", st)
    return grads


def nc_attn_bwd_prologue(q, k, v, out, lse, dout, window, scale, q_raw, k_raw, cos, sin, eps,
                         pos_offset=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward through attention and the QK prologue: (dq, dk) w.r.t. the raw
    q_raw, k_raw and dv, where q, k are the prologue outputs used in the forward."""
    import torch
    dev = _gpu(q, "q")
    (B, T, H, Hkv, D), P, grads, wsb = _bwd_args(q, k, v, out, lse, dout, dq, dk, dv, workspace, dev)
    dt = (q.dtype,)
    c, s_, T_rope = _rope_args(cos, sin, D, dev)
    st = lib().nc_attn_bwd_prologue(_dt(q), B, T, H, Hkv, D, P[0], P[1], P[2], P[3], P[4], P[5], int(window),
                                    float(scale), _arg(q_raw, "q_raw", (B, T, H, D), dt, dev),
                                    _arg(k_raw, "k_raw", (B, T, Hkv, D), dt, dev),
                                    _arg(pos_offset, "pos_offset", (B,), (torch.int32,), dev, optional=True),
                                    c, s_, T_rope, float(eps), P[6], P[7], P[8], P[9], wsb, _stream(stream))
    _raise_on("nc_attn_bwd_prologue", st)
    return grads


def nc_profile_bwd_main(dq_begin=None, dkdv_begin=None, end=None):
    """Record three torch.cuda.Event objects (already recorded once, so that
    they exist) before the dQ kernel, between it and the dK/dV kernel, and
    after the dK/dV kernel of later nc_attn_bwd calls on this thread; call
    with no arguments to stop."""
    evs = [e.cuda_event if e is not None else None for e in (dq_begin, dkdv_begin, end)]
    _raise_on("nc_profile_bwd_main", lib().nc_profile_bwd_main(*evs))


def nc_attn_fwd_cache(q, k_cache, v_cache, cache_seqlens, window, scale, out=None, lse=None, stream=None):
    """A chunk q [B,Tq,H,D] against caches [B,T_max,Hkv,D] already holding the chunk's keys at
    slots cache_seqlens[b] .. + Tq - 1 -> (out [B,Tq,H,D], lse [B,H,Tq] float32)."""
    import torch
    dev = _gpu(q, "q")
    B, Tq, H, D = _dims(q, "q", 4)
    T_max, Hkv = _dims(k_cache, "k_cache", 4)[1:3]
    dt, cs = (q.dtype,), (B, T_max, Hkv, D)
    out = _empty(q.shape, q) if out is None else out
    lse = _empty((B, H, Tq), q, torch.float32) if lse is None else lse
    st = lib().nc_attn_fwd_cache(_dt(q), B, Tq, H, Hkv, D, T_max, _arg(q, "q", None, None, dev),
                                 _arg(k_cache, "k_cache", cs, dt, dev), _arg(v_cache, "v_cache", cs, dt, dev),
                                 _arg(cache_seqlens, "cache_seqlens", (B,), (torch.int32,), dev), int(window),
                                 float(scale), _arg(out, "out", (B, Tq, H, D), dt, dev),
                                 _arg(lse, "lse", (B, H, Tq), (torch.float32,), dev), _stream(stream))
    _raise_on("nc_attn_fwd_cache", st)
    return out, lse


def nc_kv_cache_append(k_new, v_new, k_cache, v_cache, cache_seqlens, stream=None):
    """Writes k_new/v_new [B,Tq,Hkv,D] into cache slots cache_seqlens[b] .. + Tq - 1 (in place)."""
    import torch
    dev = _gpu(k_new, "k_new")
    B, Tq, Hkv, D = _dims(k_new, "k_new", 4)
    T_max = _dims(k_cache, "k_cache", 4)[1]
    dt, cs = (k_new.dtype,), (B, T_max, Hkv, D)
    st = lib().nc_kv_cache_append(_dt(k_new), B, Tq, Hkv, D, T_max, _arg(k_new, "k_new", None, None, dev),
                                  _arg(v_new, "v_new", (B, Tq, Hkv, D), dt, dev), _arg(k_cache, "k_cache", cs, dt, dev),
                                  _arg(v_cache, "v_cache", cs, dt, dev),
                                  _arg(cache_seqlens, "cache_seqlens", (B,), (torch.int32,), dev), _stream(stream))
    _raise_on("nc_kv_cache_append", st)
    return k_cache, v_cache


def nc_profile_fwd_prologue(prologue_begin=None, fwd_begin=None, end=None):
    """Record torch.cuda.Events around the two kernels of later nc_attn_fwd_prologue calls on this
    thread; call with no arguments to stop."""
    evs = [e.cuda_event if e is not None else None for e in (prologue_begin, fwd_begin, end)]
    _raise_on("nc_profile_fwd_prologue", lib().nc_profile_fwd_prologue(*evs))


def nc_attn_decode_workspace_bytes(dtype_code, B, H, Hkv, D, T_max):
    return lib().nc_attn_decode_workspace_bytes(dtype_code, B, H, Hkv, D, T_max)


def nc_attn_decode(q, k_cache, v_cache, seqlens, window, scale, out=None, lse=None,
                   workspace=None, stream=None):
    """q [B,H,D], caches [B,T_max,Hkv,D], seqlens int32 [B] (device) -> (out [B,H,D], lse [B,H])."""
    import torch
    dev = _gpu(q, "q")
    B, H, D = _dims(q, "q", 3)
    T_max, Hkv = _dims(k_cache, "k_cache", 4)[1:3]
    dt, cs = (q.dtype,), (B, T_max, Hkv, D)
    out = _empty(q.shape, q) if out is None else out
    lse = _empty((B, H), q, torch.float32) if lse is None else lse
    if workspace is None:
        need = nc_attn_decode_workspace_bytes(_dt(q), B, H, Hkv, D, T_max)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = lib().nc_attn_decode(_dt(q), B, H, Hkv, D, T_max, _arg(q, "q", None, None, dev),
                              _arg(k_cache, "k_cache", cs, dt, dev), _arg(v_cache, "v_cache", cs, dt, dev),
                              _arg(seqlens, "seqlens", (B,), (torch.int32,), dev), int(window), float(scale),
                              _arg(out, "out", (B, H, D), dt, dev), _arg(lse, "lse", (B, H), (torch.float32,), dev),
                              _arg(workspace, "workspace", None, None, dev), _nbytes(workspace), _stream(stream))
    _raise_on("nc_attn_decode", st)
    return out, lse


def nc_attn_decode_step_workspace_bytes(dtype_code, B, H, Hkv, D, T_max):
    return lib().nc_attn_decode_step_workspace_bytes(dtype_code, B, H, Hkv, D, T_max)


def nc_attn_decode_step(q, k_new, v_new, k_cache, v_cache, cache_seqlens, cos, sin, eps, window, scale,
                        out=None, lse=None, workspace=None, stream=None):
    """Prologue of the new token at position cache_seqlens[b], k'/v_new written into the caches
    there (in place), then decode over n + 1 keys. q [B,H,D], k_new/v_new [B,Hkv,D] raw,
    caches [B,T_max,Hkv,D], cache_seqlens int32 [B] (device) -> (out [B,H,D], lse [B,H])."""
    import torch
    dev = _gpu(q, "q")
    B, H, D = _dims(q, "q", 3)
    T_max, Hkv = _dims(k_cache, "k_cache", 4)[1:3]
    dt, cs = (q.dtype,), (B, T_max, Hkv, D)
    c, s_, T_rope = _rope_args(cos, sin, D, dev)
    out = _empty(q.shape, q) if out is None else out
    lse = _empty((B, H), q, torch.float32) if lse is None else lse
    if workspace is None:
        need = nc_attn_decode_step_workspace_bytes(_dt(q), B, H, Hkv, D, T_max)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = lib().nc_attn_decode_step(_dt(q), B, H, Hkv, D, T_max, _arg(q, "q", None, None, dev),
                                   _arg(k_new, "k_new", (B, Hkv, D), dt, dev), _arg(v_new, "v_new", (B, Hkv, D), dt, dev),
                                   _arg(k_cache, "k_cache", cs, dt, dev), _arg(v_cache, "v_cache", cs, dt, dev),
                                   _arg(cache_seqlens, "cache_seqlens", (B,), (torch.int32,), dev), c, s_, T_rope,
                                   float(eps), int(window), float(scale), _arg(out, "out", (B, H, D), dt, dev),
                                   _arg(lse, "lse", (B, H), (torch.float32,), dev),
                                   _arg(workspace, "workspace", None, None, dev), _nbytes(workspace), _stream(stream))
    _raise_on("nc_attn_decode_step", st)
    return out, lse


NC_NOALLOC_SCRATCH_BYTES = 32 << 20


def nc_attn_decode_step_noalloc(q, k_new, v_new, k_cache, v_cache, cache_seqlens, cos, sin, eps, window, scale,
                                out, lse, stream=None):
    """nc_attn_decode_step without a workspace (the library's per-GPU scratch holds the split-K
    partials): out [B,H,D] and lse [B,H] must be given, nothing is allocated here either."""
    import torch
    dev = _gpu(q, "q")
    B, H, D = _dims(q, "q", 3)
    T_max, Hkv = _dims(k_cache, "k_cache", 4)[1:3]
    dt, cs = (q.dtype,), (B, T_max, Hkv, D)
    c, s_, T_rope = _rope_args(cos, sin, D, dev)
    st = lib().nc_attn_decode_step_noalloc(_dt(q), B, H, Hkv, D, T_max, _arg(q, "q", None, None, dev),
                                           _arg(k_new, "k_new", (B, Hkv, D), dt, dev),
                                           _arg(v_new, "v_new", (B, Hkv, D), dt, dev),
                                           _arg(k_cache, "k_cache", cs, dt, dev), _arg(v_cache, "v_cache", cs, dt, dev),
                                           _arg(cache_seqlens, "cache_seqlens", (B,), (torch.int32,), dev), c, s_,
                                           T_rope, float(eps), int(window), float(scale),
                                           _arg(out, "out", (B, H, D), dt, dev),
                                           _arg(lse, "lse", (B, H), (torch.float32,), dev), _stream(stream))
    _raise_on("nc_attn_decode_step_noalloc", st)
    return out, lse


def nc_kv_cache_replicate(src, dst, n_tokens, stream=None):
    """Copies positions 0..n_tokens-1 of src (one cache row [>= n_tokens, Hkv, D], e.g. row 0 of a
    batch-1 prefill cache) into every row of dst [n_rows, T_max, Hkv, D]."""
    dev = _gpu(dst, "dst")
    n_rows, T_max, Hkv, D = _dims(dst, "dst", 4)
    if src.dtype != dst.dtype or src.shape[-2:] != dst.shape[-2:] or src.numel() < n_tokens * Hkv * D:
        raise ValueError("src must be one cache row of dst's dtype and [.., Hkv, D] shape")
    st = lib().nc_kv_cache_replicate(_dt(dst), n_rows, T_max, Hkv, D, int(n_tokens),
                                     _arg(src, "src", None, None, dev), _arg(dst, "dst", None, None, dev),
                                     _stream(stream))
    _raise_on("nc_kv_cache_replicate", st)
    return dst


def nc_measure_shader_clock(milliseconds, out=None, stream=None):
    """Enqueue the clock probe on `stream` (a torch.cuda.Stream, default current); returns the int64
    device tensor [2] it fills: shader cycles and 100 MHz ticks over `milliseconds` of wall time."""
    import torch
    if out is None:
        out = torch.zeros(2, dtype=torch.int64, device="cuda")
    dev = _gpu(out, "out")
    _raise_on("nc_measure_shader_clock",
              lib().nc_measure_shader_clock(_arg(out, "out", (2,), (torch.int64,), dev), int(milliseconds),
                                            _stream(stream)))
    return out


def nc_rope_table(T_rope, D, base=100000.0, device="cuda", stream=None):
    """cos, sin float32 [T_rope, D/2] built on the device in float64."""
    import torch
    c = torch.empty((T_rope, D // 2), dtype=torch.float32, device=device)
    s = torch.empty((T_rope, D // 2), dtype=torch.float32, device=device)
    dev = _gpu(c, "cos")
    st = lib().nc_rope_table(int(T_rope), int(D), float(base), _arg(c, "cos", None, None, dev),
                             _arg(s, "sin", None, None, dev), _stream(stream))
    _raise_on("nc_rope_table", st)
    return c, s


def _prologue_io(q, k, cos, sin, pos_offset, dev):
    import torch
    B, T, H, D = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[2]
    c, s_, T_rope = _rope_args(cos, sin, D, dev)
    ptrs = (_arg(q, "q", None, None, dev), _arg(k, "k", (B, T, Hkv, D), (q.dtype,), dev),
            _arg(pos_offset, "pos_offset", (B,), (torch.int32,), dev, optional=True), c, s_, T_rope)
    return (B, T, H, Hkv, D), ptrs


def nc_qk_prologue_fwd(q, k, cos, sin, eps, pos_offset=None, q_out=None, k_out=None, stream=None):
    """(RoPE(RMSNorm(q)), RoPE(RMSNorm(k))) at positions pos_offset[b] + t."""
    dev = _gpu(q, "q")
    (B, T, H, Hkv, D), P = _prologue_io(q, k, cos, sin, pos_offset, dev)
    dt = (q.dtype,)
    q_out = _empty(q.shape, q) if q_out is None else q_out
    k_out = _empty(k.shape, k) if k_out is None else k_out
    st = lib().nc_qk_prologue_fwd(_dt(q), B, T, H, Hkv, D, P[0], P[1], P[2], P[3], P[4], P[5], float(eps),
                                  _arg(q_out, "q_out", (B, T, H, D), dt, dev),
                                  _arg(k_out, "k_out", (B, T, Hkv, D), dt, dev), _stream(stream))
    _raise_on("nc_qk_prologue_fwd", st)
    return q_out, k_out


def nc_attn_fwd_prologue(q, k, v, cos, sin, eps, window, scale, pos_offset=None, q_out=None, k_out=None,
                         out=None, lse=None, stream=None):
    """Prologue + attention forward from raw q [B,T,H,D], k [B,T,Hkv,D] ->
    (q', k', out [B,T,H,D], lse [B,H,T] float32)."""
    import torch
    dev = _gpu(q, "q")
    (B, T, H, Hkv, D), P = _prologue_io(q, k, cos, sin, pos_offset, dev)
    dt = (q.dtype,)
    q_out = _empty(q.shape, q) if q_out is None else q_out
    k_out = _empty(k.shape, k) if k_out is None else k_out
    out = _empty(q.shape, q) if out is None else out
    lse = _empty((B, H, T), q, torch.float32) if lse is None else lse
    st = lib().nc_attn_fwd_prologue(_dt(q), B, T, H, Hkv, D, P[0], P[1], _arg(v, "v", (B, T, Hkv, D), dt, dev),
                                    P[2], P[3], P[4], P[5], float(eps), int(window), float(scale),
                                    _arg(q_out, "q_out", (B, T, H, D), dt, dev),
                                    _arg(k_out, "k_out", (B, T, Hkv, D), dt, dev),
                                    _arg(out, "out", (B, T, H, D), dt, dev),
                                    _arg(lse, "lse", (B, H, T), (torch.float32,), dev), _stream(stream))
    _raise_on("nc_attn_fwd_prologue", st)
    return q_out, k_out, out, lse


def nc_qk_prologue_bwd(q, k, cos, sin, eps, dq_out, dk_out, pos_offset=None, dq=None, dk=None,
                       stream=None):
    """Gradients w.r.t. raw q, k from gradients w.r.t. the prologue outputs."""
    dev = _gpu(q, "q")
    (B, T, H, Hkv, D), P = _prologue_io(q, k, cos, sin, pos_offset, dev)
    dt = (q.dtype,)
    dq = _empty(q.shape, q) if dq is None else dq
    dk = _empty(k.shape, k) if dk is None else dk
    st = lib().nc_qk_prologue_bwd(_dt(q), B, T, H, Hkv, D, P[0], P[1], P[2], P[3], P[4], P[5], float(eps),
                                  _arg(dq_out, "dq_out", (B, T, H, D), dt, dev),
                                  _arg(dk_out, "dk_out", (B, T, Hkv, D), dt, dev),
                                  _arg(dq, "dq", (B, T, H, D), dt, dev), _arg(dk, "dk", (B, T, Hkv, D), dt, dev),
                                  _stream(stream))
    _raise_on("nc_qk_prologue_bwd", st)
    return dq, dk


# ----------------------------------------------------------------------------
# autograd wrapper: saves out and lse, recomputes P in the backward kernel

def attention(q, k, v, window, scale):
    """Causal sliding-window GQA attention as a torch autograd op: q [B,T,H,D],
    k/v [B,T,Hkv,D] (bf16 or float32, contiguous, on the GPU) -> out [B,T,H,D]."""
    return _Attention.apply(q, k, v, window, scale)


def attention_qk_prologue(q, k, v, cos, sin, eps, window, scale, pos_offset=None):
    """The training-side hot path as one autograd op: weightless RMSNorm and
    half-split RoPE of the raw q, k (at positions pos_offset[b] + t), then
    attention. The forward is nc_attn_fwd_prologue, the backward
    nc_attn_bwd_prologue (gradients w.r.t. the raw q, k and v)."""
    return _AttentionQK.apply(q, k, v, cos, sin, eps, window, scale, pos_offset)


def _make_fn():
    import torch

    class Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, window, scale):
            out, lse = nc_attn_fwd(q, k, v, window, scale)
            ctx.save_for_backward(q, k, v, out, lse)
            ctx.window, ctx.scale = window, scale
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse = ctx.saved_tensors
            dq, dk, dv = nc_attn_bwd(q, k, v, out, lse, dout.contiguous(), ctx.window, ctx.scale)
            return dq, dk, dv, None, None

    class AttentionQK(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, cos, sin, eps, window, scale, pos_offset):
            qp, kp, out, lse = nc_attn_fwd_prologue(q, k, v, cos, sin, eps, window, scale, pos_offset=pos_offset)
            ctx.save_for_backward(q, k, v, cos, sin, qp, kp, out, lse)
            ctx.pos_offset, ctx.eps, ctx.window, ctx.scale = pos_offset, eps, window, scale
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, cos, sin, qp, kp, out, lse = ctx.saved_tensors
            dq, dk, dv = nc_attn_bwd_prologue(qp, kp, v, out, lse, dout.contiguous(), ctx.window, ctx.scale, q, k,
                                              cos, sin, ctx.eps, pos_offset=ctx.pos_offset)
            return dq, dk, dv, None, None, None, None, None, None

    return Attention, AttentionQK


class _Lazy:
    _fns = None

    def __init__(self, i):
        self.i = i

    def apply(self, *a):
        if _Lazy._fns is None:
            _Lazy._fns = _make_fn()
        return _Lazy._fns[self.i].apply(*a)


_Attention = _Lazy(0)
_AttentionQK = _Lazy(1)
