"""fp64 definition of causal grouped-query attention with a sliding window.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Notation (shared with the pages): B batch rows, T tokens, H query heads,
Hkv key/value heads with G = H / Hkv query heads per group, D head dim,
w the window, "scale" the logit multiplier.

  * Grouping: query head h reads key/value head floor(h / G); consecutive
    query heads share a KV head. "nanochat Admin & Developer Guide" section
    3 (GQA with n_kv_head <= n_head) and section 6 (SDPA fallback with
    enable_gqa, i.e. KV heads repeated G times in place).
  * Window: key j is visible to query i iff i - w < j <= i, so w counts the
    keys a query sees including itself; w <= 0 or w >= T means full causal.
    Section 3 "Sliding-window attention": per-layer window sizes handed to
    the attention kernel as (left, right) tuples; a (left, 0) tuple is
    w = left + 1 here.
  * Scores s_ij = scale * <q_i, k_j>; softmax over the visible keys;
    lse_i = ln sum_j exp(s_ij) (natural log). out_i = sum_j P_ij v_j.
  * Backward of L = sum(out * dout): the plain chain rule through the
    softmax, with dK/dV summed over the G query heads of each group.
  * Decode: one query per row at position L_b - 1 where L_b = seqlens[b]
    counts the cached keys including the current token; it sees keys
    max(0, L_b - w) .. L_b - 1 of that row's cache. Section 7 "KV cache"
    (per-layer (B, T, H, D) cache, int32 per-row lengths) and section 6
    (single-token decode slices the key window).
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _is_full(window, n_keys):
    """True when the window does not cut anything off for n_keys keys."""
    return window <= 0 or window >= n_keys


def visible_mask(T, window):
    """Boolean [T, T] matrix M with M[i, j] = key j visible to query i."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    m = j <= i
    if not _is_full(window, T):
        m = m & (j > i - window)
    return m


def kv_head_of(h, H, Hkv):
    """KV head read by query head h (contiguous groups of G = H / Hkv)."""
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    return h // (H // Hkv)


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, T, heads, D]")
    B, T, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise ValueError("k, v must be [B, T, Hkv, D] matching q")
    if H % k.shape[2] != 0:
        raise ValueError("H must be a multiple of Hkv")
    return B, T, H, k.shape[2], D


def _softmax_rows(s, mask):
    """Masked row softmax of s; returns (P, lse). Every row has >= 1 key."""
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    lse = (m + np.log(z))[..., 0]
    return e / z, lse


def _probs_bh(q, k, b, h, window, scale, mask):
    g = kv_head_of(h, q.shape[2], k.shape[2])
    s = scale * (q[b, :, h, :] @ k[b, :, g, :].T)
    return _softmax_rows(s, mask)


def attn_probs(q, k, window, scale):
    """P [B, H, T, T] and lse [B, H, T] (small inputs only: dense 4-D P)."""
    q, k = _f64(q), _f64(k)
    B, T, H, Hkv, D = _check(q, k, k)
    mask = visible_mask(T, window)
    P = np.zeros((B, H, T, T))
    lse = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            P[b, h], lse[b, h] = _probs_bh(q, k, b, h, window, scale, mask)
    return P, lse


def attn_fwd(q, k, v, window, scale):
    """out [B, T, H, D] and lse [B, H, T] in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, Hkv, D = _check(q, k, v)
    mask = visible_mask(T, window)
    out = np.zeros((B, T, H, D))
    lse = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            P, lse[b, h] = _probs_bh(q, k, b, h, window, scale, mask)
            out[b, :, h, :] = P @ v[b, :, kv_head_of(h, H, Hkv), :]
    return out, lse


def attn_bwd(q, k, v, dout, window, scale):
    """Gradients (dq, dk, dv) of L = sum(out * dout) w.r.t. q, k, v.

    Per (b, h) with g its KV head:
      dP_ij = <dout_i, v_j>
      dS_ij = P_ij * (dP_ij - sum_l P_il dP_il)      (softmax Jacobian)
      dq_i  = scale * sum_j dS_ij k_j
      dk_j += scale * sum_i dS_ij q_i                 (summed over the group)
      dv_j += sum_i P_ij dout_i                       (summed over the group)
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, T, H, Hkv, D = _check(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    mask = visible_mask(T, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            P, _ = _probs_bh(q, k, b, h, window, scale, mask)
            dO = dout[b, :, h, :]
            dP = dO @ v[b, :, g, :].T
            dS = P * (dP - (P * dP).sum(axis=-1, keepdims=True))
            dq[b, :, h, :] = scale * (dS @ k[b, :, g, :])
            dk[b, :, g, :] += scale * (dS.T @ q[b, :, h, :])
            dv[b, :, g, :] += P.T @ dO
    return dq, dk, dv


def decode(q, k_cache, v_cache, seqlens, window, scale):
    """Single-token decode against a per-layer KV cache.

    q [B, H, D]; k_cache, v_cache [B, T_max, Hkv, D]; seqlens [B] ints in
    1..T_max counting the keys of each row including the current token.
    Returns out [B, H, D] and lse [B, H]. Cache entries at positions >= L_b,
    and those before the window, are never read.
    """
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, H, D = q.shape
    if kc.shape != vc.shape or kc.ndim != 4 or kc.shape[0] != B or kc.shape[3] != D:
        raise ValueError("caches must be [B, T_max, Hkv, D]")
    T_max, Hkv = kc.shape[1], kc.shape[2]
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    out = np.zeros((B, H, D))
    lse = np.zeros((B, H))
    for b in range(B):
        L = int(seqlens[b])
        if not 1 <= L <= T_max:
            raise ValueError("seqlens must lie in 1..T_max")
        lo = 0 if _is_full(window, L) else L - window
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            keys = kc[b, lo:L, g, :]
            vals = vc[b, lo:L, g, :]
            s = scale * (keys @ q[b, h, :])
            m = s.max()
            e = np.exp(s - m)
            z = e.sum()
            out[b, h, :] = (e / z) @ vals
            lse[b, h] = m + np.log(z)
    return out, lse
