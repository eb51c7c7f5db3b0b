"""fp64 definition of the engine-side cache steps around single-token decode.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

  * Decode step with the cache updated in place. "nanochat Admin & Developer
    Guide", section 7 "KV cache": the cache is built for FA3's kvcache call,
    the position of each batch row is its int32 cache_seqlens entry, and the
    cache is written in place; section 3: the new token's q and k go through
    the QK prologue (weightless RMSNorm, then half-split RoPE) at that
    position before attention. Reading of the pages: row b holds
    n = cache_seqlens[b] tokens before the step; the new token is at
    position n, its k' and v land in cache slot n, and the query attends to
    slots max(0, n + 1 - w) .. n (the decode of oracle.attention with
    L_b = n + 1). The lengths array itself is the caller's to advance.
    The cache is storage of the model's dtype, so what the attention reads
    back from slot n is k' as stored in that dtype: with cache_dtype "bf16"
    (or "f32") the appended k' and v are rounded to it before the attention,
    like every other cache entry; cache_dtype None keeps them exact. q' is
    an activation of the model's dtype too (the prologue's outputs enter the
    attention as tensors of that dtype, section 3), so it is rounded to
    cache_dtype as well: the step then attends exactly as the last row of a
    prefill whose prologue outputs are stored in that dtype.
  * Cache replication. Section 7 "KV cache" and "Generation flow": the
    prompt is prefilled once with batch 1 and that cache is copied to every
    sample row. Only the prompt's positions are copied.
  * Chunked prefill against a cache. Section 6: the SDPA fallback's third
    case, chunked / sliding-window inference, where the queries of a chunk
    are fewer than the keys and the visible keys form a shifted causal
    (optionally windowed) band built as an explicit mask. Reading: row b has
    n_b = cache_seqlens[b] tokens cached; the chunk's Tq tokens sit at
    positions n_b .. n_b + Tq - 1, their k and v already written to those
    cache slots (cache_append); chunk query t attends to cache slots j with
    p - w < j <= p, p = n_b + t (all j <= p for a full layer).
"""

import numpy as np

from .attention import decode
from .prologue import ROPE_BASE, qk_prologue_fwd


def round_to(x, dtype):
    """x rounded to the storage dtype: "f32" rounds to nearest even float32,
    "bf16" to float32 and then to nearest even bfloat16 (8 significand bits);
    None leaves x as it is. Returns float64."""
    x = np.asarray(x, dtype=np.float64)
    if dtype is None:
        return x.copy()
    f = x.astype(np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    if dtype != "bf16":
        raise ValueError("dtype must be None, 'f32' or 'bf16'")
    bits = f.view(np.uint32).astype(np.uint64)
    bits = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def decode_step(q, k_new, v_new, k_cache, v_cache, cache_seqlens, window, scale, eps, base=ROPE_BASE,
                cache_dtype=None):
    """One decode step of one layer.

    q [B, H, D], k_new, v_new [B, Hkv, D] (raw, before the prologue);
    k_cache, v_cache [B, T_max, Hkv, D]; cache_seqlens [B] ints in
    0 .. T_max - 1. Returns (out [B, H, D], lse [B, H], k_cache', v_cache')
    where the returned caches are float64 copies with slot n of each row
    replaced by the new token's k' and v; the inputs are not modified.
    """
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    B, H, D = q.shape
    T_max = kc.shape[1]
    n = np.asarray(cache_seqlens, dtype=np.int64)
    if n.shape != (B,) or n.min() < 0 or n.max() >= T_max:
        raise ValueError("cache_seqlens must be [B] with values in 0..T_max-1")
    pos = n[:, None]  # [B, 1]: the new token's position
    qp, kp = qk_prologue_fwd(q[:, None], k_new[:, None], pos, eps, base)
    qp = round_to(qp, cache_dtype)
    for b in range(B):
        kc[b, n[b]] = round_to(kp[b, 0], cache_dtype)
        vc[b, n[b]] = round_to(v_new[b], cache_dtype)
    out, lse = decode(qp[:, 0], kc, vc, n + 1, window, scale)
    return out, lse, kc, vc


def kv_cache_replicate(src_row, n_rows, T_max, n_tokens):
    """[n_rows, T_max, Hkv, D] float64 cache whose rows hold positions
    0 .. n_tokens - 1 of src_row ([>= n_tokens, Hkv, D]); later positions are
    NaN (their content is not defined by the step)."""
    src = np.asarray(src_row, dtype=np.float64)
    out = np.full((n_rows, T_max) + src.shape[1:], np.nan)
    out[:, :n_tokens] = src[None, :n_tokens]
    return out


def cache_append(k_chunk, v_chunk, k_cache, v_cache, cache_seqlens, cache_dtype=None):
    """Copies of the caches with the chunk's k, v [B, Tq, Hkv, D] written at
    slots n_b .. n_b + Tq - 1 of each row (rounded to the cache dtype)."""
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    k_chunk = np.asarray(k_chunk, dtype=np.float64)
    v_chunk = np.asarray(v_chunk, dtype=np.float64)
    B, Tq = k_chunk.shape[:2]
    n = np.asarray(cache_seqlens, dtype=np.int64)
    if n.shape != (B,) or n.min() < 0 or (n + Tq).max() > kc.shape[1]:
        raise ValueError("every row needs 0 <= n_b and n_b + Tq <= T_max")
    for b in range(B):
        kc[b, n[b]:n[b] + Tq] = round_to(k_chunk[b], cache_dtype)
        vc[b, n[b]:n[b] + Tq] = round_to(v_chunk[b], cache_dtype)
    return kc, vc


def prefill_chunk(q, k_cache, v_cache, cache_seqlens, window, scale):
    """Attention of a chunk of queries against a cache that already holds the
    chunk's own keys.

    q [B, Tq, H, D]; k_cache, v_cache [B, T_max, Hkv, D]; cache_seqlens [B]
    with 0 <= n_b and n_b + Tq <= T_max. Query t of row b sits at position
    p = n_b + t and sees slots j with p - w < j <= p (w <= 0: all j <= p).
    Returns out [B, Tq, H, D] and lse [B, H, Tq]. Dense masked scores.
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, Tq, H, D = q.shape
    T_max, Hkv = kc.shape[1], kc.shape[2]
    n = np.asarray(cache_seqlens, dtype=np.int64)
    if n.shape != (B,) or n.min() < 0 or (n + Tq).max() > T_max:
        raise ValueError("every row needs 0 <= n_b and n_b + Tq <= T_max")
    G = H // Hkv
    out = np.zeros((B, Tq, H, D))
    lse = np.zeros((B, H, Tq))
    for b in range(B):
        Lk = int(n[b]) + Tq  # slots 0 .. Lk - 1 hold keys
        p = n[b] + np.arange(Tq)[:, None]
        j = np.arange(Lk)[None, :]
        vis = j <= p
        if window > 0:
            vis &= j > p - window
        for h in range(H):
            g = h // G
            s = scale * (q[b, :, h, :] @ kc[b, :Lk, g, :].T)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            out[b, :, h, :] = (e / z) @ vc[b, :Lk, g, :]
            lse[b, h, :] = (m + np.log(z))[:, 0]
    return out, lse
