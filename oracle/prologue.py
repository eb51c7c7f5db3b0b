"""fp64 definition of the weightless QK RMSNorm + half-split RoPE prologue.

TEST INFRASTRUCTURE ONLY (see the package docstring).

  * RMSNorm without a weight: y = x / sqrt(mean_d x_d^2 + eps), per head
    vector of length D. "nanochat Admin & Developer Guide" section 3 ("no
    learnable params in RMSNorm"; queries and keys RMS-normalised before
    attention); "nanochat (Fucina port)", "Architecture" (no-weight RMSNorm).
    eps is not given on the pages; it is an argument here.
  * RoPE, half-split: element d < D/2 is paired with element d + D/2 and
    the pair is rotated by theta = p * inv_freq_d, inv_freq_d = base^(-2d/D),
    base = 100000. Section 3 (rotary embeddings, base theta 100000, no
    learned positions); Fucina "Architecture" (half-split RoPE from an
    inverse-frequency table, base 100000). The pages do not print the
    rotation's sign; this uses (a, b) -> (a cos t - b sin t, a sin t + b cos t).
  * Order: normalise, then rotate. A rotation preserves the mean square and
    the norm has no weight, so the two orders agree exactly in real
    arithmetic (pinned by a commutation test).
  * The 1.2 gain that section 3 applies after the norm is a scalar on the
    logits and is carried by the attention "scale" argument, not here.
  * Backward: the transpose of each linear map in reverse order: rotate the
    incoming gradient by -theta, then apply the transposed Jacobian of the
    norm, d/dx_k (x_i / r) = delta_ik / r - x_i x_k / (D r^3).
"""

import numpy as np

ROPE_BASE = 100000.0


def inv_freq(D, base=ROPE_BASE):
    """inv_freq_d = base^(-2d/D) for d = 0 .. D/2 - 1 (float64)."""
    if D % 2:
        raise ValueError("D must be even")
    d = np.arange(D // 2, dtype=np.float64)
    return base ** (-2.0 * d / D)


def rope_angles(positions, D, base=ROPE_BASE):
    """theta[..., d] = position * inv_freq_d for an integer array of positions."""
    p = np.asarray(positions, dtype=np.float64)
    return p[..., None] * inv_freq(D, base)


def rms_norm(x, eps):
    """x / sqrt(mean(x^2) + eps) over the last axis, no weight."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return x / r


def rope_rotate(x, positions, base=ROPE_BASE, inverse=False):
    """Rotate each half-split pair of x [B, T, heads, D] by theta (or -theta).

    positions is an integer array [B, T] giving the position of each token.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    th = rope_angles(positions, D, base)[:, :, None, :]  # [B, T, 1, D/2]
    c, s = np.cos(th), np.sin(th)
    if inverse:
        s = -s
    a, b = x[..., : D // 2], x[..., D // 2 :]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def positions_from_offsets(B, T, pos_offset=None):
    """positions[b, t] = pos_offset[b] + t (pos_offset None means all zero)."""
    off = np.zeros(B, dtype=np.int64) if pos_offset is None else np.asarray(pos_offset, dtype=np.int64)
    return off[:, None] + np.arange(T, dtype=np.int64)[None, :]


def qk_prologue_fwd(q, k, positions, eps, base=ROPE_BASE):
    """(q', k') = (RoPE(RMSNorm(q)), RoPE(RMSNorm(k))) at the given positions."""
    return (rope_rotate(rms_norm(q, eps), positions, base),
            rope_rotate(rms_norm(k, eps), positions, base))


def _prologue_bwd_one(x, dy, positions, eps, base):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    u = rope_rotate(dy, positions, base, inverse=True)  # transpose of the rotation
    r = np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    xu = (x * u).sum(axis=-1, keepdims=True)
    return u / r - x * xu / (D * r ** 3)


def qk_prologue_bwd(q, k, positions, dq_out, dk_out, eps, base=ROPE_BASE):
    """Gradients w.r.t. raw q and k given gradients w.r.t. q' and k'."""
    return (_prologue_bwd_one(q, dq_out, positions, eps, base),
            _prologue_bwd_one(k, dk_out, positions, eps, base))
