"""Host-side logic of the path: the per-layer window schedule, the workload
shapes and the algorithmic work counters used for throughput.

Window schedule ("nanochat Admin & Developer Guide", section 3,
"Sliding-window attention"): a pattern string over {S, L} is tiled across
the layers, L meaning full context and S a short window; the last layer is
always L. The page's example of the S size is self-contradictory (a quarter
of 2048 is not 768), so the short window is a parameter; the workloads here
use 1024.

Work counters (section 3, "FLOPs and scaling-parameter accounting": the FLOP
estimate counts attention over the reduced effective sequence of the
sliding-window layers). Only visible (query, key) pairs count:
  pairs(T, w) = w*T - w*(w-1)/2 for 1 <= w < T, T*(T+1)/2 for full causal;
  forward  = 4 * D flops per visible pair per (b, h)   (QK^T and PV);
  backward = 8 * D flops per visible pair per (b, h)   (twice the forward).
Decode bytes count each visible cached K and V row once plus q, out, lse and
the length word; split-K partials and cache re-reads are not counted.
"""

from dataclasses import dataclass, field
from typing import List

FULL = 0  # window value meaning full causal attention


def layer_windows(n_layer, short_window, pattern="SSSL"):
    """Per-layer window list: pattern tiled over layers, last layer full."""
    if not pattern or any(c not in "SL" for c in pattern.upper()):
        raise ValueError("pattern must be a non-empty string over {S, L}")
    pat = pattern.upper()
    w = [short_window if pat[l % len(pat)] == "S" else FULL for l in range(n_layer)]
    if n_layer:
        w[-1] = FULL
    return w


def is_full(window, n_keys):
    return window <= 0 or window >= n_keys


def band_pairs(T, window):
    """Number of visible (query, key) pairs for one (b, h) at length T."""
    if is_full(window, T):
        return T * (T + 1) // 2
    w = window
    return w * T - w * (w - 1) // 2


def attn_flops(B, T, H, D, windows, kind="fwd"):
    """Band-counted flops over a list of per-call windows."""
    per_pair = {"fwd": 4 * D, "bwd": 8 * D, "fwdbwd": 12 * D}[kind]
    return sum(B * H * band_pairs(T, w) * per_pair for w in windows)


def chunk_pairs(n_cached, Tq, window):
    """Visible (query, key) pairs of one (b, h) for a chunk of Tq queries after
    n_cached cached tokens: query t at position p = n_cached + t sees
    min(p + 1, window) keys (p + 1 for a full layer)."""
    lo, hi = n_cached + 1, n_cached + Tq  # keys seen by the first and last query, full layer
    if window <= 0 or window >= hi:
        return (lo + hi) * Tq // 2
    if window <= lo:
        return window * Tq
    ramp = window - lo  # queries still below the window
    return (lo + window - 1) * ramp // 2 + window * (Tq - ramp)


def decode_keys(seqlen, window):
    """Keys a decode query at length seqlen reads."""
    return seqlen if is_full(window, seqlen) else window


def decode_bytes(seqlens, H, Hkv, D, window, elem_bytes=2):
    """Algorithmic HBM bytes of one decode call."""
    total = 0
    for L in seqlens:
        n = decode_keys(int(L), window)
        total += 2 * Hkv * n * D * elem_bytes  # K and V rows
        total += 2 * H * D * elem_bytes  # q in, out
        total += H * 4 + 4  # lse, seqlen
    return total


def decode_step_bytes(cache_seqlens, H, Hkv, D, window, elem_bytes=2):
    """Algorithmic HBM bytes of one decode step (append + decode): the cached
    keys the new query sees are read (K and V), the new k' and v are written
    once, the raw q, k, v of the token are read, out and lse written, plus
    the row's length and the cos/sin row of its position (float32)."""
    total = 0
    for n in cache_seqlens:
        old = decode_keys(int(n) + 1, window) - 1  # visible keys other than the new one
        total += 2 * Hkv * old * D * elem_bytes  # cached K and V rows read
        total += 2 * Hkv * D * elem_bytes  # k', v written into the cache
        total += (H + 2 * Hkv) * D * elem_bytes  # raw q, k, v read
        total += H * D * elem_bytes + H * 4 + 4  # out, lse, length
        total += D * 4  # cos and sin rows (D/2 each)
    return total


@dataclass
class Workload:
    name: str
    dtype: str
    B: int
    T: int
    H: int
    Hkv: int
    D: int
    windows: List[int] = field(default_factory=list)
    prologue: bool = False
    decode: bool = False

    @property
    def scale(self):
        return 1.0 / float(self.D) ** 0.5


def workloads():
    """The five synthetic workloads (shapes as the pages' models use them)."""
    return {
        "tiny_f32": Workload("tiny_f32", "f32", 1, 64, 2, 1, 32, [16, FULL], prologue=True),
        "d12_bf16": Workload("d12_bf16", "bf16", 16, 2048, 6, 6, 128, layer_windows(12, 1024)),
        "d20_bf16": Workload("d20_bf16", "bf16", 32, 2048, 10, 10, 128, layer_windows(20, 1024)),
        "gqa_bf16": Workload("gqa_bf16", "bf16", 8, 2048, 16, 4, 128, [1024, FULL]),
        "decode_bf16": Workload("decode_bf16", "bf16", 64, 2048, 10, 10, 128,
                                layer_windows(20, 1024), decode=True),
    }
