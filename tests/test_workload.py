"""Host logic: window schedule (golden, from the page's rule) and the work
counters (closed forms against brute-force enumeration)."""

import json
import os

import numpy as np
import pytest

from transformer_attention_06_amd import workload as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_window_schedule_golden():
    with open(os.path.join(GOLDEN, "window_schedule.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        w = W.layer_windows(c["n_layer"], 1024, c["pattern"])
        assert "".join("L" if x == W.FULL else "S" for x in w) == c["expect"]
        assert all(x in (W.FULL, 1024) for x in w)


def test_schedule_rejects_bad_pattern():
    with pytest.raises(ValueError):
        W.layer_windows(4, 1024, "SXL")


def _brute_pairs(T, w):
    n = 0
    for i in range(T):
        for j in range(T):
            if j <= i and (w <= 0 or w >= T or j > i - w):
                n += 1
    return n


@pytest.mark.parametrize("T,w", [(1, 0), (5, 1), (5, 2), (64, 16), (64, 0), (64, 64), (64, 65), (100, 37), (130, 129)])
def test_band_pairs_brute_force(T, w):
    assert W.band_pairs(T, w) == _brute_pairs(T, w)


def test_band_pairs_at_the_workload_sizes():
    # closed form by hand: T(T+1)/2 and wT - w(w-1)/2
    assert W.band_pairs(2048, 0) == 2048 * 2049 // 2 == 2098176
    assert W.band_pairs(2048, 1024) == 1024 * 2048 - 1024 * 1023 // 2 == 1573376
    d20 = W.workloads()["d20_bf16"]
    assert d20.windows.count(W.FULL) == 5 and d20.windows.count(1024) == 15
    pairs = sum(d20.B * d20.H * W.band_pairs(d20.T, w) for w in d20.windows)
    assert pairs == 10909286400
    assert W.attn_flops(d20.B, d20.T, d20.H, d20.D, d20.windows, "fwdbwd") == 12 * 128 * pairs


def test_decode_bytes_brute_force():
    rng = np.random.default_rng(0)
    lens = rng.integers(1, 50, 17)
    H, Hkv, D = 6, 2, 16
    for w in (0, 7, 60):
        total = 0
        for L in lens:
            keys = [j for j in range(L) if w <= 0 or j >= L - w]
            total += len(keys) * Hkv * D * 2 * 2 + H * D * 2 * 2 + H * 4 + 4
        assert W.decode_bytes(lens, H, Hkv, D, w) == total


def test_decode_step_bytes_brute_force():
    rng = np.random.default_rng(1)
    n_cached = rng.integers(0, 50, 17)
    H, Hkv, D = 6, 2, 16
    for w in (0, 1, 7, 60):
        total = 0
        for n in n_cached:
            old = [j for j in range(n) if w <= 0 or j >= n + 1 - w]  # cached keys the query sees
            total += len(old) * Hkv * D * 2 * 2 + Hkv * D * 2 * 2 + (H + 2 * Hkv) * D * 2
            total += H * D * 2 + H * 4 + 4 + D * 4
        assert W.decode_step_bytes(n_cached, H, Hkv, D, w) == total


def test_chunk_pairs_brute_force():
    for n in (0, 1, 5, 40, 300):
        for Tq in (1, 2, 17, 64):
            for w in (0, 1, 3, 6, 41, 100, 400):
                want = sum(min(n + t + 1, w) if w > 0 else n + t + 1 for t in range(Tq))
                assert W.chunk_pairs(n, Tq, w) == want, (n, Tq, w)
    assert W.chunk_pairs(0, 2048, 0) == W.band_pairs(2048, 0)
    assert W.chunk_pairs(0, 2048, 1024) == W.band_pairs(2048, 1024)
