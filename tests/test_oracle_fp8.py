"""Pins of the fp8 (e4m3) oracle against things other than itself: the
format's closed-form values, torch's float8_e4m3fn conversion (a library
routine) over every code and over random values, round-to-nearest-even tie
cases worked by hand, saturation, and invariants of the fp8 attention
forward (descale linearity, the one-key window). The last test reproduces
the tolerance budget of the GPU path: the only rounding it adds beyond
float32 is P rounded to e4m3 before the P V product."""

import math

import numpy as np
import pytest

import oracle


def test_closed_form_values():
    assert oracle.e4m3_value(0x00) == 0.0
    assert oracle.e4m3_value(0x80) == 0.0 and math.copysign(1.0, oracle.e4m3_value(0x80)) < 0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9  # smallest subnormal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert oracle.e4m3_value(0x08) == 2.0 ** -6  # smallest normal
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x39) == 1.125
    assert oracle.e4m3_value(0xB8) == -1.0
    assert oracle.e4m3_value(0x7E) == 448.0 == oracle.E4M3_MAX
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    # exactly two NaN codes, all other values distinct
    vals = oracle.e4m3_decode(np.arange(256))
    assert np.isnan(vals).sum() == 2
    finite = vals[~np.isnan(vals)]
    assert len(np.unique(finite)) == 253  # +0 and -0 compare equal


def test_decode_matches_torch_on_every_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ov = oracle.e4m3_decode(codes)
    assert np.array_equal(np.isnan(tv), np.isnan(ov))
    assert np.array_equal(tv[~np.isnan(tv)], ov[~np.isnan(ov)])


def test_encode_round_trip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)
    # ties go to the even mantissa
    assert oracle.e4m3_encode(1.0625) == 0x38  # between 1.0 (even) and 1.125
    assert oracle.e4m3_encode(1.1875) == 0x3A  # between 1.125 and 1.25 (even)
    assert oracle.e4m3_encode(0.5 * 2.0 ** -9) == 0x00  # between 0 (even) and the smallest subnormal
    assert oracle.e4m3_encode(1.5 * 2.0 ** -9) == 0x02  # between codes 1 and 2 (even)
    assert oracle.e4m3_encode(-1.0625) == 0xB8
    # just off a tie rounds to the nearer value
    assert oracle.e4m3_encode(np.nextafter(1.0625, 2.0)) == 0x39
    # saturation (no infinities in this format)
    assert oracle.e4m3_encode(464.0) == 0x7E and oracle.e4m3_encode(1e9) == 0x7E
    assert oracle.e4m3_encode(-1e9) == 0xFE
    assert oracle.e4m3_encode(float("nan")) == 0x7F


def test_encode_matches_torch_in_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0, 40, 100000), rng.uniform(-448, 448, 50000), rng.normal(0, 0.01, 50000)])
    te = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(te, oracle.e4m3_encode(x))


def test_tensorwise_scaling_maps_amax_to_the_largest_code():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 50, 7))
    codes, s = oracle.quantize_tensorwise(x)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] in (0x7E, 0xFE)
    assert s == np.max(np.abs(x)) / 448.0
    # every dequantized value is within half a step of the original
    err = np.abs(oracle.e4m3_decode(codes) * s - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-12))
    assert oracle.quantize_tensorwise(np.zeros(4))[1] == 1.0


def _codes(rng, shape):
    return oracle.quantize_tensorwise(rng.standard_normal(shape))


def test_fp8_forward_invariants():
    rng = np.random.default_rng(7)
    B, T, H, Hkv, D = 1, 40, 4, 2, 32
    (q8, sq), (k8, sk), (v8, sv) = _codes(rng, (B, T, H, D)), _codes(rng, (B, T, Hkv, D)), _codes(rng, (B, T, Hkv, D))
    scale = 1 / math.sqrt(D)
    o1, l1 = oracle.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, 9, scale)
    # v's descale scales out only
    o2, l2 = oracle.attn_fwd_fp8(q8, k8, v8, sq, sk, 2 * sv, 9, scale)
    np.testing.assert_allclose(o2, 2 * o1, rtol=1e-14, atol=0)
    np.testing.assert_allclose(l2, l1, rtol=1e-14, atol=0)
    # q's descale acts like the softmax scale
    o3, l3 = oracle.attn_fwd_fp8(q8, k8, v8, 3 * sq, sk, sv, 9, scale)
    o4, l4 = oracle.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, 9, 3 * scale)
    np.testing.assert_allclose(o3, o4, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l3, l4, rtol=1e-12, atol=1e-14)
    # a one-key window returns the dequantized v of the same position
    o5, l5 = oracle.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, 1, scale)
    vd = oracle.e4m3_decode(v8) * sv
    G = H // Hkv
    for h in range(H):
        np.testing.assert_array_equal(o5[:, :, h], vd[:, :, h // G])
        s_ii = scale * np.einsum("btd,btd->bt", oracle.e4m3_decode(q8[:, :, h]) * sq,
                                 oracle.e4m3_decode(k8[:, :, h // G]) * sk)
        np.testing.assert_allclose(l5[:, h], s_ii, rtol=1e-12, atol=1e-14)


def test_tolerance_budget_of_p_in_e4m3():
    """Emulates the GPU path's one extra rounding (P = exp(s - m) rounded to
    e4m3 for P V, the row sum from the unrounded P, out rounded to bf16) and
    checks its distance from the definition stays well inside the fp8
    tolerance of the parity tests (out rel-L2 <= 4e-2)."""
    torch = pytest.importorskip("torch")
    from tests.parity import TOL
    tol = TOL["fp8"]["out"][1]
    rng = np.random.default_rng(8)
    B, T, H, D = 1, 256, 2, 128
    for w in (0, 64):
        (q8, sq), (k8, sk), (v8, sv) = (_codes(rng, (B, T, H, D)) for _ in range(3))
        scale = 1 / math.sqrt(D)
        ro, _ = oracle.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, w, scale)
        q, k, v = (oracle.e4m3_decode(c) * s for c, s in ((q8, sq), (k8, sk), (v8, sv)))
        mask = oracle.visible_mask(T, w)
        eo = np.zeros_like(ro)
        for h in range(H):
            s = np.where(mask, scale * q[0, :, h] @ k[0, :, h].T, -np.inf)
            p = np.exp(s - s.max(1, keepdims=True))
            p8 = oracle.e4m3_decode(oracle.e4m3_encode(p))
            eo[0, :, h] = (p8 @ v[0, :, h]) / p.sum(1, keepdims=True)
        eo = torch.from_numpy(eo).to(torch.bfloat16).double().numpy()
        rel = np.linalg.norm(eo - ro) / np.linalg.norm(ro)
        assert rel < tol / 1.5, (w, rel)
