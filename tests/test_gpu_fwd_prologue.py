"""GPU parity of nc_attn_fwd_prologue (QK prologue and attention forward in
one call; bf16 applies the query prologue inside the forward kernel) against
the fp64 oracle, and against the two separate calls."""

import math

import numpy as np
import pytest

import oracle
from tests.parity import check, f64, inputs

pytestmark = pytest.mark.gpu
EPS = 2.0 ** -23

CASES = [
    # B, T, H, Hkv, D, window, offsets
    (1, 64, 2, 1, 32, 16, False),
    (2, 130, 4, 2, 64, 0, True),
    (1, 257, 4, 2, 128, 100, True),
    (2, 200, 2, 2, 128, 0, False),
    (3, 97, 6, 3, 32, 0, True),
    (1, 300, 8, 2, 64, 129, False),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}T{}H{}Hkv{}D{}w{}o{}".format(*c))
def test_fwd_prologue_vs_oracle(gpu, dtype, case):
    import torch
    from transformer_attention_06_amd import native
    B, T, H, Hkv, D, w, offsets = case
    print("case", case, dtype, flush=True)
    scale = 1.0 / math.sqrt(D)
    q, k, v = inputs([(B, T, H, D), (B, T, Hkv, D), (B, T, Hkv, D)], 600, dtype)
    c, s = native.nc_rope_table(4096, D)
    offs = np.array([3, 900, 41][:B], np.int32) if offsets else None
    po = torch.from_numpy(offs).cuda() if offsets else None
    qp, kp, out, lse = native.nc_attn_fwd_prologue(q, k, v, c, s, EPS, w, scale, pos_offset=po)
    pos = oracle.positions_from_offsets(B, T, offs)
    rq, rk = (oracle.round_to(x, dtype) for x in oracle.qk_prologue_fwd(f64(q), f64(k), pos, EPS))
    ro, rl = oracle.attn_fwd(rq, rk, f64(v), w, scale)
    check("q'", f64(qp), rq, dtype, "out")
    check("k'", f64(kp), rk, dtype, "out")
    check("out", f64(out), ro, dtype, "out")
    check("lse", f64(lse), rl, dtype, "lse")


def test_fwd_prologue_matches_the_two_calls(gpu):
    import torch
    from transformer_attention_06_amd import native
    B, T, H, Hkv, D = 2, 333, 4, 2, 128
    q, k, v = inputs([(B, T, H, D), (B, T, Hkv, D), (B, T, Hkv, D)], 610, "bf16")
    c, s = native.nc_rope_table(1024, D)
    po = torch.tensor([0, 500], dtype=torch.int32, device="cuda")
    for w in (0, 100):
        qp, kp, out, lse = native.nc_attn_fwd_prologue(q, k, v, c, s, EPS, w, 0.1, pos_offset=po)
        qp2, kp2 = native.nc_qk_prologue_fwd(q, k, c, s, EPS, pos_offset=po)
        o2, l2 = native.nc_attn_fwd(qp2, kp2, v, w, 0.1)
        assert torch.equal(kp, kp2)
        # q' sums its squares in another order: at most one bf16 step apart, rarely
        dq = (qp.float() - qp2.float()).abs()
        step = qp2.float().abs() * 2.0 ** -7 + 1e-30
        assert bool((dq <= step).all()), "q' differs by more than one bf16 rounding"
        assert float((dq > 0).float().mean()) < 1e-3
        same = bool(torch.equal(qp, qp2))
        if same:
            assert torch.equal(out, o2) and torch.equal(lse, l2)
        else:
            assert float((out.float() - o2.float()).abs().max()) < 2e-2
            assert float((lse - l2).abs().max()) < 1e-3


def test_fwd_prologue_position_outside_table_is_nan(gpu):
    import torch
    from transformer_attention_06_amd import native
    B, T, H, D = 2, 40, 2, 64
    q, k, v = inputs([(B, T, H, D), (B, T, H, D), (B, T, H, D)], 620, "bf16")
    c, s = native.nc_rope_table(64, D)
    po = torch.tensor([0, 30], dtype=torch.int32, device="cuda")  # row 1 reaches position 69 >= 64
    qp, kp, out, lse = native.nc_attn_fwd_prologue(q, k, v, c, s, EPS, 0, 0.125, pos_offset=po)
    assert torch.isfinite(qp[0].float()).all() and torch.isfinite(out[0].float()).all()
    assert torch.isnan(qp[1, 34:].float()).all() and torch.isfinite(qp[1, :34].float()).all()
