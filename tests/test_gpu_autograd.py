"""The torch autograd ops over the C ABI: attention and attention with the
QK prologue, against the entry points they call (bit for bit) and against
the fp64 oracle, with a loss that is not linear in the output."""

import math

import numpy as np
import pytest

import oracle
from tests.parity import check, f64, inputs

pytestmark = pytest.mark.gpu
EPS = 2.0 ** -23


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,T,H,Hkv,D,w", [(2, 300, 4, 2, 128, 64), (1, 200, 2, 2, 64, 0)])
def test_attention_autograd(gpu, dtype, B, T, H, Hkv, D, w):
    import torch
    from transformer_attention_06_amd import native
    print("case", B, T, H, Hkv, D, w, dtype, flush=True)
    scale = 1.0 / math.sqrt(D)
    q, k, v, do = inputs([(B, T, H, D), (B, T, Hkv, D), (B, T, Hkv, D), (B, T, H, D)], 800, dtype)
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = native.attention(qa, ka, va, w, scale)
    out.backward(do)
    # the same calls made directly
    o2, l2 = native.nc_attn_fwd(q, k, v, w, scale)
    dq2, dk2, dv2 = native.nc_attn_bwd(q, k, v, o2, l2, do, w, scale)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), o2)
    assert torch.equal(qa.grad, dq2) and torch.equal(ka.grad, dk2) and torch.equal(va.grad, dv2)
    ro, _ = oracle.attn_fwd(f64(q), f64(k), f64(v), w, scale)
    gq, gk, gv = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), w, scale)
    check("autograd out", f64(out.detach()), ro, dtype, "out")
    check("autograd dq", f64(qa.grad), gq, dtype, "grad")
    check("autograd dk", f64(ka.grad), gk, dtype, "grad")
    check("autograd dv", f64(va.grad), gv, dtype, "grad")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_qk_prologue_autograd(gpu, dtype):
    import torch
    from transformer_attention_06_amd import native
    B, T, H, Hkv, D, w = 2, 260, 4, 2, 128, 100
    scale = 1.0 / math.sqrt(D)
    q, k, v = inputs([(B, T, H, D), (B, T, Hkv, D), (B, T, Hkv, D)], 810, dtype)
    c, s = native.nc_rope_table(2048, D)
    offs = np.array([5, 700], np.int32)
    po = torch.from_numpy(offs).cuda()
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = native.attention_qk_prologue(qa, ka, va, c, s, EPS, w, scale, pos_offset=po)
    # a loss that is not linear in out: L = sum(out^2) / 2, so dL/dout = out
    (out.float().pow(2).sum() / 2).backward()
    do = out.detach().clone()
    qp, kp, o2, l2 = native.nc_attn_fwd_prologue(q, k, v, c, s, EPS, w, scale, pos_offset=po)
    dq2, dk2, dv2 = native.nc_attn_bwd_prologue(qp, kp, v, o2, l2, do, w, scale, q, k, c, s, EPS, pos_offset=po)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), o2)
    assert torch.equal(qa.grad, dq2) and torch.equal(ka.grad, dk2) and torch.equal(va.grad, dv2)
    pos = oracle.positions_from_offsets(B, T, offs)
    rq, rk = (oracle.round_to(x, dtype) for x in oracle.qk_prologue_fwd(f64(q), f64(k), pos, EPS))
    ro, _ = oracle.attn_fwd(rq, rk, f64(v), w, scale)
    check("prologue autograd out", f64(out.detach()), ro, dtype, "out")
    gqp, gkp, gv = oracle.attn_bwd(rq, rk, f64(v), f64(do), w, scale)
    gq, gk = oracle.qk_prologue_bwd(f64(q), f64(k), pos, gqp, gkp, EPS)
    check("prologue autograd dq", f64(qa.grad), gq, dtype, "grad")
    check("prologue autograd dk", f64(ka.grad), gk, dtype, "grad")
    check("prologue autograd dv", f64(va.grad), gv, dtype, "grad")
