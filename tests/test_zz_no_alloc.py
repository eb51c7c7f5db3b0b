"""nc_attn_decode_step_noalloc (the decode step with the split-K partials in
the library's per-GPU scratch instead of a caller workspace) against
nc_attn_decode_step, through the C ABI: two calls in a row, the second with
a smaller input, each on identical copies of the caches. Both run the same
kernels on the same inputs, so out, lse and the written cache slots must be
identical bit for bit (stronger than the oracle tolerances they both meet)."""

import math

import numpy as np
import pytest

from tests.parity import inputs
from transformer_attention_06_amd import synth

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -23


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _case(native, B, H, Hkv, D, T_max, w, seed):
    import torch
    print("no-alloc decode step case", B, H, Hkv, D, T_max, w, flush=True)
    scale = 1.0 / math.sqrt(D)
    q, kn, vn, kc, vc = inputs([(B, H, D), (B, Hkv, D), (B, Hkv, D), (B, T_max, Hkv, D), (B, T_max, Hkv, D)],
                               seed, "bf16")
    n = (synth.seqlens_np(B, T_max, seed + 9) - 1).astype(np.int32)
    n[0] = T_max - 1
    nd = torch.from_numpy(n).cuda()
    c, s = native.nc_rope_table(T_max, D)
    kc2, vc2 = kc.clone(), vc.clone()
    ref_o, ref_l = native.nc_attn_decode_step(q, kn, vn, kc, vc, nd, c, s, EPS, w, scale)
    out = torch.full((B, H, D), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    native.nc_attn_decode_step_noalloc(q, kn, vn, kc2, vc2, nd, c, s, EPS, w, scale, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref_o))
    assert torch.equal(_bits(lse), _bits(ref_l))
    assert torch.equal(_bits(kc2), _bits(kc)) and torch.equal(_bits(vc2), _bits(vc))


def test_noalloc_decode_step_matches_the_workspace_call(gpu):
    from transformer_attention_06_amd import native
    # the decode workload's shape (partials ~10.6 MB of the 32 MiB scratch), then a smaller one
    _case(native, 64, 10, 10, 128, 2048, 1024, 1500)
    _case(native, 3, 8, 2, 64, 300, 0, 1510)


def test_noalloc_rejects_sizes_beyond_the_scratch(gpu):
    import torch
    from transformer_attention_06_amd import native
    B, H, Hkv, D, T_max = 64, 32, 4, 128, 4096  # partials (~272 MB) far beyond 32 MiB
    need = native.nc_attn_decode_step_workspace_bytes(native.NC_BF16, B, H, Hkv, D, T_max)
    assert need > native.NC_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, D), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, 16, Hkv, D), dtype=torch.bfloat16, device="cuda")
    L = native.lib()
    c, s = native.nc_rope_table(16, D)
    n = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    lse = torch.zeros((B, H), dtype=torch.float32, device="cuda")
    # raw C call with T_max larger than the (never read) cache tensors: validation
    # rejects the size before any launch, so nothing is touched
    st = L.nc_attn_decode_step_noalloc(native.NC_BF16, B, H, Hkv, D, T_max, q.data_ptr(), kn.data_ptr(),
                                       kn.data_ptr(), kc.data_ptr(), kc.data_ptr(), n.data_ptr(), c.data_ptr(),
                                       s.data_ptr(), 16, EPS, 0, 0.088, out.data_ptr(), lse.data_ptr(), None)
    assert st == 2, st
    assert b"scratch" in L.nc_last_error_message()
    assert (out == 0).all() and (lse == 0).all()
