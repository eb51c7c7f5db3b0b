"""The entry points only enqueue kernels on the caller's stream (no
allocation, no memset, no synchronisation), so a caller can capture them in
a HIP graph. One training layer (fused prologue + forward, backward through
attention and prologue) and a decode call are captured once and replayed
three times, with eager calls of the same entry points on other buffers and
synchronisations in between; every replay must reproduce the eager results
bit for bit (all kernels here are deterministic)."""

import numpy as np
import pytest

from tests.parity import inputs

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -23


def test_captured_layer_replays_match_eager(gpu):
    import torch
    from transformer_attention_06_amd import native
    B, T, H, Hkv, D, w, scale = 2, 300, 4, 2, 128, 100, 0.0884
    dt = native.NC_BF16
    q, k, v, do = inputs([(B, T, H, D), (B, T, Hkv, D), (B, T, Hkv, D), (B, T, H, D)], 950, "bf16")
    cos, sin = native.nc_rope_table(T, D)
    lens = torch.from_numpy(np.array([T, 137], np.int32)).cuda()
    qd = q[:, 5].contiguous()

    def buffers():
        e = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda")  # noqa: E731
        return dict(qp=e(B, T, H, D), kp=e(B, T, Hkv, D), out=e(B, T, H, D),
                    lse=torch.empty(B, H, T, device="cuda"), dq=e(B, T, H, D), dk=e(B, T, Hkv, D),
                    dv=e(B, T, Hkv, D), od=e(B, H, D), ld=torch.empty(B, H, device="cuda"),
                    ws=torch.empty(native.nc_attn_bwd_workspace_bytes(dt, B, T, H, Hkv, D), dtype=torch.uint8,
                                   device="cuda"),
                    dws=torch.empty(native.nc_attn_decode_workspace_bytes(dt, B, H, Hkv, D, T), dtype=torch.uint8,
                                    device="cuda"))

    def run(x, qq, kk, vv):
        native.nc_attn_fwd_prologue(qq, kk, vv, cos, sin, EPS, w, scale, q_out=x["qp"], k_out=x["kp"],
                                    out=x["out"], lse=x["lse"])
        native.nc_attn_bwd_prologue(x["qp"], x["kp"], vv, x["out"], x["lse"], do, w, scale, qq, kk, cos, sin, EPS,
                                    dq=x["dq"], dk=x["dk"], dv=x["dv"], workspace=x["ws"])
        native.nc_attn_decode(qd, x["kp"], vv, lens, w, scale, out=x["od"], lse=x["ld"], workspace=x["dws"])

    names = ("qp", "kp", "out", "lse", "dq", "dk", "dv", "od", "ld")
    eager = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(eager, q, k, v)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    want = {n: eager[n].clone() for n in names}

    cap = buffers()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(cap, q, k, v)
    torch.cuda.synchronize()
    other = buffers()
    q2, k2, v2 = (t.flip(1).contiguous() for t in (q, k, v))
    for rep in range(3):
        print("replay", rep, flush=True)
        for n in names:
            cap[n].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            a, b = cap[n], want[n]
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), (rep, n)
        run(other, q2, k2, v2)  # eager work between replays
        torch.cuda.synchronize()


def test_captured_decode_step_replays_match_eager(gpu):
    # nc_attn_decode_step writes the new token into the caches in place: the
    # caches are restored (eagerly) before every replay, and each replay must
    # give the eager out, lse and caches bit for bit
    import torch
    from transformer_attention_06_amd import native
    B, H, Hkv, D, T_max, w, scale = 5, 8, 2, 128, 700, 256, 0.0884
    dt = native.NC_BF16
    q, kn, vn, kc0, vc0 = inputs([(B, H, D), (B, Hkv, D), (B, Hkv, D), (B, T_max, Hkv, D), (B, T_max, Hkv, D)],
                                 960, "bf16")
    cos, sin = native.nc_rope_table(T_max, D)
    n = torch.from_numpy(np.array([0, 63, 64, 300, T_max - 1], np.int32)).cuda()
    ws = torch.empty(native.nc_attn_decode_step_workspace_bytes(dt, B, H, Hkv, D, T_max), dtype=torch.uint8,
                     device="cuda")

    def state():
        return dict(kc=kc0.clone(), vc=vc0.clone(), od=torch.empty(B, H, D, dtype=torch.bfloat16, device="cuda"),
                    ld=torch.empty(B, H, device="cuda"))

    def run(x):
        native.nc_attn_decode_step(q, kn, vn, x["kc"], x["vc"], n, cos, sin, EPS, w, scale, out=x["od"],
                                   lse=x["ld"], workspace=ws)

    names = ("kc", "vc", "od", "ld")
    eager = state()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(eager)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    cap = state()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(cap)
    torch.cuda.synchronize()
    other = state()
    for rep in range(3):
        print("decode step replay", rep, flush=True)
        cap["kc"].copy_(kc0)
        cap["vc"].copy_(vc0)
        cap["od"].fill_(float("nan"))
        cap["ld"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for nm in names:
            a, b = cap[nm], eager[nm]
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), (rep, nm)
        other["kc"].copy_(kc0)
        other["vc"].copy_(vc0)
        run(other)  # eager work between replays (same workspace, ordered on this stream)
        torch.cuda.synchronize()
