"""The Python binding checks what the C ABI cannot see (the library gets
only pointers and sizes): device, exact shape, dtype and contiguity of every
tensor, before anything is launched. CPU tests of the checks themselves and
of the device check; the GPU test passes mismatched tensors through the
entry points."""

import pytest

torch = pytest.importorskip("torch")

from transformer_attention_06_amd import native  # noqa: E402

CPU = torch.device("cpu")


def test_arg_accepts_a_matching_tensor():
    t = torch.zeros(2, 3, 4)
    assert native._arg(t, "x", (2, 3, 4), (torch.float32,), CPU) == t.data_ptr()
    assert native._arg(None, "x", (1,), None, CPU, optional=True) is None


@pytest.mark.parametrize("bad, err, what", [
    (torch.zeros(2, 3, 5), ValueError, "shape"),
    (torch.zeros(2, 3, 4, dtype=torch.bfloat16), TypeError, "dtype"),
    (torch.zeros(2, 4, 3).transpose(1, 2), ValueError, "contiguous"),
    ([0.0] * 24, TypeError, "torch.Tensor"),
])
def test_arg_rejects(bad, err, what):
    with pytest.raises(err, match=what):
        native._arg(bad, "x", (2, 3, 4), (torch.float32,), CPU)


def test_arg_rejects_a_missing_required_tensor():
    with pytest.raises(ValueError, match="required"):
        native._arg(None, "x", None, None, CPU)


def test_entry_points_reject_host_tensors():
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on a GPU"):
        native.nc_attn_fwd(q, q[:, :, :1].contiguous(), q[:, :, :1].contiguous(), 0, 0.125)
    with pytest.raises(ValueError, match="on a GPU"):
        native.nc_attn_decode(torch.zeros(2, 2, 64), torch.zeros(2, 8, 2, 64), torch.zeros(2, 8, 2, 64),
                              torch.ones(2, dtype=torch.int32), 0, 0.125)


@pytest.mark.gpu
def test_mismatched_tensors_raise_before_launch(gpu):
    B, T, H, Hkv, D = 2, 40, 4, 2, 64
    dev = "cuda"
    q = torch.randn(B, T, H, D, device=dev, dtype=torch.bfloat16)
    k = torch.randn(B, T, Hkv, D, device=dev, dtype=torch.bfloat16)
    v = torch.randn(B, T, Hkv, D, device=dev, dtype=torch.bfloat16)
    bad = [
        dict(v=torch.randn(B, T - 1, Hkv, D, device=dev, dtype=torch.bfloat16)),
        dict(v=v.float()),
        dict(v=v.cpu()),
        dict(out=torch.empty(B, T, H, D - 1, device=dev, dtype=torch.bfloat16)),
        dict(lse=torch.empty(B, T, H, device=dev)),
        dict(lse=torch.empty(B, H, T, device=dev, dtype=torch.bfloat16)),
    ]
    for kw in bad:
        args = dict(q=q, k=k, v=v)
        args.update({n: t for n, t in kw.items() if n in args})
        extra = {n: t for n, t in kw.items() if n not in args}
        print("mismatch", list(kw), flush=True)
        with pytest.raises((ValueError, TypeError)):
            native.nc_attn_fwd(args["q"], args["k"], args["v"], 0, 0.125, **extra)
    out, lse = native.nc_attn_fwd(q, k, v, 0, 0.125)
    with pytest.raises(ValueError):  # dout one row short
        native.nc_attn_bwd(q, k, v, out, lse, out[:, :-1].contiguous(), 0, 0.125)
    torch.cuda.synchronize()
