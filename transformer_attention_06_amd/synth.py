"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module draws random numbers and converts storage types; it holds none
of the attention arithmetic. Small inputs come from numpy's PCG64
(``default_rng(seed)``) in float32 and are rounded to bfloat16 by torch's
round-to-nearest-even cast on the CPU; full-size inputs are drawn directly
on the GPU from a seeded torch generator so that tens of GB of activations
do not pass through the host.

Value recipe: every tensor is i.i.d. N(0, 1). After the weightless QK
RMSNorm each head vector has unit RMS, so N(0, 1) q and k carry the scale
the attention kernels see in the model; v and dout are likewise unit scale.
Decode cache lengths are uniform integers in [1, T_max].
"""

import numpy as np


def normal_np(shape, seed):
    """float32 N(0, 1) array from numpy PCG64."""
    return np.random.default_rng(seed).standard_normal(size=shape, dtype=np.float32)


def seqlens_np(B, T_max, seed):
    """int32 lengths uniform on 1..T_max (inclusive)."""
    return np.random.default_rng(seed).integers(1, T_max + 1, size=B).astype(np.int32)


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def normal_torch(shape, seed, dtype="f32", device="cpu"):
    """N(0, 1) tensor from numpy PCG64, cast (RNE) to dtype, moved to device."""
    import torch
    t = torch.from_numpy(normal_np(shape, seed)).to(torch_dtype(dtype))
    return t.to(device)


def normal_device(shape, seed, dtype="bf16", device="cuda"):
    """N(0, 1) tensor drawn on the device from a seeded torch generator.

    Used for the full-size workloads; the float32 draw is cast (RNE) to
    dtype on the device.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return t.to(torch_dtype(dtype))


def to_f64(t):
    """Exact float64 numpy copy of a (CPU or device) float32/bfloat16 tensor."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
