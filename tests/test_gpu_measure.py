"""The shader-clock probe (a measurement aid of the C ABI): it runs for the
requested wall time and reports a clock within the part's range, alone and
beside an attention forward on another stream."""

import math

import pytest

from transformer_attention_06_amd import synth

pytestmark = pytest.mark.gpu


def _mhz(out):
    cyc, ticks = (int(x) for x in out.cpu())
    return cyc, ticks, cyc / ticks * 100.0


def test_clock_probe_alone(gpu):
    import torch
    from transformer_attention_06_amd import native
    out = native.nc_measure_shader_clock(20)
    torch.cuda.synchronize()
    cyc, ticks, mhz = _mhz(out)
    print("probe alone:", cyc, "cycles", ticks, "ticks", round(mhz), "MHz", flush=True)
    assert 2_000_000 <= ticks < 2_000_000 + 1_000_000  # 20 ms of 100 MHz ticks, plus one sleep
    assert 50.0 < mhz < 3000.0


def test_clock_probe_beside_attention(gpu):
    import torch
    from transformer_attention_06_amd import native
    B, T, H, D = 4, 2048, 8, 128
    q, k, v = (synth.normal_device((B, T, H, D), 900 + i, "bf16") for i in range(3))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = native.nc_measure_shader_clock(30, stream=side)
    for _ in range(20):
        native.nc_attn_fwd(q, k, v, 0, 1.0 / math.sqrt(D))
    torch.cuda.synchronize()
    cyc, ticks, mhz = _mhz(out)
    print("probe beside the forward:", round(mhz), "MHz", flush=True)
    assert 3_000_000 <= ticks < 4_000_000
    assert 50.0 < mhz < 3000.0
