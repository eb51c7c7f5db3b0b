#!/usr/bin/env python3
"""Throughput of the nanochat attention hot path on one MI355X.

One step = one pass of the training-side hot path over one batch of the
d20-shaped workload (B=32, T=2048, H=Hkv=10, D=128, bf16, 20 layers in the
SSSL window schedule: 15 layers with a 1024-key window, 5 full causal):
for every layer the QK prologue (RMSNorm + RoPE) forward and attention
forward, then, in reverse layer order, the backward through attention and
the prologue (one call; the prologue backward is applied as the backward
kernels store dq and dk). The reported value is band-counted attention fwd+bwd FLOPs
(12 * D per visible query/key pair, per (b, h)) divided by the step time, so
the prologue's time counts against it. The decode workload (64 rows, one
query each, cache lengths uniform on 1..2048, same 20-layer schedule) is
timed as a separate phase and reported in GB/s of algorithmic bytes.
After the timed steps the same steps run twice more: once with events
between the kernels (per-kernel times) and once beside a one-wave probe on
a second stream that reads the shader clock they run at (`sclk_mhz`, and
the roofline fraction at that clock next to the nominal one).

Inputs are seeded N(0, 1) bf16 tensors drawn on the device and resident in
HBM before the timed region. Prints one JSON line on stdout; progress goes
to stderr.
"""

import argparse
import json
import math
import os
import sys
import time

# Host threads for the oracle baseline: the CPUs this process may run on,
# capped by OMP_NUM_THREADS where the environment sets it; the BLAS pools
# are sized before numpy loads.
AFFINITY_CPUS = len(os.sched_getaffinity(0))
CPU_THREADS = max(1, min(AFFINITY_CPUS, int(os.environ.get("OMP_NUM_THREADS", AFFINITY_CPUS) or AFFINITY_CPUS)))
for _v in ("OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "OMP_NUM_THREADS"):
    os.environ.setdefault(_v, str(CPU_THREADS))

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
NOMINAL_SCLK_MHZ = 2400.0  # the shader clock that peak is quoted at
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "attn fwd+bwd TFLOP/s (band-counted) at d20 T=2048; decode GB/s"


ROOT = os.path.dirname(os.path.abspath(__file__))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(label):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary (profiles/attn_d20_traffic.json: FETCH_SIZE and WRITE_SIZE, each
    scaled by a plain-copy calibration), or None when there is no summary for
    it or its source file has changed since the counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "attn_d20_traffic.json")) as f:
            d = json.load(f)[label]
        with open(os.path.join(ROOT, d["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != d["source_sha256"]:
                return None
        return {"bytes": round(d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"]),
                "read": round(d["fetch_bytes_per_launch"]), "written": round(d["write_bytes_per_launch"])}
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the d12, GQA and tiny rows")
    return ap.parse_args()


class Timer:
    """Pairs of torch.cuda events on the current stream, summed per label."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def pair(self, label):
        t = self.torch
        b, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        self.pairs.setdefault(label, []).append((b, e))
        return b, e

    def add(self, label, b, e):
        self.pairs.setdefault(label, []).append((b, e))

    def totals(self):
        return {k: (sum(b.elapsed_time(e) for b, e in v), len(v)) for k, v in self.pairs.items()}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(attention shards by batch row or GQA group with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from transformer_attention_06_amd import native, synth
    from transformer_attention_06_amd.workload import (FULL, attn_flops, band_pairs, chunk_pairs, decode_bytes,
                                                       decode_step_bytes, workloads)

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    native.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    wl = workloads()["d20_bf16"]
    B, T, H, Hkv, D = wl.B, wl.T, wl.H, wl.Hkv, wl.D
    L = len(wl.windows)
    scale, eps = wl.scale, 2.0 ** -23
    log(f"allocating d20 inputs: {L} layers x q,k,v,dout [{B},{T},{H},{D}] bf16")
    qr = [synth.normal_device((B, T, H, D), 1000 + 10 * l, "bf16") for l in range(L)]
    kr = [synth.normal_device((B, T, Hkv, D), 1001 + 10 * l, "bf16") for l in range(L)]
    vv = [synth.normal_device((B, T, Hkv, D), 1002 + 10 * l, "bf16") for l in range(L)]
    do = [synth.normal_device((B, T, H, D), 1003 + 10 * l, "bf16") for l in range(L)]
    qp = [torch.empty_like(x) for x in qr]
    kp = [torch.empty_like(x) for x in kr]
    out = [torch.empty_like(x) for x in qr]
    lse = [torch.empty((B, H, T), dtype=torch.float32, device=dev) for _ in range(L)]
    dv = torch.empty_like(vv[0])
    dq, dk = torch.empty_like(qr[0]), torch.empty_like(kr[0])
    ws = torch.empty(native.nc_attn_bwd_workspace_bytes(native.NC_BF16, B, T, H, Hkv, D),
                     dtype=torch.uint8, device=dev)
    cos, sin = native.nc_rope_table(10 * T, D, 100000.0)

    def wtag(w):
        return "full" if w == FULL or w <= 0 else str(w)

    def step(tm=None):
        def ev(label):
            return tm.pair(label) if tm else (None, None)

        for l in range(L):
            # prologue and attention forward in one call: the keys' prologue
            # kernel, then the forward kernel, which applies the queries'
            # prologue as it loads them and stores q' for the backward
            if tm:
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                for x in (e0, e1, e2):
                    x.record()  # materialise the events before handing them to the library
                tm.add("prologue_fwd_k", e0, e1)
                tm.add("attn_fwd", e1, e2)
                tm.add("attn_fwd@" + wtag(wl.windows[l]), e1, e2)
                native.nc_profile_fwd_prologue(e0, e1, e2)
            native.nc_attn_fwd_prologue(qr[l], kr[l], vv[l], cos, sin, eps, wl.windows[l], scale, q_out=qp[l],
                                        k_out=kp[l], out=out[l], lse=lse[l])
            if tm:
                native.nc_profile_fwd_prologue()
        for l in reversed(range(L)):
            b, e = ev("attn_bwd")
            if tm:
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                for x in (e0, e1, e2):
                    x.record()  # materialise the events before handing them to the library
                tm.add("attn_bwd_dq", e0, e1)
                tm.add("attn_bwd_dkdv", e1, e2)
                tm.add("attn_bwd_dq@" + wtag(wl.windows[l]), e0, e1)
                tm.add("attn_bwd_dkdv@" + wtag(wl.windows[l]), e1, e2)
                tm.add("attn_bwd@" + wtag(wl.windows[l]), e0, e2)
                native.nc_profile_bwd_main(e0, e1, e2)
            b and b.record()
            # attention backward and the prologue backward in one call: the
            # backward kernels store dq, dk w.r.t. the raw q, k directly
            native.nc_attn_bwd_prologue(qp[l], kp[l], vv[l], out[l], lse[l], do[l], wl.windows[l], scale,
                                        qr[l], kr[l], cos, sin, eps, dq=dq, dk=dk, dv=dv, workspace=ws)
            e and e.record()
            if tm:
                native.nc_profile_bwd_main()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # whole-step timing: nothing but the work between the two events
    # (an event after every step, for the spread of step times)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(args.steps):
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    ms_step = marks[0].elapsed_time(marks[-1]) / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    spread = {q: round(float(np.percentile(per_step, pc)), 4) for q, pc in (("p10", 10), ("median", 50), ("p90", 90))}
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step, per step {json.dumps(spread)}")

    def time_phase(fn):
        """Warmup, then args.steps repetitions of fn with an event after each:
        (mean ms per repetition, p10/median/p90 of the repetitions)."""
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record()
        for i in range(args.steps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        reps = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
        return (ev[0].elapsed_time(ev[-1]) / args.steps,
                {q: round(float(np.percentile(reps, pc)), 4) for q, pc in (("p10", 10), ("median", 50), ("p90", 90))})
    # The shader clock while the same steps run again: a one-wave probe on a
    # second stream that reads the shader-cycle and 100 MHz counters.
    side = torch.cuda.Stream()
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    side.wait_stream(torch.cuda.current_stream())
    native.nc_measure_shader_clock(max(1, min(10000, int(0.9 * ms_step * args.steps))), out=clk, stream=side)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    cyc, ticks = (int(x) for x in clk.cpu())
    sclk_mhz = cyc / ticks * 100.0 if ticks else None
    log(f"shader clock during the steps: {sclk_mhz and round(sclk_mhz)} MHz")
    # per-kernel timing in a second pass of the same steps (events between launches)
    tm = Timer(torch)
    for _ in range(args.steps):
        step(tm)
    torch.cuda.synchronize()
    tot = tm.totals()
    flops_f = attn_flops(B, T, H, D, wl.windows, "fwd")
    flops_b = attn_flops(B, T, H, D, wl.windows, "bwd")
    value = (flops_f + flops_b) / (ms_step * 1e-3) / 1e12
    # Algorithmic (band-counted) flops per visible pair of each unit: the
    # forward 4*D; the whole backward 8*D = the dV, dP, dK and dQ products,
    # of which the dK/dV kernel produces dV, dP and dK (6*D) and the dQ
    # kernel dQ (2*D), so the two kernels' shares add up to the backward's.
    # Executed flops differ: the dK/dV kernel also recomputes S (8*D), the
    # dQ kernel recomputes S and dP (6*D); those rates are reported apart.
    ALG = {"attn_fwd": 4, "attn_bwd": 8, "attn_bwd_dkdv": 6, "attn_bwd_dq": 2}
    EXE = {"attn_fwd": 4, "attn_bwd": 14, "attn_bwd_dkdv": 8, "attn_bwd_dq": 6}

    def kf(name, windows, table):  # flops of one unit over the given layers
        return attn_flops(B, T, H, D, windows, "fwd") // 4 * table[name]

    kern, per_window = {}, {}
    for label, (ms, n) in tot.items():
        if "@" in label:  # one layer type: per-launch time and its own band-counted rate
            name, tag = label.split("@")
            w = FULL if tag == "full" else int(tag)
            per_ms = ms / n
            alg = kf(name, [w], ALG) / (per_ms * 1e-3) / 1e12
            exe = kf(name, [w], EXE) / (per_ms * 1e-3) / 1e12
            per_window.setdefault(tag, {})[name] = {
                "avg_ms_per_launch": round(per_ms, 5), "tflops": round(alg, 2),
                "frac_bf16_peak": round(alg / PEAK_BF16_TFLOPS, 4), "executed_tflops": round(exe, 2),
                "executed_frac_bf16_peak": round(exe / PEAK_BF16_TFLOPS, 4)}
            continue
        per_step = ms / args.steps
        row = {"ms_per_step": round(per_step, 4), "launches_per_step": n // args.steps,
               "avg_ms_per_launch": round(ms / n, 5)}
        if label in ALG:
            row["tflops"] = round(kf(label, wl.windows, ALG) / (per_step * 1e-3) / 1e12, 2)
            row["frac_bf16_peak"] = round(row["tflops"] / PEAK_BF16_TFLOPS, 4)
            row["executed_tflops"] = round(kf(label, wl.windows, EXE) / (per_step * 1e-3) / 1e12, 2)
            row["executed_frac_bf16_peak"] = round(row["executed_tflops"] / PEAK_BF16_TFLOPS, 4)
        if label == "prologue_fwd_k":  # reads k, writes k'
            nbytes = 2 * L * (B * T * Hkv * D * 2)
            row["gbs"] = round(nbytes / (per_step * 1e-3) / 1e9, 1)
        kern[label] = row
    log("kernels:", json.dumps(kern))

    # ---------------------------------------------------------------- decode
    decode = None
    if not args.no_decode:
        dw = workloads()["decode_bf16"]
        DB, DH, DHkv, DD, Tm = dw.B, dw.H, dw.Hkv, dw.D, dw.T
        lens = synth.seqlens_np(DB, Tm, 2000)
        sl = torch.from_numpy(lens).to(dev)
        log(f"allocating decode caches: {len(dw.windows)} layers x [{DB},{Tm},{DHkv},{DD}] bf16 x2")
        dq_ = [synth.normal_device((DB, DH, DD), 2001 + 10 * l, "bf16") for l in range(len(dw.windows))]
        kc = [synth.normal_device((DB, Tm, DHkv, DD), 2002 + 10 * l, "bf16") for l in range(len(dw.windows))]
        vc = [synth.normal_device((DB, Tm, DHkv, DD), 2003 + 10 * l, "bf16") for l in range(len(dw.windows))]
        dout_ = torch.empty_like(dq_[0])
        dlse = torch.empty((DB, DH), dtype=torch.float32, device=dev)
        dws = torch.empty(native.nc_attn_decode_workspace_bytes(native.NC_BF16, DB, DH, DHkv, DD, Tm),
                          dtype=torch.uint8, device=dev)

        def dstep():
            for l, w in enumerate(dw.windows):
                native.nc_attn_decode(dq_[l], kc[l], vc[l], sl, w, dw.scale, out=dout_, lse=dlse,
                                      workspace=dws)

        dms, dms_spread = time_phase(dstep)
        nbytes = sum(decode_bytes(lens, DH, DHkv, DD, w) for w in dw.windows)
        gbs = nbytes / (dms * 1e-3) / 1e9
        decode = {"workload": "decode_bf16: 64 rows x 1 query, H=Hkv=10, D=128, cache lengths "
                              "uniform 1..2048, 20-layer SSSL step (15 x w=1024, 5 full)",
                  "ms_per_step": round(dms, 4), "ms_per_step_spread": dms_spread, "bytes_per_step": nbytes, "gbs": round(gbs, 1),
                  "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        log("decode:", json.dumps(decode))

        # decode step: the same caches and lengths with the token before the
        # last appended in place (cache_seqlens = lens - 1), prologue included
        kn_ = [synth.normal_device((DB, DHkv, DD), 2004 + 10 * l, "bf16") for l in range(len(dw.windows))]
        vn_ = [synth.normal_device((DB, DHkv, DD), 2005 + 10 * l, "bf16") for l in range(len(dw.windows))]
        csl = torch.from_numpy(lens - 1).to(dev)
        dcos, dsin = native.nc_rope_table(Tm, DD)
        sws = torch.empty(native.nc_attn_decode_step_workspace_bytes(native.NC_BF16, DB, DH, DHkv, DD, Tm),
                          dtype=torch.uint8, device=dev)

        def sstep():
            for l, w in enumerate(dw.windows):
                native.nc_attn_decode_step(dq_[l], kn_[l], vn_[l], kc[l], vc[l], csl, dcos, dsin, eps, w,
                                           dw.scale, out=dout_, lse=dlse, workspace=sws)

        sms, sms_spread = time_phase(sstep)
        sbytes = sum(decode_step_bytes(lens - 1, DH, DHkv, DD, w) for w in dw.windows)
        sgbs = sbytes / (sms * 1e-3) / 1e9
        decode["step_with_append"] = {
            "what": "nc_attn_decode_step per layer: prologue of the new token at position "
                    "cache_seqlens[b] = L_b - 1, k'/v appended in place, split-K decode over L_b keys",
            "ms_per_step": round(sms, 4), "ms_per_step_spread": sms_spread, "bytes_per_step": sbytes, "gbs": round(sgbs, 1),
            "frac_hbm_peak": round(sgbs / PEAK_HBM_GBS, 4)}
        log("decode step:", json.dumps(decode["step_with_append"]))

        # chunked prefill against the same caches: a 512-token chunk per row at
        # seeded offsets uniform on 0 .. T_max - 512 (its keys taken as already
        # appended), 20 layers with the SSSL windows
        CQ = 512
        coff = np.random.default_rng(2006).integers(0, Tm - CQ + 1, DB).astype(np.int32)
        coff_d = torch.from_numpy(coff).to(dev)
        cq_ = [synth.normal_device((DB, CQ, DH, DD), 2007 + 10 * l, "bf16") for l in range(len(dw.windows))]
        cout = torch.empty_like(cq_[0])
        clse = torch.empty((DB, DH, CQ), dtype=torch.float32, device=dev)

        def cstep():
            for l, w in enumerate(dw.windows):
                native.nc_attn_fwd_cache(cq_[l], kc[l], vc[l], coff_d, w, dw.scale, out=cout, lse=clse)

        cms, cms_spread = time_phase(cstep)
        cflops = sum(4 * DD * DH * chunk_pairs(int(n0), CQ, w) for w in dw.windows for n0 in coff)
        ctf = cflops / (cms * 1e-3) / 1e12
        decode["prefill_chunk"] = {
            "what": "nc_attn_fwd_cache per layer: 64 rows x 512-token chunk at offsets uniform 0..1536 "
                    "against the [64, 2048, 10, 128] caches, 20-layer SSSL windows",
            "ms_per_step": round(cms, 4), "ms_per_step_spread": cms_spread, "band_flops": cflops, "tflops": round(ctf, 2),
            "frac_bf16_peak": round(ctf / PEAK_BF16_TFLOPS, 4)}
        log("prefill chunk:", json.dumps(decode["prefill_chunk"]))
        del kc, vc, cq_

    # ------------------------------------------------------- fp8 forward
    fp8 = None
    if not args.no_fp8:
        # the d20 operands quantized to e4m3 with one descale per tensor
        # (outside the timed region), then the 20-layer forward
        def q8(x):
            s8 = float(x.abs().max()) / 448.0
            return (x.float() / s8).to(torch.float8_e4m3fn), s8
        f8 = [(q8(qr[l]), q8(kr[l]), q8(vv[l])) for l in range(L)]
        f8o = torch.empty_like(qr[0])
        f8l = torch.empty((B, H, T), dtype=torch.float32, device=dev)

        def fp8_step():
            for l in range(L):
                (a, sa), (b_, sb), (c, sc) = f8[l]
                native.nc_attn_fwd_fp8(a, b_, c, sa, sb, sc, wl.windows[l], scale, out=f8o, lse=f8l)

        fms, fms_spread = time_phase(fp8_step)
        fp8 = {"what": "nc_attn_fwd_fp8 per layer on the d20 operands quantized to float8 e4m3 (one descale per "
                       "tensor), 20-layer SSSL windows; bf16 out",
               "ms_per_step": round(fms, 4), "ms_per_step_spread": fms_spread, "tflops": round(flops_f / (fms * 1e-3) / 1e12, 2),
               "frac_fp8_peak": round(flops_f / (fms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
        log("fp8 forward:", json.dumps(fp8))
        del f8

    # ------------------------------------------------------------- roofline
    dom = max(("attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq"), key=lambda k: kern[k]["ms_per_step"])
    dom_flops = kf(dom, wl.windows, ALG)
    n_launch = kern[dom]["launches_per_step"]
    achieved = dom_flops / n_launch / (kern[dom]["avg_ms_per_launch"] * 1e-3) / 1e12
    tr = measured_traffic(dom)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": tr["bytes"] if tr else None,
                "traffic_split": tr,
                "sclk_mhz": round(sclk_mhz, 1) if sclk_mhz else None,
                "peak_at_sclk": round(PEAK_BF16_TFLOPS * sclk_mhz / NOMINAL_SCLK_MHZ, 1) if sclk_mhz else None,
                "frac_at_sclk": round(achieved / (PEAK_BF16_TFLOPS * sclk_mhz / NOMINAL_SCLK_MHZ), 4)
                if sclk_mhz else None,
                "flops_per_launch": dom_flops // n_launch,
                "note": "achieved = algorithmic band-counted flops per launch (per visible pair: 4*D "
                        "forward; of the backward's 8*D, 6*D for the dK/dV kernel (dV, dP, dK) and 2*D "
                        "for the dQ kernel (dQ); B*H*pairs(T,w) pairs) / average launch time, averaged "
                        "over the 20 layers"}
    fractions = {
        "attn_fwd_frac_bf16_peak": kern["attn_fwd"]["frac_bf16_peak"],
        "attn_bwd_frac_bf16_peak": kern["attn_bwd"]["frac_bf16_peak"],
        "decode_frac_hbm_peak": decode["frac_hbm_peak"] if decode else None,
        "decode_step_frac_hbm_peak": decode["step_with_append"]["frac_hbm_peak"] if decode else None,
        "targets": {"attn_fwd": 0.50, "attn_bwd": 0.35, "decode": 0.70}}

    # --------------------------------------------------------- cpu baseline
    others = None
    if not args.no_workloads:
        del qr, kr, vv, do, qp, kp, out, lse
        torch.cuda.empty_cache()
        others = other_workloads(args, np, torch, native, synth, time_phase)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, np, torch, synth, wl, cos, eps, band_pairs, FULL, decode_bytes)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_step_spread": spread, "sclk_mhz": round(sclk_mhz, 1) if sclk_mhz else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, drawn on the device)",
        "config": {"workload": "d20_bf16: B=32 T=2048 H=Hkv=10 D=128, 20 layers SSSL "
                               "(15 x window 1024, 5 full causal); step = per layer the QK prologue and attention "
                               "forward (one call: keys' prologue kernel, then the forward kernel applying the "
                               "queries' prologue as it loads them), then per layer in reverse the backward "
                               "through attention and prologue (one call)",
                   "B": B, "T": T, "H": H, "Hkv": Hkv, "D": D, "windows": wl.windows,
                   "band_flops_fwd": flops_f, "band_flops_bwd": flops_b},
        "attn_only_tflops": round((flops_f + flops_b) /
                                  ((kern["attn_fwd"]["ms_per_step"] + kern["attn_bwd"]["ms_per_step"]) * 1e-3)
                                  / 1e12, 2),
        "kernels": kern,
        "per_window": per_window,
        "decode": decode,
        "fp8_forward": fp8,
        "workloads": others,
        "fractions": fractions,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def other_workloads(args, np, torch, native, synth, time_phase):
    """The other training-side configurations at their full sizes, each timed
    as whole phases: every call's attention forward, then every call's
    backward in reverse order (d12: 12 SSSL layers; GQA: a windowed and a
    full call, dK/dV summed over each group of 4 query heads; both without
    the prologue, whose inputs the configurations give directly). Tiny
    (float32, the prologue forward and backward around each call, two
    calls) is reported as time only: it is launch-bound by design."""
    from transformer_attention_06_amd.workload import attn_flops, workloads
    res = {}
    for name in ("d12_bf16", "gqa_bf16"):
        w = workloads()[name]
        B, T, H, Hkv, D = w.B, w.T, w.H, w.Hkv, w.D
        n = len(w.windows)
        log(f"{name}: {n} calls, B={B} T={T} H={H} Hkv={Hkv} D={D}")
        seed = 3000 if name == "d12_bf16" else 4000
        q = [synth.normal_device((B, T, H, D), seed + 10 * l, "bf16") for l in range(n)]
        k = [synth.normal_device((B, T, Hkv, D), seed + 10 * l + 1, "bf16") for l in range(n)]
        v = [synth.normal_device((B, T, Hkv, D), seed + 10 * l + 2, "bf16") for l in range(n)]
        g = [synth.normal_device((B, T, H, D), seed + 10 * l + 3, "bf16") for l in range(n)]
        o = [torch.empty_like(x) for x in q]
        ls = [torch.empty((B, H, T), dtype=torch.float32, device="cuda") for _ in range(n)]
        dq, dk, dv = torch.empty_like(q[0]), torch.empty_like(k[0]), torch.empty_like(v[0])
        ws = torch.empty(native.nc_attn_bwd_workspace_bytes(native.NC_BF16, B, T, H, Hkv, D), dtype=torch.uint8,
                         device="cuda")

        def fwd():
            for l, win in enumerate(w.windows):
                native.nc_attn_fwd(q[l], k[l], v[l], win, w.scale, out=o[l], lse=ls[l])

        def bwd():
            for l in reversed(range(n)):
                native.nc_attn_bwd(q[l], k[l], v[l], o[l], ls[l], g[l], w.windows[l], w.scale, dq=dq, dk=dk, dv=dv,
                                   workspace=ws)

        fms, fsp = time_phase(fwd)
        bms, bsp = time_phase(bwd)
        ff, fb = attn_flops(B, T, H, D, w.windows, "fwd"), attn_flops(B, T, H, D, w.windows, "bwd")
        res[name] = {
            "calls": n, "windows": w.windows, "band_flops_fwd": ff, "band_flops_bwd": fb,
            "fwd_ms": round(fms, 4), "fwd_ms_spread": fsp, "bwd_ms": round(bms, 4), "bwd_ms_spread": bsp,
            "fwd_tflops": round(ff / (fms * 1e-3) / 1e12, 2), "bwd_tflops": round(fb / (bms * 1e-3) / 1e12, 2),
            "fwdbwd_tflops": round((ff + fb) / ((fms + bms) * 1e-3) / 1e12, 2),
            "fwd_frac_bf16_peak": round(ff / (fms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "bwd_frac_bf16_peak": round(fb / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(name, json.dumps(res[name]))
        del q, k, v, g, o, ls, dq, dk, dv, ws
        torch.cuda.empty_cache()
    # tiny float32 with the prologue around each call (as its configuration states)
    w = workloads()["tiny_f32"]
    B, T, H, Hkv, D = w.B, w.T, w.H, w.Hkv, w.D
    q, k, v, g = (synth.normal_torch(sh, 5000 + i, "f32", "cuda") for i, sh in
                  enumerate([(B, T, H, D), (B, T, Hkv, D), (B, T, Hkv, D), (B, T, H, D)]))
    c, sn = native.nc_rope_table(10 * T, D)
    eps = 2.0 ** -23

    def tiny():
        for win in w.windows:
            qp, kp = native.nc_qk_prologue_fwd(q, k, c, sn, eps)
            o, ls = native.nc_attn_fwd(qp, kp, v, win, w.scale)
            dqp, dkp, _ = native.nc_attn_bwd(qp, kp, v, o, ls, g, win, w.scale)
            native.nc_qk_prologue_bwd(q, k, c, sn, eps, dqp, dkp)

    tms, tsp = time_phase(tiny)
    res["tiny_f32"] = {"calls": len(w.windows), "windows": w.windows, "ms": round(tms, 4), "ms_spread": tsp,
                       "what": "prologue fwd + attention fwd + bwd + prologue bwd per call, float32 "
                               "(time only: latency-bound)"}
    log("tiny_f32", json.dumps(res["tiny_f32"]))
    return res


def cpu_baseline(args, np, torch, synth, wl, cos, eps, band_pairs, FULL, decode_bytes):
    """The fp64 oracle, as it stands, on bounded samples of the same inputs,
    with the BLAS pools at CPU_THREADS threads:
      * training: whole batch rows (all heads) of one windowed and one full
        d20 layer, prologue + attention forward + backward, alternating
        until about --cpu-seconds are spent; band-counted TFLOP/s like the
        GPU value;
      * decode: one windowed and one full layer of the decode workload (all
        64 rows, the bench's seeded lengths and caches), oracle.decode
        timed alone; GB/s over the same algorithmic bytes as the GPU's."""
    import oracle
    from transformer_attention_06_amd.workload import workloads
    try:
        from threadpoolctl import threadpool_limits, threadpool_info
        limiter = threadpool_limits(CPU_THREADS)
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        limiter, threads = None, CPU_THREADS
    layers = [wl.windows.index(1024), wl.windows.index(FULL)]
    T, H, D = wl.T, wl.H, wl.D
    pos = oracle.positions_from_offsets(1, T)
    done_flops, n_rows, elapsed = 0, 0, 0.0
    b = 0
    while elapsed < args.cpu_seconds and b < wl.B:
        for l in layers:
            w = wl.windows[l]
            # the bench's d20 inputs of layer l, batch row b (same seeds, drawn again)
            q = synth.to_f64(synth.normal_device((wl.B, T, H, D), 1000 + 10 * l, "bf16")[b:b + 1])
            k = synth.to_f64(synth.normal_device((wl.B, T, wl.Hkv, D), 1001 + 10 * l, "bf16")[b:b + 1])
            v = synth.to_f64(synth.normal_device((wl.B, T, wl.Hkv, D), 1002 + 10 * l, "bf16")[b:b + 1])
            g = synth.to_f64(synth.normal_device((wl.B, T, H, D), 1003 + 10 * l, "bf16")[b:b + 1])
            torch.cuda.empty_cache()
            t = time.perf_counter()
            q1, k1 = oracle.qk_prologue_fwd(q, k, pos, eps)
            oracle.attn_fwd(q1, k1, v, w, wl.scale)
            gq, gk, _ = oracle.attn_bwd(q1, k1, v, g, w, wl.scale)
            oracle.qk_prologue_bwd(q, k, pos, gq, gk, eps)
            elapsed += time.perf_counter() - t
            done_flops += 12 * D * H * band_pairs(T, w)
            n_rows += 1
        b += 1
        log(f"cpu baseline: {n_rows} row-layers in {elapsed:.1f} s")
    # decode: the bench's decode inputs of one windowed and one full layer
    dw = workloads()["decode_bf16"]
    lens = synth.seqlens_np(dw.B, dw.T, 2000)
    d_bytes, d_el = 0, 0.0
    for l in (dw.windows.index(1024), dw.windows.index(FULL)):
        w = dw.windows[l]
        qd = synth.to_f64(synth.normal_device((dw.B, dw.H, dw.D), 2001 + 10 * l, "bf16"))
        kc = synth.to_f64(synth.normal_device((dw.B, dw.T, dw.Hkv, dw.D), 2002 + 10 * l, "bf16"))
        vc = synth.to_f64(synth.normal_device((dw.B, dw.T, dw.Hkv, dw.D), 2003 + 10 * l, "bf16"))
        torch.cuda.empty_cache()
        reps = 0
        t = time.perf_counter()
        while reps < 3 or time.perf_counter() - t < 1.0:  # repeated for a stable rate
            oracle.decode(qd, kc, vc, lens, w, dw.scale)
            reps += 1
        d_el += time.perf_counter() - t
        d_bytes += reps * decode_bytes(lens, dw.H, dw.Hkv, dw.D, w)
        del kc, vc
    log(f"cpu baseline decode: 2 layers in {d_el:.2f} s")
    if limiter is not None:
        limiter.unregister()
    return {"value": round(done_flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "affinity_cpus": AFFINITY_CPUS,
            "kind": "oracle",
            "sample": f"{n_rows} (batch row, layer) pairs of d20 (all 10 heads, T=2048; layers with "
                      f"window 1024 and full alternating): fp64 numpy prologue + attention fwd + bwd, "
                      f"{elapsed:.1f} s",
            "decode": {"value": round(d_bytes / d_el / 1e9, 3), "unit": "GB/s",
                       "sample": f"oracle.decode on one windowed and one full layer of the decode workload "
                                 f"(64 rows, lengths uniform 1..2048), each repeated for at least 1 s "
                                 f"({d_el:.2f} s in all); rate over the GPU's algorithmic bytes of those calls "
                                 f"({d_bytes} B)"}}


if __name__ == "__main__":
    main()
