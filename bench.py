#!/usr/bin/env python3
"""Throughput of the selective-scan forward pass on one MI355X.

One step = one ssm_scan_fwd over the Mamba-2.8B-layer-shaped workload: batch 8, L = 2048,
d_inner 5120, N = 16, bf16 x / delta / z / B / C / y, float32 state and arithmetic, SiLU(z) gate and
D term on, final state returned. Inputs are synthetic (seeded; the same generator the parity tests
use) and resident in HBM before the timed region; three independent input sets rotate so the
256 MB last-level cache cannot serve them.

Prints ONE JSON line: value = algorithmic HBM GB/s of the whole step (wall clock, synchronised),
plus Gelem/s (token-channels per second), the roofline of the dominant kernel (measured with HIP
events on the stream the kernel runs on), the fp64 CPU oracle timed on the host, and secondary
figures for the long-sequence, decode and Mamba-2 (SSD) workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0                       # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0                   # dense bf16 MFMA, published
CUS, SIMDS, LANES, CLOCK = 256, 4, 16, 2.4e9
PEAK_VALU_TOPS = CUS * SIMDS * LANES * CLOCK / 1e12   # fp32 lane-ops/s without packed FP32: 39.3
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "scan_layer_8x2048x5120_bf16_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_37_amd", "csrc", f)
                  for f in ("scan.hip", "device_common.h")]

LAYER = dict(B=8, L=2048, D=5120, N=16)


def scan_bytes(B, L, D, N, es, gate=True, dskip=True, bias=False, h0=False, h_last=True):
    """Algorithmic HBM bytes of one scan: every input once, every output once; the N-wide state
    never goes to HBM (only the optional initial and final states)."""
    tok = B * L * D * es
    n = tok * (3 + (1 if gate else 0))          # x, delta, y (+ z)
    n += 2 * B * L * N * es                     # B_t, C_t
    n += D * N * 4 + (D * 4 if dskip else 0) + (D * 4 if bias else 0)
    n += (B * D * N * 4 if h0 else 0) + (B * D * N * 4 if h_last else 0)
    return n


def source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source; else None."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    kv = {}
    for line in open(PROFILE_TRAFFIC):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed(fn, steps, warmup, torch):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return wall_ms, e0.elapsed_time(e1) / steps


def per_launch_ms(fn, steps, torch):
    """Duration of each launch alone: an event pair around every launch on the current stream.
    Returns (median, min) in ms."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    d = sorted(a.elapsed_time(b) for a, b in evs)
    return d[len(d) // 2], d[0]


def copy_ceiling_gbs(torch, nbytes=1 << 30, reps=10):
    """Read+write GB/s of a plain device-to-device copy of nbytes (torch copy_), the practical
    HBM ceiling beside the published peak."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


# each secondary figure is timed after this much back-to-back work of its own (see settle)
SECONDARY_SETTLE_S = 0.3


def settle(fn, torch, seconds):
    """Launch fn back to back (batches of 64, synchronised) for the given time. The GPU raises its
    clocks only under sustained load: after several seconds idle (input generation) the first
    milliseconds of work run about 10% slower, so the timed region must not start cold."""
    i, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(64):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    return i


def smi_during(fn, torch, min_s=0.5, max_s=20.0):
    """Socket power and clocks from amd-smi, sampled while fn is launched back to back (in
    batches of 64 with a synchronisation between them) for at least min_s and until amd-smi
    has answered or max_s has passed. An "error" entry when amd-smi is not available."""
    proc = None
    try:
        # the driver's metrics lag the load: amd-smi starts after a second of sustained work
        settle(fn, torch, 1.0)
        proc = subprocess.Popen(["amd-smi", "metric", "--power", "--clock", "--json"],
                                stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
        i, t0 = 0, time.perf_counter()
        while (proc.poll() is None or time.perf_counter() - t0 < min_s) and time.perf_counter() - t0 < max_s:
            for _ in range(64):
                fn(i)
                i += 1
            torch.cuda.synchronize()
        out, _ = proc.communicate(timeout=30)
        g = json.loads(out)["gpu_data"][0]
        val = lambda d: d["value"] if isinstance(d, dict) else None
        gfx = [val(v["clk"]) for k, v in g["clock"].items() if k.startswith("gfx_") and isinstance(v, dict)]
        gfx = [c for c in gfx if c is not None]
        return {"socket_power_W": val(g["power"]["socket_power"]),
                "gfx_clk_MHz_mean": round(sum(gfx) / len(gfx), 1) if gfx else None,
                "gfx_clk_MHz_min": min(gfx) if gfx else None,
                "mem_clk_MHz": val(g["clock"].get("mem_0", {}).get("clk")),
                "launches_during_sample": i,
                "sampled": "amd-smi metric, once, while the benchmark kernel ran back to back "
                           "just before the timed region"}
    except Exception as e:  # reporting only: a missing or changed tool must not stop the bench
        torch.cuda.synchronize()
        if proc is not None and proc.poll() is None:
            proc.kill()
        settle(fn, torch, min_s)
        return {"error": type(e).__name__}


def valu_rates(torch, blocks=8192, iters=64):
    """Measured vector-ALU rates of this GPU from the probe library (probe/valu_rates.hip): lane
    FMAs/s, lane v_exp_f32/s, and lane state-steps/s of the scan's per-state-step mix (Delta a,
    2^t, (Abar - 1)/a, B x, product, h update, readout: 6 VALU + 1 exp, plus 0.25 VALU of token
    bookkeeping in the probe). 8192 workgroups of 256 threads = 8 waves per SIMD; each probe kernel
    is timed with HIP events on the stream it runs on, best of 5 after a warm launch."""
    import ctypes
    from selective_state_space_37_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    lib.probe_valu_rates.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3
    buf_in = torch.rand(16, device="cuda") + 0.5
    buf_out = torch.empty(blocks * 256, device="cuda")
    st = torch.cuda.current_stream()
    ops = blocks * 256 * iters * 16 * 8
    res = {}
    for kind, name in ((0, "fma"), (1, "exp"), (2, "mix")):
        run = lambda: lib.probe_valu_rates(kind, blocks, iters, buf_in.data_ptr(), buf_out.data_ptr(), st.cuda_stream)
        assert run() == 0
        best = None
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            run()
            e1.record(st)
            e1.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        res[name] = ops / (best * 1e-3)
    return {"fma_T_lane_per_s": round(res["fma"] / 1e12, 3), "exp_T_lane_per_s": round(res["exp"] / 1e12, 3),
            "mix_G_state_steps_per_s": round(res["mix"] / 1e9, 1),
            "mix_fma_slots_per_state_step": round(res["fma"] / res["mix"], 3)}


def device_layer_set(torch, seed, B, L, D, N):
    """An extra independent input set drawn on the device with the same distributions as the
    layer workload (timing only; parity runs use the host generator)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    bf = torch.bfloat16
    r = lambda *s: torch.randn(*s, generator=g, device="cuda", dtype=torch.float32)
    delta = torch.clamp(torch.nn.functional.softplus(r(B, L, D) - 4.0), 1e-3, 0.1).to(bf)
    return dict(x=r(B, L, D).to(bf), delta=delta, z=r(B, L, D).to(bf), Bm=r(B, L, N).to(bf),
                Cm=r(B, L, N).to(bf))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=3, help="rotating independent input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-generation", action="store_true",
                    help="leave the 48-block generation figure out of the secondary figures")
    ap.add_argument("--no-smi", action="store_true", help="skip the amd-smi clock/power sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 512 MiB device copy three times (counter calibration)")
    ap.add_argument("--valu-rates-only", action="store_true",
                    help="print only the measured vector-ALU rates (FMA, exp, the scan's mix) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU: this library has no multi-GPU path "
                         "(--gpus %d requested). Run with --gpus 1.\n" % args.gpus)
        sys.exit(2)

    import numpy as np
    import torch
    from selective_state_space_37_amd import inputs, ssm
    ssm.load()  # fails loudly without the built HIP library
    torch.cuda.set_device(0)
    if args.valu_rates_only:
        print(json.dumps({"valu_rates": valu_rates(torch)}), flush=True)
        return
    if args.copy_calibration:
        src = torch.ones(1 << 27, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    B, L, D, N = LAYER["B"], LAYER["L"], LAYER["D"], LAYER["N"]
    host = inputs.scan_layer()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16) \
        if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    A, Dskip = dev(host.A), dev(host.Dskip)
    sets = [dict(x=dev(host.x), delta=dev(host.delta), z=dev(host.z), Bm=dev(host.Bm), Cm=dev(host.Cm))]
    for s in range(1, max(1, args.sets)):
        sets.append(device_layer_set(torch, 1000 + s, B, L, D, N))
    for s in sets:
        s["y"] = torch.empty_like(s["x"])
        s["h"] = torch.empty((B, D, N), dtype=torch.float32, device="cuda")

    def step(i):
        s = sets[i % len(sets)]
        ssm.scan_fwd(s["x"], s["delta"], A, s["Bm"], s["Cm"], Dskip=Dskip, z=s["z"], y=s["y"], h_last=s["h"])

    # before the timed region: sustained load (the clock/power sample doubles as the settle
    # phase), so the W warmup steps and K timed steps run at the clocks a busy GPU holds
    if args.no_smi:
        settle(step, torch, 0.5)
        clocks = None
    else:
        clocks = smi_during(step, torch)
    wall_ms, kern_ms = timed(step, args.steps, args.warmup, torch)
    med_ms, min_ms = per_launch_ms(step, args.steps, torch)
    nbytes = scan_bytes(B, L, D, N, 2)
    elems = B * L * D
    value = nbytes / (wall_ms * 1e-3) / 1e9
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    state_steps = elems * N
    traffic = read_traffic()
    rates = valu_rates(torch)
    # ALU ceiling: the general-A recurrence needs the probe's mix once per state-step, so at the
    # measured mix rate the kernel cannot take less than floor_ms (the probe's mix carries 0.25
    # VALU per state-step of its own bookkeeping, so this floor is slightly conservative)
    floor_ms = state_steps / (rates["mix_G_state_steps_per_s"] * 1e9) * 1e3

    out = {
        "metric": "selective-scan HBM GB/s (% of peak) + Gelem/s at B=8,L=2048,D=5120,N=16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) x/z/B/C, delta = clip(softplus(N(-4,1)), 1e-3, 0.1), A[d,n] = -(n+1))",
        "config": {"workload": "selective scan, Mamba-2.8B layer shape: batch 8, L 2048, d_inner 5120, N 16",
                   "B": B, "L": L, "D": D, "N": N, "io_dtype": "bf16", "state_dtype": "f32",
                   "gate": True, "D_term": True, "final_state": True, "input_sets": len(sets)},
        "gelem_per_s": round(elems / (wall_ms * 1e-3) / 1e9, 2),
        "state_updates_per_s_G": round(elems * N / (wall_ms * 1e-3) / 1e9, 1),
        "hbm_frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "kernel_ms": round(kern_ms, 5),
        "kernel_ms_single_launch": {"median": round(med_ms, 5), "min": round(min_ms, 5),
                                    "how": "event pair around each of %d further launches" % args.steps},
        # The roofline of the metric: algorithmic HBM bytes per launch over the kernel's mean
        # launch time (HIP events on the stream it runs on) against the published 8 TB/s.
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": nbytes, "kernel_ms": round(kern_ms, 5),
                     "kernel": "scan_kernel<bf16, CH=32, NS=2, KS=8, T=16, N=16, full>"},
        # The second ceiling at N = 16: vector-ALU issue. From the measured rates of this GPU, the
        # launch's state-steps at the scan mix's rate take floor_ms; at that time the HBM
        # fraction would be hbm_frac_at_floor.
        "alu_ceiling": dict(rates, state_steps_per_launch=state_steps, floor_ms=round(floor_ms, 5),
                            hbm_frac_at_floor=round(nbytes / (floor_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                            kernel_frac_of_floor=round(floor_ms / kern_ms, 4)),
    }

    out["copy_ceiling_GB_s"] = round(copy_ceiling_gbs(torch), 1)
    if clocks is not None:
        out["gpu_clocks_power"] = clocks

    if not args.no_secondary:
        out["secondary"] = secondary(torch, np, inputs, ssm, dev, generation_figure=not args.no_generation)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(host, np, inputs)

    print(json.dumps(out), flush=True)


def secondary(torch, np, inputs, ssm, dev, generation_figure=True):
    """Long-sequence scan, scan backward, prefill with the fused convolution, decode step and SSD
    layer: kernel-time throughput (HIP events)."""
    res = {}
    g = torch.Generator(device="cuda").manual_seed(7)
    r = lambda *s: torch.randn(*s, generator=g, device="cuda", dtype=torch.float32)

    # long, narrow scan: 1 x 1,048,576 x 256, N = 16, fp32 (segmented plan)
    B, L, D, N = 1, 1 << 20, 256, 16
    x, z = r(B, L, D), r(B, L, D)
    delta = 0.5 * r(B, L, D)
    Bm, Cm = r(B, L, N), r(B, L, N)
    A = dev(inputs.structured_A(D, N))
    bias = torch.full((D,), inputs.DELTA_BIAS_SMALL, device="cuda")
    Dk = r(D)
    y = torch.empty_like(x)
    hl = torch.empty((B, D, N), device="cuda")
    nb = ssm.load().ssm_scan_fwd_workspace_bytes(B, L, D, N, ssm.SSM_F32)
    ws = ssm.workspace(nb, "cuda")
    fn = lambda i: ssm.scan_fwd(x, delta, A, Bm, Cm, delta_bias=bias, delta_softplus=True, Dskip=Dk, z=z,
                                y=y, h_last=hl, ws=ws)
    settle(fn, torch, SECONDARY_SETTLE_S)
    _, ms = timed(fn, 10, 3, torch)
    nbytes = scan_bytes(B, L, D, N, 4, bias=True)
    res["scan_long_1x1048576x256_f32"] = {"ms": round(ms, 4), "GB_s": round(nbytes / ms / 1e6, 1),
                                           "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
                                           "gelem_s": round(B * L * D / ms / 1e6, 1)}
    del x, z, delta, Bm, Cm, y

    # scan backward at the layer shape: 8 x 2048 x 5120, N 16, bf16, gate and D term
    B, L, D, N = LAYER["B"], LAYER["L"], LAYER["D"], LAYER["N"]
    bf = torch.bfloat16
    x, z, dy = r(B, L, D).to(bf), r(B, L, D).to(bf), r(B, L, D).to(bf)
    delta = torch.clamp(torch.nn.functional.softplus(r(B, L, D) - 4), 1e-3, 0.1).to(bf)
    Bm, Cm = r(B, L, N).to(bf), r(B, L, N).to(bf)
    A = dev(inputs.structured_A(D, N))
    Dk = r(D)
    nb = ssm.load().ssm_scan_bwd_workspace_bytes(B, L, D, N, ssm.SSM_BF16)
    ws = ssm.workspace(nb, "cuda")
    fn = lambda i: ssm.scan_bwd(x, delta, A, Bm, Cm, dy, Dskip=Dk, z=z, ws=ws)
    settle(fn, torch, SECONDARY_SETTLE_S)
    _, ms = timed(fn, 10, 3, torch)
    # essential I/O: x, delta, z, dy, B, C in; dx, ddelta, dz (bf16), dB, dC (fp32) out
    nbytes = 7 * B * L * D * 2 + 2 * B * L * N * 2 + 2 * B * L * N * 4 + 2 * D * N * 4 + 2 * D * 4
    steps = B * L * D * N
    # VALU model: checkpoint pass 5 single-rate + 1 half-rate exp (7 slots), main pass forward
    # recompute 6 + exp (8 slots) and reverse walk 14 single-rate ops: 29 slots per state-step
    res["scan_bwd_8x2048x5120_n16_bf16"] = {
        "ms": round(ms, 4), "GB_s_essential_io": round(nbytes / ms / 1e6, 1),
        "gelem_s": round(B * L * D / ms / 1e6, 1),
        "valu_slot_frac": round(steps * 29 / (ms * 1e-3) / (PEAK_VALU_TOPS * 1e12), 4),
        "workspace_MB": round(nb / 1e6, 1)}
    del x, z, dy, delta, Bm, Cm, ws

    # prefill with the fused width-4 causal convolution: batch 128, 2048 prompt tokens, d_inner 4096,
    # N 16, bf16 (the generation workload's prompt), register returned for the decode steps
    B, L, D, N, W = 128, 2048, 4096, 16, 4
    x, z = r(B, L, D).to(bf), r(B, L, D).to(bf)
    delta = torch.clamp(torch.nn.functional.softplus(r(B, L, D) - 4), 1e-3, 0.1).to(bf)
    Bm, Cm = r(B, L, N).to(bf), r(B, L, N).to(bf)
    A = dev(inputs.structured_A(D, N))
    Dk, cw = r(D), r(D, W) * 0.5
    reg = torch.zeros(B, D, W, dtype=bf, device="cuda")
    y = torch.empty_like(x)
    hl = torch.empty((B, D, N), device="cuda")
    fn = lambda i: ssm.scan_fwd_conv(x, delta, A, Bm, Cm, cw, conv_state=reg, Dskip=Dk, z=z, y=y, h_last=hl)
    settle(fn, torch, SECONDARY_SETTLE_S)
    _, ms = timed(fn, 5, 3, torch)
    nbytes = scan_bytes(B, L, D, N, 2) + D * W * 4 + 2 * B * D * W * 2
    res["prefill_conv_128x2048x4096_n16_bf16"] = {
        "ms": round(ms, 4), "GB_s": round(nbytes / ms / 1e6, 1),
        "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4), "gelem_s": round(B * L * D / ms / 1e6, 1)}
    del x, z, delta, Bm, Cm, y, reg

    # decode: batch 128, d_inner 4096, N 16, bf16 I/O, conv width 4; 16 layers' states rotate
    B, D, N, W, layers = 128, 4096, 16, 4, 16
    bf = torch.bfloat16
    A = dev(inputs.structured_A(D, N))
    hs = [r(B, D, N) * 0.1 for _ in range(layers)]
    cs = [r(B, D, W).to(bf) for _ in range(layers)]
    cw, Dk = r(D, W) * 0.5, r(D)
    xs = [r(B, D).to(bf) for _ in range(layers)]
    ds = [torch.clamp(torch.nn.functional.softplus(r(B, D) - 4), 1e-3, 0.1).to(bf) for _ in range(layers)]
    zs = [r(B, D).to(bf) for _ in range(layers)]
    Bs = [r(B, N).to(bf) for _ in range(layers)]
    Cs = [r(B, N).to(bf) for _ in range(layers)]
    ys = [torch.empty(B, D, dtype=bf, device="cuda") for _ in range(layers)]

    def dec(i):
        k = i % layers
        ssm.state_update(xs[k], ds[k], A, Bs[k], Cs[k], hs[k], Dskip=Dk, z=zs[k], conv_state=cs[k], conv_w=cw,
                         y=ys[k])

    # one graph holds 16 layer steps, so Python launch overhead is not measured
    for i in range(layers):
        dec(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(layers):
            dec(i)
    settle(lambda i: graph.replay(), torch, SECONDARY_SETTLE_S)
    _, ms = timed(lambda i: graph.replay(), 20, 3, torch)
    per_step = ms / layers
    nbytes = B * D * (2 * N * 4 + 2 * W * 2 + 4 * 2) + D * N * 4 + D * W * 4 + D * 4 + 2 * B * N * 2
    res["decode_128x4096_n16_bf16_16_layers"] = {
        "us_per_step": round(per_step * 1e3, 3), "GB_s": round(nbytes / per_step / 1e6, 1),
        "hbm_frac": round(nbytes / per_step / 1e6 / PEAK_HBM_GBS, 4),
        "tokens_per_s_per_layer": round(B / (per_step * 1e-3), 1)}
    # the same steps on one layer's state only (about 42 MB: it stays in the 256 MB last-level
    # cache, so this is a cache figure, not an HBM one)
    graph1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph1):
        for i in range(layers):
            dec(0)
    settle(lambda i: graph1.replay(), torch, SECONDARY_SETTLE_S)
    _, ms1 = timed(lambda i: graph1.replay(), 20, 3, torch)
    per1 = ms1 / layers
    res["decode_128x4096_n16_bf16_single_layer_cache_resident"] = {
        "us_per_step": round(per1 * 1e3, 3), "GB_s": round(nbytes / per1 / 1e6, 1),
        "note": "one layer's state reused every step: served from the last-level cache, not HBM"}
    del hs, cs, xs, ds, zs, Bs, Cs, ys, graph, graph1

    # Mamba-2 SSD: batch 2, L 8192, 80 heads x 64, N 128, chunk 256, bf16
    B, L, H, P, N, Q = 2, 8192, 80, 64, 128, 256
    x = r(B, L, H, P).to(bf)
    delta = torch.clamp(torch.nn.functional.softplus(r(B, L, H) - 4), 1e-3, 0.1).to(bf)
    Bm, Cm = r(B, L, N).to(bf), r(B, L, N).to(bf)
    Ah = -(1.0 + 15.0 * torch.rand(H, generator=g, device="cuda"))
    y = torch.empty_like(x)
    nb = ssm.load().ssd_chunk_fwd_workspace_bytes(B, L, H, P, N, Q, ssm.SSM_BF16)
    ws = ssm.workspace(nb, "cuda")
    fn = lambda i: ssm.ssd_chunk_fwd(x, delta, Ah, Bm, Cm, chunk=Q, y=y, ws=ws)
    settle(fn, torch, SECONDARY_SETTLE_S)
    _, ms = timed(fn, 10, 3, torch)
    nbytes = 2 * B * L * H * P * 2 + B * L * H * 2 + 2 * B * L * N * 2 + H * 4 + B * H * P * N * 4
    nch = L // Q
    flops = B * nch * H * (2 * Q * Q * P + 2 * Q * P * N * 2) + B * nch * 2 * Q * Q * N
    res["ssd_2x8192x80x64_n128_q256_bf16"] = {
        "ms": round(ms, 4), "GB_s": round(nbytes / ms / 1e6, 1), "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
        "TFLOP_s": round(flops / ms / 1e9, 1), "mfma_frac": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}

    # its gradients (dx, ddelta, dA, dB, dC, dh0 for dy; no gate, no D, as the forward figure)
    dy = r(B, L, H, P).to(bf)
    nbw = ssm.load().ssd_chunk_bwd_workspace_bytes(B, L, H, P, N, 1, ssm.SSM_BF16)
    wsb = ssm.workspace(nbw, "cuda")
    Bg, Cg = Bm.unsqueeze(2), Cm.unsqueeze(2)
    fnb = lambda i: ssm.ssd_chunk_bwd(x, delta, Ah, Bg, Cg, dy, ws=wsb)
    settle(fnb, torch, SECONDARY_SETTLE_S)
    _, msb = timed(fnb, 10, 3, torch)
    # essential I/O: x, dy, dx; delta, ddelta (bf16); B, C (bf16) and dB, dC (float32); dh0
    nbytes_b = 3 * B * L * H * P * 2 + 2 * B * L * H * 2 + 2 * B * L * N * 2 + 2 * B * L * N * 4 + B * H * P * N * 4
    Qb = 64
    nchb = L // Qb
    # per chunk and head: U (Q^2 P), the within-chunk dB, dC (2 Q^2 N) and w (Q^2 P), the carried
    # terms of dB, dC, y and w (4 Q P N), the two state passes (2 Q P N); G once per chunk
    flops_b = B * nchb * H * 2 * (2 * Qb * Qb * P + 2 * Qb * Qb * N + 6 * Qb * P * N) + B * nchb * 2 * Qb * Qb * N
    res["ssd_bwd_2x8192x80x64_n128_bf16"] = {
        "ms": round(msb, 4), "GB_s_essential_io": round(nbytes_b / msb / 1e6, 1),
        "hbm_frac": round(nbytes_b / msb / 1e6 / PEAK_HBM_GBS, 4),
        "TFLOP_s": round(flops_b / msb / 1e9, 1), "mfma_frac": round(flops_b / msb / 1e9 / PEAK_BF16_TFLOPS, 4),
        "workspace_MB": round(nbw / 1e6, 1)}
    del dy, wsb

    if generation_figure:
        res["generation_mamba_1.4b_b128"] = generation(torch, ssm, g)
    return res


def generation(torch, ssm, g):
    """Decode steps of a Mamba-1.4B-shaped model at batch 128 (the pages' generation setting):
    48 blocks (d_model 2048, d_inner 4096, N 16, conv 4, rank 128) with synthetic weights drawn on
    the device, then the final LayerNorm and the LM head (vocabulary 50280, padded to 50288).
    One step = one token for each of the 128 sequences through the whole stack, captured in one
    HIP graph. Sampling and the embedding lookup are not timed."""
    layers, Bsz, Dm, Di, N, W, R, V = 48, 128, 2048, 4096, 16, 4, 128, 50288
    bf, f32, dev = torch.bfloat16, torch.float32, "cuda"
    nrm = lambda *shape, fan: (torch.randn(*shape, generator=g, device=dev) / fan ** 0.5).to(bf)
    blocks = []
    for _ in range(layers):
        step = torch.exp(torch.empty(Di, device=dev).uniform_(-6.9, -2.3, generator=g))
        blocks.append(dict(
            ln_w=torch.ones(Dm, device=dev), ln_b=torch.zeros(Dm, device=dev),
            W_in=nrm(2 * Di, Dm, fan=Dm),
            conv_w=torch.randn(Di, W, generator=g, device=dev) / 2, conv_b=torch.zeros(Di, device=dev),
            W_xp=nrm(R + 2 * N, Di, fan=Di),
            W_dt=(nrm(Di, R, fan=R).float() * 0.1).to(bf), b_dt=torch.log(torch.expm1(step)),
            A=-torch.arange(1, N + 1, device=dev, dtype=f32).repeat(Di, 1).contiguous(), D=torch.ones(Di, device=dev),
            W_out=nrm(Dm, Di, fan=Di)))
    regs = [torch.randn(Bsz, Di, W, generator=g, device=dev).to(bf) for _ in range(layers)]
    hs = [torch.zeros(Bsz, Di, N, device=dev, dtype=f32) for _ in range(layers)]
    ln_w, ln_b = torch.ones(Dm, device=dev), torch.zeros(Dm, device=dev)
    W_lm = nrm(V, Dm, fan=Dm)
    hidden = torch.randn(Bsz, Dm, generator=g, device=dev).to(bf)
    hn = torch.empty_like(hidden)
    logits = torch.empty(Bsz, V, device=dev, dtype=bf)
    lib = ssm.load()
    ws = ssm.workspace(max(lib.ssm_block_step_workspace_bytes(Bsz, Dm, Di, N, W, R),
                           lib.ssm_linear_workspace_bytes(Bsz, Dm, V), 16), dev)

    def one_step():
        for l in range(layers):
            ssm.block_step(hidden, regs[l], hs[l], blocks[l], ws=ws)
        ssm.layernorm(hidden, ln_w, ln_b, y=hn)
        ssm.linear(hn, W_lm, y=logits, ws=ws)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        one_step()   # warm (and load) before capture
    torch.cuda.current_stream().wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_step()
    settle(lambda i: graph.replay(), torch, SECONDARY_SETTLE_S)
    _, ms = timed(lambda i: graph.replay(), 20, 3, torch)
    # HBM bytes per step: every weight once; the SSM state (float32) and the conv register (bf16)
    # of every layer read and written; activations are small and mostly cache-resident
    wbytes = layers * (2 * Di * Dm + R * Di + 2 * N * Di + Di * R + Dm * Di) * 2 + V * Dm * 2
    sbytes = layers * Bsz * Di * (N * 4 + W * 2) * 2
    gbs = (wbytes + sbytes) / ms / 1e6
    del blocks, regs, hs, W_lm, graph
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(Bsz / (ms * 1e-3), 1),
            "GB_s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "bytes_per_step": {"weights": wbytes, "states": sbytes},
            "model": "48 blocks d_model 2048 d_inner 4096 N 16 conv 4 rank 128, vocab 50288, batch 128, bf16 weights"}


def cpu_baseline(host, np, inputs):
    """The fp64 oracle (as it stands) on the host cores, over the same layer workload."""
    import oracle
    w = lambda a: inputs.widen(a, "bf16")
    x, d, z, Bm, Cm = w(host.x), w(host.delta), w(host.z), w(host.Bm), w(host.Cm)
    B, L, D = x.shape
    N = host.A.shape[1]
    t0 = time.perf_counter()
    oracle.scan(x, d, host.A, Bm, Cm, Dskip=host.Dskip, z=z)
    dt = time.perf_counter() - t0
    nbytes = scan_bytes(B, L, D, N, 2)
    threads = oracle.num_threads()
    # one core on a slice of the same workload (one sequence, 256 channels)
    oracle.set_num_threads(1)
    sl = (slice(0, 1), slice(None), slice(0, 256))
    t1 = time.perf_counter()
    oracle.scan(x[sl], d[sl], host.A[:256], Bm[:1], Cm[:1], Dskip=host.Dskip[:256], z=z[sl])
    dt1 = time.perf_counter() - t1
    oracle.set_num_threads(threads)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3), "gelem_per_s": round(B * L * D / dt / 1e9, 5),
            "sample": "the whole layer workload (8 x 2048 x 5120, N 16): fp64 recurrence, OpenMP over (b, d)",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model,
            "one_core_gelem_per_s": round(L * 256 / dt1 / 1e9, 6),
            "one_core_sample": "1 x 2048 x 256 channels of the same inputs, one thread"}


if __name__ == "__main__":
    main()
