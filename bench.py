#!/usr/bin/env python3
"""Benchmark of the guarded W8A8 linear on one MI355X.

Workload (one step): the video FFN pair, all through the INT8 path —
    X [24576 x 4096] bf16 --quantise--> qX, sX
    U = W8A8(qX, W1 [16384 x 4096]) + b1                   bf16 [24576 x 16384]
    U --GELU-tanh + quantise (fused)--> qH, sH            (H = GELU(U) never stored)
    Y = W8A8(qH, W2 [4096 x 16384]) + b2                   bf16 [24576 x 4096]
The weights are quantised once before timing (static, per output channel).
Inputs are seeded synthetic tensors of the workload's shapes and value
distributions, resident in HBM before the timed region.

Prints ONE JSON line on stdout.  `value` is whole-step throughput in INT8
tera-ops per second: 2 * (2*M*N*K) ops of the two GEMMs divided by the step
time (quantisation and GELU included in the time).  `roofline` describes the
dominant kernel (the INT8 GEMM), timed with HIP events around its launches on
the stream it runs on.  `cpu_baseline` is the CPU oracle on a bounded row
sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_i8_video_ffn.json")
GEMM_SOURCE = os.path.join(ROOT, "int8_w8a8_gemm_amd", "csrc", "gemm_tiled.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--M", type=int, default=24576)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="rows of the oracle sample (0: sized to ~15 s)")
    p.add_argument("--no-extra", action="store_true", help="skip the secondary kernel benches")
    p.add_argument("--probe-traffic", action="store_true",
                   help="run a known-size copy and the step's kernels a few times, for "
                        "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs, then exit")
    p.add_argument("--probe-hbm", action="store_true",
                   help="run the HBM-bound kernels on their workloads (for rocprofv3)")
    p.add_argument("--probe-small", action="store_true",
                   help="run the small MFMA-bound kernels (audio 2048^3 and text-projection INT8 "
                        "GEMMs, both BF16 fallbacks) on their workloads (for rocprofv3)")
    p.add_argument("--power-clock", action="store_true",
                   help="sample the GPU's gfx clock and socket power (amdsmi) while each main "
                        "kernel runs back to back; print JSON, exit")
    p.add_argument("--hbm-from", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                   help="achieved HBM rate per kernel from rocprofv3 runs of --probe-hbm")
    p.add_argument("--small-from", nargs=2, metavar=("TRACE_DIR", "PMC_DIR"),
                   help="per-kernel duration and MFMA counters from rocprofv3 runs of --probe-small")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn the two rocprofv3 counter outputs of --probe-traffic into "
                        + TRAFFIC_FILE + " and exit (no GPU needed)")
    return p.parse_args()


def source_hash(path):
    """Hash of the kernel source without its comments and blank lines: the stored
    counters stay valid across comment edits and lapse with any change of code."""
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def stored_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != source_hash(GEMM_SOURCE):
        return None
    return t


COPY_BYTES = 1 << 30  # the calibration copy reads and writes 1 GiB
HBM_PROBE_WARM, HBM_PROBE_REPS = 20, 30  # launches per kernel in --probe-hbm
SMALL_PROBE_WARM, SMALL_PROBE_REPS = 20, 10  # ... and in --probe-small


def traffic_from(fetch_dir, write_dir):
    """Per-launch HBM bytes of the GEMM from two rocprofv3 --pmc runs of
    --probe-traffic, each counter scaled by what it reads for a plain copy of
    known size (COPY_BYTES read, COPY_BYTES written)."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
                vals[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: sum(v.values()) / len(v) for k, v in vals.items()}

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy_f = [v for k, v in fetch.items() if "neg_kernel" in k or "neg" in k]
    copy_w = [v for k, v in write.items() if "neg_kernel" in k or "neg" in k]
    # the INT8 tiled GEMM's launches (the video FFN shapes run 256 x 256 tiles)
    def is_gemm(k):
        return "gemm_tiled" in k and "ElemI8" in k
    gemm_f = [v for k, v in fetch.items() if is_gemm(k)]
    gemm_w = [v for k, v in write.items() if is_gemm(k)]
    assert copy_f and copy_w and gemm_f and gemm_w, "counter runs lack the copy or the GEMM"
    kf = COPY_BYTES / (copy_f[0] * 1024.0)   # true bytes per counted byte
    kw = COPY_BYTES / (copy_w[0] * 1024.0)
    rd = gemm_f[0] * 1024.0 * kf
    wr = gemm_w[0] * 1024.0 * kw
    out = {"kernel": "gemm_tiled<Cfg<256,256,...,16>, ElemI8> (video FFN up and down launches, averaged)",
           "kernel_source_sha256_16": source_hash(GEMM_SOURCE),
           "copy_scale_fetch": kf, "copy_scale_write": kw,
           "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
           "hbm_bytes_per_launch": rd + wr,
           "command": "rocprofv3 --pmc FETCH_SIZE -d <FETCH_DIR> -f csv -- python3 bench.py "
                      "--probe-traffic ; rocprofv3 --pmc WRITE_SIZE -d <WRITE_DIR> -f csv -- "
                      "python3 bench.py --probe-traffic ; python3 bench.py --traffic-from "
                      "<FETCH_DIR> <WRITE_DIR>"}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))



def probe_hbm():
    """The HBM-bound kernels, each WARM + REPS times back to back on its workload
    (--hbm-from takes the median of each kernel's last REPS launches, at settled clocks
    and with its buffers' translations cached), for rocprofv3 (kernel trace,
    FETCH_SIZE, WRITE_SIZE): the row quantiser on 4 rotating X [24576 x 4096] (then the
    norm + modulation, fused with the quantiser and alone, on the same inputs), GELU +
    quantise of U [24576 x 16384], the per-block Q / K quantiser (24576 tokens x 32 heads
    x 128; blocks of 128 and 64), compaction and compaction + quantise of the text rows
    [8 x 512 x 4096]; first a 1 GiB calibration copy."""
    import numpy as np
    import torch

    import int8_w8a8_gemm_amd as w8
    import workloads as wl

    dev = torch.device("cuda:0")
    REPS = HBM_PROBE_WARM + HBM_PROBE_REPS
    src = torch.zeros((COPY_BYTES // 2,), dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    del src, dst
    gen = torch.Generator(device=dev).manual_seed(0)
    M, K = 24576, 4096
    xs = [torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16) for _ in range(4)]
    qs = [torch.empty((M, K), dtype=torch.int8, device=dev) for _ in range(4)]
    ss = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(4)]
    for i in range(REPS):
        w8.quantize_rows(xs[i % 4], qs[i % 4], ss[i % 4])
    for blk in (128, 64):
        sb = torch.empty((1, -(-M // blk), 32), dtype=torch.float32, device=dev)
        for i in range(REPS):
            w8.quantize_blocks(xs[i % 4], 1, 32, blk, q=qs[i % 4], scale=sb)
    mods = [(torch.randn((8, K), device=dev, generator=gen) * 0.3).to(torch.bfloat16)
            for _ in range(2)]
    for i in range(REPS):
        w8.norm_mod_quantize_rows(xs[i % 4], mods[0], mods[1], M // 8, q=qs[i % 4],
                                  qscale=ss[i % 4])
    y = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    for i in range(REPS):
        w8.norm_mod_bf16(xs[i % 4], mods[0], mods[1], M // 8, y=y)
    del xs, qs, ss, y
    u = (torch.randn((M, 16384), device=dev, generator=gen) * 0.64).to(torch.bfloat16)
    qh = torch.empty((M, 16384), dtype=torch.int8, device=dev)
    sh = torch.empty((M,), dtype=torch.float32, device=dev)
    for _ in range(REPS):
        w8.gelu_quantize_rows(u, qh, sh)
    del u, qh, sh
    g = wl.guarded_mixed()
    B, L, Dm = g.x.shape
    xd = torch.from_numpy(np.ascontiguousarray(g.x.reshape(B * L, Dm)).view(np.int16)).to(dev)
    xd = xd.view(torch.bfloat16).view(B, L, Dm)
    md = torch.from_numpy(g.mask).to(dev)
    buf = torch.empty((B * L, Dm), dtype=torch.bfloat16, device=dev)
    qb = torch.empty((B * L, Dm), dtype=torch.int8, device=dev)
    sb = torch.empty((B * L,), dtype=torch.float32, device=dev)
    src_row = torch.empty((B * L,), dtype=torch.int32, device=dev)
    cnt = torch.empty((1,), dtype=torch.int32, device=dev)
    for _ in range(REPS):
        w8.compact_padded_rows(xd, md, buf, src_row, cnt)
    for _ in range(REPS):
        w8.compact_quantize_rows(xd, md, qb, sb, src_row, cnt)
    torch.cuda.synchronize()
    log(f"hbm probe done (text rows kept: {int(cnt.item())})")


def _small_workloads(torch, w8, wl, np, dev):
    """Operands of the small MFMA-bound kernels, as the bench's extras build them:
    the audio GEMM 2048^3 on quantised N(0,1) activations and N(0, 0.02^2)
    weights, the text projection on the fused compaction + quantisation's codes
    of the text rows [8 x 512 x 4096], both BF16 fallbacks, and a 256-row
    sequence through the FFN down projection, plain and split-K."""
    gen = torch.Generator(device=dev).manual_seed(0)
    out = {}
    xa = torch.randn((2048, 2048), device=dev, generator=gen).to(torch.bfloat16)
    wa = (torch.randn((2048, 2048), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    qa, sa = w8.quantize_rows(xa)
    qw, sw = w8.quantize_rows(wa)
    ba = (torch.randn((2048,), device=dev, generator=gen) * 0.01).to(torch.bfloat16)
    ya = torch.empty((2048, 2048), dtype=torch.bfloat16, device=dev)
    out["gemm_audio_2048^3"] = (lambda: w8.gemm(qa, sa, qw, sw, ba, out=ya), 2.0 * 2048 ** 3, "int8")
    g = wl.guarded_mixed()
    B, L, Dm = g.x.shape

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    xd = d(g.x.reshape(B * L, Dm)).view(B, L, Dm)
    md = torch.from_numpy(g.mask).to(dev)
    qb, sb, src, cnt = w8.compact_quantize_rows(xd, md)
    mc = int(cnt.item())
    lw = w8.W8A8Linear.prepare(d(g.w), d(g.b))
    yc = torch.empty((mc, 4096), dtype=torch.bfloat16, device=dev)
    out["gemm_int8_text_Mc_x4096x4096"] = (
        lambda: w8.gemm(qb[:mc], sb[:mc], lw.qw, lw.sw, lw.bias, out=yc), 2.0 * mc * 4096 * 4096, "int8")
    buf, _, _ = w8.compact_padded_rows(xd, md)
    xc = buf[:mc]
    wfa, bfa = d(g.w_a), d(g.b_a)
    yfa = torch.empty((mc, 4100), dtype=torch.bfloat16, device=dev)
    out["fallback_bf16_N4100"] = (lambda: w8.linear_bf16(xc, wfa, bfa, y=yfa),
                                  2.0 * mc * 4100 * 4096, "bf16")
    xb, wfb, bfb = d(g.x_b), d(g.w_b), d(g.b_b)
    yfb = torch.empty((2048, 2048), dtype=torch.bfloat16, device=dev)
    out["fallback_bf16_K2050"] = (lambda: w8.linear_bf16(xb, wfb, bfb, y=yfb),
                                  2.0 * 2048 * 2048 * 2050, "bf16")
    # a short sequence through the FFN down projection, plain and split-K
    Ms, Ns, Ks = 256, 4096, 16384
    qs, ss = w8.quantize_rows(torch.randn((Ms, Ks), device=dev, generator=gen).to(torch.bfloat16))
    qws, sws = w8.quantize_rows((torch.randn((Ns, Ks), device=dev, generator=gen) * 0.02)
                                .to(torch.bfloat16))
    bs = (torch.randn((Ns,), device=dev, generator=gen) * 0.01).to(torch.bfloat16)
    ys = torch.empty((Ms, Ns), dtype=torch.bfloat16, device=dev)
    wss = torch.empty((w8.gemm_splitk_workspace_bytes(Ms, Ns, Ks),), dtype=torch.uint8, device=dev)
    out["gemm_256x4096x16384"] = (lambda: w8.gemm(qs, ss, qws, sws, bs, out=ys),
                                  2.0 * Ms * Ns * Ks, "int8")
    out["gemm_splitk_256x4096x16384"] = (
        lambda: w8.gemm_splitk(qs, ss, qws, sws, bs, out=ys, workspace=wss), 2.0 * Ms * Ns * Ks,
        "int8")
    return out, mc


def probe_small():
    """The small MFMA-bound kernels, each SMALL_PROBE_WARM + SMALL_PROBE_REPS times back
    to back on its workload, for rocprofv3 (kernel trace and counters; a summary takes
    each kernel's last SMALL_PROBE_REPS launches)."""
    import numpy as np
    import torch

    import int8_w8a8_gemm_amd as w8
    import workloads as wl

    dev = torch.device("cuda:0")
    work, mc = _small_workloads(torch, w8, wl, np, dev)
    for name, (fn, _, _) in work.items():
        for _ in range(SMALL_PROBE_WARM + SMALL_PROBE_REPS):
            fn()
        torch.cuda.synchronize()
        log(f"probe-small: {name} done")
    log(f"probe-small done (text rows kept: {mc})")


def power_clock():
    """Shader clock and package power while each main kernel runs back to back for
    4 s (small kernels 3 s).  A thread reads amdsmi's GPU metrics table every ~2 ms
    and keeps each new table (the firmware refreshes it a few times a second): gfx
    clock of every XCD, the energy accumulator, and the accumulated time the package
    power tracking (PPT) limit held the clock down.  Power = energy between the
    first and the last new table inside the busy window over the host time between
    them.  Reported per kernel: mean clock, power from the energy
    accumulator over the window, the share of the window spent PPT-limited, and
    the rate as a fraction of the peak at the measured clock."""
    import threading

    import amdsmi
    import numpy as np
    import torch

    import int8_w8a8_gemm_amd as w8
    import workloads as wl

    amdsmi.amdsmi_init()
    handle = amdsmi.amdsmi_get_processor_handles()[0]
    dev = torch.device("cuda:0")
    info = {}
    try:
        cap = amdsmi.amdsmi_get_power_cap_info(handle)
        info["power_cap_W"] = float(cap.get("power_cap", 0)) / 1e6
    except Exception as e:  # pragma: no cover - depends on the driver
        info["power_cap_error"] = repr(e)
    try:
        e = amdsmi.amdsmi_get_energy_count(handle)
        info["energy_counter_resolution_uJ"] = float(e.get("counter_resolution", 0.0))
    except Exception as e:  # pragma: no cover
        info["energy_error"] = repr(e)
    res_uj = info.get("energy_counter_resolution_uJ") or 15.3

    def num(v):
        return float(v) if isinstance(v, (int, float)) else None

    def snapshot():
        m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
        return {"ts": num(m.get("system_clock_counter")), "energy": num(m.get("energy_accumulator")),
                "ppt": num(m.get("ppt_residency_acc")), "acc": num(m.get("accumulation_counter")),
                "clk": float(np.mean(clks)) if clks else num(m.get("current_gfxclk")),
                "power": num(m.get("current_socket_power"))}

    def run(fn, seconds=4.0):
        snaps = []
        stop = threading.Event()

        def sampler():
            last = None
            while not stop.is_set():
                try:
                    sn = snapshot()
                    if sn["ts"] != last:
                        sn["host"] = time.perf_counter()
                        snaps.append(sn)
                        last = sn["ts"]
                except Exception:
                    pass
                time.sleep(0.002)

        for _ in range(10):   # settle the clocks on this kernel first
            fn()
        torch.cuda.synchronize()
        th = threading.Thread(target=sampler)
        th.start()
        time.sleep(0.05)
        t0 = time.perf_counter()
        n = 0
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                fn()
                n += 1
            torch.cuda.synchronize()
        e_ev.record()
        e_ev.synchronize()
        stop.set()
        th.join()
        out = {"calls": n, "ms_per_call": s_ev.elapsed_time(e_ev) / n, "tables": len(snaps)}
        inner = snaps[1:-1] if len(snaps) > 3 else snaps   # tables inside the busy window
        clk = [x["clk"] for x in inner if x["clk"]]
        if clk:
            out["gfxclk_MHz_mean"] = round(float(np.mean(clk)), 1)
            out["gfxclk_MHz_min_max"] = [min(clk), max(clk)]
        pw = [x["power"] for x in inner if x["power"]]
        if pw:
            out["socket_power_W_mean"] = round(float(np.mean(pw)), 1)
        a, b = (inner[0], inner[-1]) if len(inner) >= 2 else (None, None)
        if a and b and a["ts"] and b["ts"] and b["ts"] > a["ts"]:
            dt = b["host"] - a["host"]          # between the first and last new tables
            out["table_period_s"] = round(dt / (len(inner) - 1), 3)
            out["firmware_ticks_per_s"] = round((b["ts"] - a["ts"]) / dt, -6)
            if a["energy"] is not None and b["energy"] is not None:
                out["energy_power_W"] = round((b["energy"] - a["energy"]) * res_uj * 1e-6 / dt, 1)
            if a["ppt"] is not None and a["acc"] and b["acc"] > a["acc"]:
                out["ppt_limited_frac"] = round((b["ppt"] - a["ppt"]) / (b["acc"] - a["acc"]), 3)
            out["window_s"] = round(dt, 3)
        return out

    res = {}
    M, D, F = 24576, 4096, 16384
    ffn = wl.video_ffn(M=M)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x = d(ffn.x)
    qw1, sw1 = w8.quantize_rows(d(ffn.w1))
    qw2, sw2 = w8.quantize_rows(d(ffn.w2))
    b1, b2 = d(ffn.b1), d(ffn.b2)
    qx, sx = w8.quantize_rows(x)
    u = w8.gemm(qx, sx, qw1, sw1, b1)
    qh, sh = w8.gelu_quantize_rows(u)
    y = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    gen = torch.Generator(device=dev).manual_seed(0)
    shm, scm = [(torch.randn((8, D), device=dev, generator=gen) * 0.3).to(torch.bfloat16)
                for _ in range(2)]
    ops = 2.0 * M * F * D
    for name, fn, work, unit in (
            ("gemm_up", lambda: w8.gemm(qx, sx, qw1, sw1, b1, out=u), ops, "int8"),
            ("gemm_down", lambda: w8.gemm(qh, sh, qw2, sw2, b2, out=y), ops, "int8"),
            ("quantize_x", lambda: w8.quantize_rows(x, qx, sx), 3.0 * M * D + 4 * M, "bytes"),
            ("gelu_quantize_u", lambda: w8.gelu_quantize_rows(u, qh, sh), 3.0 * M * F + 4 * M, "bytes"),
            ("norm_mod_quantize_x", lambda: w8.norm_mod_quantize_rows(x, shm, scm, M // 8, q=qx, qscale=sx),
             3.0 * M * D + 4 * M, "bytes"),
            ("norm_mod_bf16_x", lambda: w8.norm_mod_bf16(x, shm, scm, M // 8, y=y), 4.0 * M * D, "bytes")):
        r = run(fn)
        t = r["ms_per_call"] * 1e-3
        if unit == "int8":
            r["TOPS"] = round(work / t / 1e12, 1)
            r["frac_of_5000"] = round(work / t / 1e12 / PEAK_INT8_TOPS, 4)
            if r.get("gfxclk_MHz_mean"):
                # the same rate against the peak at the clock the kernel ran at: the
                # share of the matrix cores' cycles spent on MFMAs
                r["frac_of_peak_at_measured_clock"] = round(
                    r["frac_of_5000"] * 2400.0 / r["gfxclk_MHz_mean"], 4)
            if r.get("energy_power_W"):
                r["nJ_per_MFMA_32x32x32"] = round(r["energy_power_W"] / (work / t / 65536.0) * 1e9, 2)
        else:
            r["TB/s"] = round(work / t / 1e12, 3)
        res[name] = r
        log(f"{name}: {json.dumps(r)}")
    del u, qh, y
    small, _ = _small_workloads(torch, w8, wl, np, dev)
    for name, (fn, work, kind) in small.items():
        r = run(fn, 3.0)
        peak = PEAK_INT8_TOPS if kind == "int8" else PEAK_BF16_TFLOPS
        r["TOPS"] = round(work / (r["ms_per_call"] * 1e-3) / 1e12, 1)
        r["frac_peak"] = round(r["TOPS"] / peak, 4)
        res[name] = r
        log(f"{name}: {json.dumps(r)}")
    print(json.dumps({"power_clock": res, "device": info}))


def hbm_from(trace_dir, fetch_dir, write_dir):
    """Per-kernel duration (kernel trace) and HBM bytes (FETCH_SIZE, WRITE_SIZE, each
    scaled by what it reads for the calibration copy) of --probe-hbm: the achieved
    HBM rate of each kernel as rocprofv3 sees it."""
    import csv
    import glob

    def rows(d, pat):
        out = []
        for f in glob.glob(os.path.join(d, "**", pat), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    dur = {}
    for r in sorted(rows(trace_dir, "*kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
        dur.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    # each kernel's last HBM_PROBE_REPS launches (the first HBM_PROBE_WARM warm up)
    dur = {k: v[-HBM_PROBE_REPS:] for k, v in dur.items()}

    def counter(d, name):
        per = {}
        for r in rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] == name:
                k = (r["Kernel_Name"], r["Dispatch_Id"])
                per[k] = per.get(k, 0.0) + float(r["Counter_Value"]) * 1024.0
        by = {}
        for (kn, _), v in per.items():
            by.setdefault(kn, []).append(v)
        return {k: sum(v) / len(v) for k, v in by.items()}

    fetch, write = counter(fetch_dir, "FETCH_SIZE"), counter(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "neg" in k]
    kf = COPY_BYTES / fetch[copy[0]]
    kw = COPY_BYTES / write[[k for k in write if "neg" in k][0]]
    out = {}
    for k, ds in dur.items():
        if "w8a8" not in k or k not in fetch or k not in write:
            continue
        t = sorted(ds)[len(ds) // 2]
        rd, wr = fetch[k] * kf, write[k] * kw
        import re
        names = re.findall(r"(\w+(?:<[^()]*>)?)\(", k)  # the kernel name with its template arguments
        short = names[-1] if names else k
        out[short] = {"launches": len(ds), "median_us": round(t * 1e6, 2),
                      "read_GB": round(rd / 1e9, 4), "write_GB": round(wr / 1e9, 4),
                      "TB/s": round((rd + wr) / t / 1e12, 3),
                      "frac_of_8TBs": round((rd + wr) / t / 1e12 / (PEAK_HBM_GBS / 1e3), 4)}
    print(json.dumps(out, indent=1))


def small_from(trace_dir, pmc_dir):
    """Per-kernel duration (kernel trace, median of each kernel's last SMALL_PROBE_REPS
    launches) and counters (median launch) of a rocprofv3 run of --probe-small (or of
    any other probe: a directory without a kernel trace gives counters only).  With
    SQ_INSTS_MFMA and SQ_VALU_MFMA_BUSY_CYCLES: the rate the matrix cores were issued
    at, and their busy share of the 1024 SIMDs at 2.4 GHz over the kernel's duration;
    with the per-CU texture-path counters (TA, TD, TCP) and GRBM_GUI_ACTIVE: their busy
    or stalled share of the active cycles."""
    import csv
    import glob
    import re

    def rows(d, pat):
        out = []
        for f in glob.glob(os.path.join(d, "**", pat), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    def short(k):  # the kernel with its template arguments, without namespaces and parameters
        k = re.sub(r"w8a8::\(anonymous namespace\)::", "", k)
        return re.sub(r"^void |\([^()]*\)$", "", k)

    def mine(k):
        return "gemm_tiled" in k or "splitk_reduce" in k

    dur = {}
    for r in sorted(rows(trace_dir, "*kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
        if mine(r["Kernel_Name"]):
            dur.setdefault(short(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    per = {}
    for r in rows(pmc_dir, "*counter_collection.csv"):
        if mine(r["Kernel_Name"]):
            k = (short(r["Kernel_Name"]), r["Dispatch_Id"])
            per.setdefault(k, {}).setdefault(r["Counter_Name"], 0.0)
            per[k][r["Counter_Name"]] += float(r["Counter_Value"])
    cnt = {}
    for (kn, _), v in per.items():
        cnt.setdefault(kn, []).append(v)
    out = {}
    for k in sorted(set(dur) | set(cnt)):
        ds = dur.get(k, [])[-SMALL_PROBE_REPS:]
        t = sorted(ds)[len(ds) // 2] if ds else None
        r = {"launches": len(ds), "median_us": round(t * 1e6, 2)} if ds else {}
        cs = cnt.get(k, [])
        if cs:
            # every counter of the median launch; per-CU blocks (TA, TD, TCP: one per CU,
            # 256) as a share of the active cycles of one XCC (GRBM_GUI_ACTIVE is summed
            # over the 8 XCCs)
            c = cs[len(cs) // 2]
            r["counters"] = {n: v for n, v in sorted(c.items())}
            act = c.get("GRBM_GUI_ACTIVE", 0.0) / 8
            for n in ("TA_TA_BUSY_sum", "TA_ADDR_STALLED_BY_TC_CYCLES_sum",
                      "TA_DATA_STALLED_BY_TC_CYCLES_sum", "TD_TD_BUSY_sum", "TD_TC_STALL_sum",
                      "TCP_PENDING_STALL_CYCLES_sum", "TCP_TCP_TA_DATA_STALL_CYCLES_sum"):
                if n in c and act > 0:
                    r[n.replace("_sum", "") + "_per_cu_frac"] = round(c[n] / (256 * act), 4)
        if cs and t and "SQ_INSTS_MFMA" in cs[0]:
            c = cs[len(cs) // 2]
            n, busy = c["SQ_INSTS_MFMA"], c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
            # the MFMA tile edge: Cfg's tenth template argument
            mt = re.search(r"Cfg<(?:[^,<>]*, ){9}(16|32)\b", k)
            # int8: 32x32x32 or 16x16x64; bf16: 32x32x16 or 16x16x32 (ops = 2 x MACs)
            ops = n * (65536 if "ElemI8" in k else 32768) // (2 if mt and mt.group(1) == "16" else 1)
            r.update({"mfma": int(n), "mfma_busy_cycles": int(busy),
                      "issued_TOPS": round(ops / t / 1e12, 1),
                      "mfma_busy_frac_at_2.4GHz": round(busy / (1024 * t * 2.4e9), 4)})
        out[k] = r
    print(json.dumps(out, indent=1))


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.probe_hbm:
        probe_hbm()
        return
    if args.probe_small:
        probe_small()
        return
    if args.power_clock:
        power_clock()
        return
    if args.hbm_from:
        hbm_from(*args.hbm_from)
        return
    if args.small_from:
        small_from(*args.small_from)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU mode "
              "(it would shard rows or output channels with no exchange); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int8_w8a8_gemm_amd as w8
    import workloads as wl

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w8.lib()

    M, D, F = args.M, 4096, 16384
    log(f"generating inputs M={M} D={D} F={F}")
    ffn = wl.video_ffn(M=M)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x = d(ffn.x)
    w1, b1, w2, b2 = d(ffn.w1), d(ffn.b1), d(ffn.w2), d(ffn.b2)
    qw1, sw1 = w8.quantize_rows(w1)   # static weight quantisation, untimed
    qw2, sw2 = w8.quantize_rows(w2)
    del w1, w2
    qx = torch.empty((M, D), dtype=torch.int8, device=dev)
    sx = torch.empty((M,), dtype=torch.float32, device=dev)
    u = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    qh = torch.empty((M, F), dtype=torch.int8, device=dev)
    sh = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    assert w8.guard(F, D) and w8.guard(D, F)
    stream = torch.cuda.current_stream()

    nev = 5
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)]
              for _ in range(args.steps)]

    def step(ev=None):
        # quantise X, up GEMM, fused GELU + quantise of its output, down GEMM;
        # each C-ABI call separately so each kernel can be timed
        if ev: ev[0].record(stream)
        w8.quantize_rows(x, qx, sx)
        if ev: ev[1].record(stream)
        w8.gemm(qx, sx, qw1, sw1, b1, act=w8.ACT_NONE, out=u)
        if ev: ev[2].record(stream)
        w8.gelu_quantize_rows(u, qh, sh)
        if ev: ev[3].record(stream)
        w8.gemm(qh, sh, qw2, sw2, b2, act=w8.ACT_NONE, out=y)
        if ev: ev[4].record(stream)

    if args.probe_traffic:
        src = torch.zeros((COPY_BYTES // 2,), dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)   # reads and writes COPY_BYTES each
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        log("traffic probe done")
        return

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    ops_gemm = 2.0 * M * F * D  # each of the two GEMMs
    value = 2 * ops_gemm / (ms_per_step * 1e-3) / 1e12

    def avg(a, b):
        return float(np.mean([events[i][a].elapsed_time(events[i][b]) for i in range(args.steps)]))

    t_qx, t_up, t_qh, t_down = avg(0, 1), avg(1, 2), avg(2, 3), avg(3, 4)
    # medians over 50 more event-timed steps, run after the timed region (they
    # do not enter `value` or ms_per_step)
    NMED = 50
    ev_med = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(NMED)]
    for i in range(NMED):
        step(ev_med[i])
    torch.cuda.synchronize()

    def med(a, b):
        return float(np.median([ev_med[i][a].elapsed_time(ev_med[i][b]) for i in range(NMED)]))

    m_qx, m_up, m_qh, m_down, m_step = med(0, 1), med(1, 2), med(2, 3), med(3, 4), med(0, 4)
    tops_up = ops_gemm / (t_up * 1e-3) / 1e12
    tops_down = ops_gemm / (t_down * 1e-3) / 1e12
    bytes_qx = 3.0 * M * D + 4.0 * M
    bytes_qh = 3.0 * M * F + 4.0 * M
    log(f"step {ms_per_step:.3f} ms: quant X {t_qx*1e3:.1f} us, GEMM up {t_up:.3f} ms "
        f"({tops_up:.0f} TOPS), GELU+quant U {t_qh*1e3:.1f} us, GEMM down {t_down:.3f} ms "
        f"({tops_down:.0f} TOPS)")

    # dominant kernel: the INT8 GEMM (one kernel, launched for the up and the
    # down projection with the same op count): average launch duration
    dom_name = ("gemm_tiled, INT8, 256x256 tiles, v_mfma_i32_16x16x64_i8 "
                "(video FFN up and down, averaged)")
    dom_t = 0.5 * (t_up + t_down)
    achieved = ops_gemm / (dom_t * 1e-3) / 1e12
    traffic = None
    st = stored_traffic()
    if st is not None:
        traffic = st.get("hbm_bytes_per_launch")
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_INT8_TOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                "traffic": traffic, "kernel": dom_name,
                "algorithmic_per_launch": f"2*M*N*K = {ops_gemm:.4e} int8 ops"}

    result = {
        "metric": "INT8 W8A8 GEMM TOPS + % of MI355X INT8 MFMA peak (video FFN shape)",
        "value": round(value, 1),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "video FFN pair, guarded W8A8 linear x2: "
                               f"X[{M}x{D}] . W1[{F}x{D}]^T +b1, GELU-tanh (fused into the "
                               f"down projection's quantisation), . W2[{D}x{F}]^T +b2",
                   "M": M, "D": D, "F": F, "act_up": "gelu_tanh", "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": {
            "timing": f"mean over the {args.steps} timed steps; median_* over {NMED} further "
                      "event-timed steps run after them",
            "quantize_x": {"us": round(t_qx * 1e3, 2), "median_us": round(m_qx * 1e3, 2),
                           "GB/s": round(bytes_qx / (t_qx * 1e-3) / 1e9, 1),
                           "frac_hbm": round(bytes_qx / (t_qx * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "gemm_up": {"ms": round(t_up, 4), "median_ms": round(m_up, 4),
                        "TOPS": round(tops_up, 1),
                        "frac_peak": round(tops_up / PEAK_INT8_TOPS, 4),
                        "median_frac_peak": round(ops_gemm / (m_up * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4)},
            "gelu_quantize_u": {"us": round(t_qh * 1e3, 2), "median_us": round(m_qh * 1e3, 2),
                           "GB/s": round(bytes_qh / (t_qh * 1e-3) / 1e9, 1),
                           "frac_hbm": round(bytes_qh / (t_qh * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "gemm_down": {"ms": round(t_down, 4), "median_ms": round(m_down, 4),
                          "TOPS": round(tops_down, 1),
                          "frac_peak": round(tops_down / PEAK_INT8_TOPS, 4),
                          "median_frac_peak": round(ops_gemm / (m_down * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4)},
            "step_median_ms": round(m_step, 4),
        },
    }

    if not args.no_extra:
        result["extra"] = extra_benches(w8, wl, np, torch, dev, d, log)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(ffn, args.cpu_rows, np, log)

    print(json.dumps(result), flush=True)


def _time(fn, iters, torch, warm_ms=20.0):
    """Average ms per call over `iters` calls, timed with events on the current stream,
    after at least `warm_ms` of untimed calls: the GPU's clocks take some tens of
    milliseconds of steady work to settle (a 350 us GEMM measured ~15% slower over
    its first 20 calls after other work)."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    import time
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(8):  # back to back, so that short kernels keep the GPU busy
            fn()
        torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


def extra_benches(w8, wl, np, torch, dev, d, log):
    """Secondary kernels: the quantiser on rotating buffers (so the 256 MB
    Infinity Cache cannot hold the input), compaction, and the BF16 fallback."""
    out = {}
    # quantise X [24576 x 4096] rotating over 4 distinct inputs (4 x 201 MB)
    M, K = 24576, 4096
    gen = torch.Generator(device=dev).manual_seed(0)
    xs = [torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16) for _ in range(4)]
    qs = [torch.empty((M, K), dtype=torch.int8, device=dev) for _ in range(4)]
    ss = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(4)]
    it = [0]

    def q():
        i = it[0] % 4
        it[0] += 1
        w8.quantize_rows(xs[i], qs[i], ss[i])

    t = _time(q, 40, torch)
    gbs = (3.0 * M * K + 4.0 * M) / (t * 1e-3) / 1e9
    out["quantize_24576x4096_rotating"] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1),
                                           "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    # per-block quantisation of the video self-attention Q and K (24576 tokens x
    # 32 heads x 128; blocks of 128 tokens for Q, 64 for K), rotating over the
    # same 4 inputs as the row quantiser
    for name, blk in (("quantize_blocks_q_24576x32x128_b128", 128),
                      ("quantize_blocks_k_24576x32x128_b64", 64)):
        nsc = 32 * (-(-M // blk))
        sbs = [torch.empty((1, -(-M // blk), 32), dtype=torch.float32, device=dev) for _ in range(4)]

        def qblocks(blk=blk, sbs=sbs):
            i = it[0] % 4
            it[0] += 1
            w8.quantize_blocks(xs[i], 1, 32, blk, q=qs[i], scale=sbs[i])

        t = _time(qblocks, 20, torch)
        nbytes = 3 * M * K + 4 * nsc
        out[name] = {"us": round(t * 1e3, 2), "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    # LayerNorm + modulation of the same video token rows in 8 conditioning
    # groups of 3072 rows, fused with the quantisation (int8 out) and alone
    # (bf16 out), rotating over the same 4 inputs
    G = 8
    mods = [(torch.randn((G, K), device=dev, generator=gen) * 0.3).to(torch.bfloat16)
            for _ in range(2)]

    def nmq():
        i = it[0] % 4
        it[0] += 1
        w8.norm_mod_quantize_rows(xs[i], mods[0], mods[1], M // G, q=qs[i], qscale=ss[i])

    t = _time(nmq, 40, torch)
    nbytes = 3.0 * M * K + 4.0 * M + 4.0 * G * K
    out["norm_mod_quantize_24576x4096_rotating"] = {
        "us": round(t * 1e3, 2), "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1),
        "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del qs
    ys = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(4)]

    def nmb():
        i = it[0] % 4
        it[0] += 1
        w8.norm_mod_bf16(xs[i], mods[0], mods[1], M // G, y=ys[i])

    t = _time(nmb, 40, torch)
    nbytes = 4.0 * M * K + 4.0 * G * K
    out["norm_mod_bf16_24576x4096_rotating"] = {
        "us": round(t * 1e3, 2), "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1),
        "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del xs, ss, ys
    # compaction of the text rows [8 x 512 x 4096]
    g = wl.guarded_mixed()
    B, L, Dm = g.x.shape
    xd = d(g.x.reshape(B * L, Dm)).view(B, L, Dm)
    md = torch.from_numpy(g.mask).to(dev)
    buf = torch.empty((B * L, Dm), dtype=torch.bfloat16, device=dev)
    src = torch.empty((B * L,), dtype=torch.int32, device=dev)
    cnt = torch.empty((1,), dtype=torch.int32, device=dev)
    t = _time(lambda: w8.compact_padded_rows(xd, md, buf, src, cnt), 50, torch)
    mc = int(cnt.item())
    nbytes = 4.0 * mc * Dm + B * L + 4.0 * mc + 4
    out["compact_8x512x4096"] = {"us": round(t * 1e3, 2), "rows_kept": mc,
                                 "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1),
                                 "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    # compaction fused with the per-row quantisation (reads the valid rows once,
    # writes their int8 codes and scales)
    qb = torch.empty((B * L, Dm), dtype=torch.int8, device=dev)
    sb = torch.empty((B * L,), dtype=torch.float32, device=dev)
    t = _time(lambda: w8.compact_quantize_rows(xd, md, qb, sb, src, cnt), 50, torch)
    nbytes = 3.0 * mc * Dm + B * L + 8.0 * mc + 4
    out["compact_quantize_8x512x4096"] = {"us": round(t * 1e3, 2), "rows_kept": mc,
                                          "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1),
                                          "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    # the linear-time compaction path (more than 8192 rows): 64 x 8192 rows of 4096
    # under a general mask (runs of valid and padded rows, about half valid)
    Bl, Ll = 64, 8192
    gl = torch.Generator(device=dev).manual_seed(1)
    xl = torch.randn((Bl * Ll, Dm), device=dev, generator=gl).to(torch.bfloat16).view(Bl, Ll, Dm)
    runs = torch.randint(1, 3000, (4096,), device=dev, generator=gl)
    starts = torch.cumsum(runs, 0)
    run_id = torch.searchsorted(starts, torch.arange(Bl * Ll, device=dev), right=True)
    ml = ((run_id % 2) == 0).to(torch.uint8).view(Bl, Ll)
    bufl = torch.empty((Bl * Ll, Dm), dtype=torch.bfloat16, device=dev)
    srcl = torch.empty((Bl * Ll,), dtype=torch.int32, device=dev)
    t = _time(lambda: w8.compact_padded_rows(xl, ml, bufl, srcl, cnt), 10, torch)
    mcl = int(cnt.item())
    nbytes = 4.0 * mcl * Dm + Bl * Ll + 4.0 * mcl + 4   # algorithmic: the mask once
    out["compact_64x8192x4096_linear_path"] = {
        "us": round(t * 1e3, 2), "rows_kept": mcl, "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1),
        "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del bufl
    qbl = torch.empty((Bl * Ll, Dm), dtype=torch.int8, device=dev)
    sbl = torch.empty((Bl * Ll,), dtype=torch.float32, device=dev)
    t = _time(lambda: w8.compact_quantize_rows(xl, ml, qbl, sbl, srcl, cnt), 10, torch)
    nbytes = 3.0 * mcl * Dm + Bl * Ll + 8.0 * mcl + 4
    out["compact_quantize_64x8192x4096_linear_path"] = {
        "us": round(t * 1e3, 2), "rows_kept": mcl, "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1),
        "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del xl, qbl, sbl, srcl, ml
    # the text projection both ways: guarded linear on the compacted bf16 rows
    # (quantise + GEMM), and the INT8 GEMM on the fused kernel's codes
    xc = buf[:mc]
    lw = w8.W8A8Linear.prepare(d(g.w), d(g.b))
    yc = torch.empty((mc, 4096), dtype=torch.bfloat16, device=dev)
    t = _time(lambda: lw(xc, y=yc), 20, torch)
    out["linear_int8_text_Mc_x4096x4096"] = {"us": round(t * 1e3, 2),
                                             "TOPS": round(2.0 * mc * 4096 * 4096 / (t * 1e-3) / 1e12, 1)}
    t = _time(lambda: w8.gemm(qb[:mc], sb[:mc], lw.qw, lw.sw, lw.bias, out=yc), 20, torch)
    out["gemm_int8_text_Mc_x4096x4096"] = {"us": round(t * 1e3, 2),
                                           "TOPS": round(2.0 * mc * 4096 * 4096 / (t * 1e-3) / 1e12, 1)}
    wa = d(g.w_a)
    ba = d(g.b_a)
    ya = torch.empty((mc, 4100), dtype=torch.bfloat16, device=dev)
    t = _time(lambda: w8.linear_bf16(xc, wa, ba, y=ya), 10, torch)
    out["fallback_bf16_N4100"] = {"us": round(t * 1e3, 2),
                                  "TFLOP/s": round(2.0 * mc * 4100 * 4096 / (t * 1e-3) / 1e12, 1)}
    xb, wb, bb = d(g.x_b), d(g.w_b), d(g.b_b)
    yb = torch.empty((2048, 2048), dtype=torch.bfloat16, device=dev)
    t = _time(lambda: w8.linear_bf16(xb, wb, bb, y=yb), 10, torch)
    out["fallback_bf16_K2050"] = {"us": round(t * 1e3, 2),
                                  "TFLOP/s": round(2.0 * 2048 * 2048 * 2050 / (t * 1e-3) / 1e12, 1)}
    # audio 2048^3 and attention projection 24576x4096x4096 GEMM alone, on the
    # codes and scales the quantiser gives for seeded N(0,1) activations and
    # N(0, 0.02^2) weights (the value distribution the step's GEMMs see: under
    # the power cap the clock, and so the rate, depends on the operand data)
    for name, (Mg, Ng, Kg) in {"gemm_audio_2048^3": (2048, 2048, 2048),
                               "gemm_attn_proj_24576x4096x4096": (24576, 4096, 4096)}.items():
        xa = torch.randn((Mg, Kg), device=dev, generator=gen).to(torch.bfloat16)
        wg = (torch.randn((Ng, Kg), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
        qa, sa = w8.quantize_rows(xa)
        qb, sb = w8.quantize_rows(wg)
        del xa, wg
        bias = (torch.randn((Ng,), device=dev, generator=gen) * 0.01).to(torch.bfloat16)
        yo = torch.empty((Mg, Ng), dtype=torch.bfloat16, device=dev)
        t = _time(lambda: w8.gemm(qa, sa, qb, sb, bias, out=yo), 20, torch)
        tops = 2.0 * Mg * Ng * Kg / (t * 1e-3) / 1e12
        out[name] = {"us": round(t * 1e3, 2), "TOPS": round(tops, 1),
                     "frac_peak": round(tops / PEAK_INT8_TOPS, 4)}
    # a short sequence through the FFN down projection (256 x 4096 x 16384): the
    # tiles cover a quarter of the CUs; split-K across workgroups against the
    # plain GEMM, same codes
    Mg, Ng, Kg = 256, 4096, 16384
    qa, sa = w8.quantize_rows(torch.randn((Mg, Kg), device=dev, generator=gen).to(torch.bfloat16))
    qb, sb = w8.quantize_rows((torch.randn((Ng, Kg), device=dev, generator=gen) * 0.02)
                              .to(torch.bfloat16))
    bias = (torch.randn((Ng,), device=dev, generator=gen) * 0.01).to(torch.bfloat16)
    yo = torch.empty((Mg, Ng), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((w8.gemm_splitk_workspace_bytes(Mg, Ng, Kg),), dtype=torch.uint8, device=dev)
    for name, fn in (("gemm_256x4096x16384", lambda: w8.gemm(qa, sa, qb, sb, bias, out=yo)),
                     ("gemm_splitk_256x4096x16384",
                      lambda: w8.gemm_splitk(qa, sa, qb, sb, bias, out=yo, workspace=ws))):
        t = _time(fn, 20, torch)
        tops = 2.0 * Mg * Ng * Kg / (t * 1e-3) / 1e12
        out[name] = {"us": round(t * 1e3, 2), "TOPS": round(tops, 1),
                     "frac_peak": round(tops / PEAK_INT8_TOPS, 4)}
    out["gemm_splitk_256x4096x16384"]["slices"] = ws.numel() // (Mg * Ng * 4)
    del qa, qb, ws
    # the attention projection with its LayerNorm + modulation prologue (8
    # conditioning groups of 3072 rows): fused (one kernel, then the GEMM) and
    # unfused (bf16 norm rows, quantise, GEMM)
    Mg, Kg = 24576, 4096
    xa = torch.randn((Mg, Kg), device=dev, generator=gen).to(torch.bfloat16)
    mods = [(torch.randn((8, Kg), device=dev, generator=gen) * 0.3).to(torch.bfloat16)
            for _ in range(2)]
    wg = (torch.randn((Kg, Kg), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    bias = (torch.randn((Kg,), device=dev, generator=gen) * 0.01).to(torch.bfloat16)
    layer = w8.W8A8Linear.prepare(wg, bias)
    del wg
    t = _time(lambda: layer.normed(xa, mods[0], mods[1], Mg // 8), 10, torch)
    out["normed_linear_attn_24576x4096x4096"] = {
        "us": round(t * 1e3, 2), "TOPS": round(2.0 * Mg * Kg * Kg / (t * 1e-3) / 1e12, 1)}
    zb = torch.empty_like(xa)

    def unfused():
        w8.norm_mod_bf16(xa, mods[0], mods[1], Mg // 8, y=zb)
        q, sq = w8.quantize_rows(zb)
        w8.gemm(q, sq, layer.qw, layer.sw, layer.bias)

    t = _time(unfused, 10, torch)
    out["normed_linear_attn_unfused_24576x4096x4096"] = {
        "us": round(t * 1e3, 2), "TOPS": round(2.0 * Mg * Kg * Kg / (t * 1e-3) / 1e12, 1)}
    del xa, zb
    log("extra: " + json.dumps(out))
    return out


def cpu_baseline(ffn, rows, np, log):
    """The CPU oracle, as it stands, on a bounded row sample of the same step
    (quantise X rows, INT32 product with W1, epilogue + GELU, quantise H rows,
    INT32 product with W2, epilogue), weights quantised beforehand."""
    import oracle

    threads = oracle.default_threads()
    qw1, sw1 = oracle.quantize_rows(ffn.w1, nthreads=threads)
    qw2, sw2 = oracle.quantize_rows(ffn.w2, nthreads=threads)

    def run(n):
        xs = np.ascontiguousarray(ffn.x[:n])
        t0 = time.perf_counter()
        qx, sx = oracle.quantize_rows(xs, nthreads=threads)
        uu = oracle.epilogue(oracle.gemm_i32(qx, qw1, nthreads=threads), sx, sw1, ffn.b1,
                             nthreads=threads)
        qh, sh = oracle.gelu_quantize_rows(uu, nthreads=threads)
        oracle.epilogue(oracle.gemm_i32(qh, qw2, nthreads=threads), sh, sw2, ffn.b2,
                        nthreads=threads)
        return time.perf_counter() - t0

    if rows <= 0:
        # size the sample to ~15 s from the marginal time per row of two probes (a
        # single small probe is dominated by its fixed cost and sized it too small)
        p1 = max(threads, 16)
        p2 = 4 * p1
        t1, t2 = run(p1), run(p2)
        per_row = max((t2 - t1) / (p2 - p1), t2 / p2 / 4, 1e-6)
        rows = int(min(ffn.x.shape[0], max(p2, 15.0 / per_row)))
        rows = max(threads, rows - rows % threads)
    log(f"cpu baseline: oracle on {rows} rows with {threads} threads")
    t = run(rows)
    ops = 2 * (2.0 * rows * ffn.w1.shape[0] * ffn.w1.shape[1])
    return {"value": round(ops / t / 1e12, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "threads": threads, "host_cores": os.cpu_count(),
            "usable_cores": oracle.usable_cores(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "cpu_model": oracle.cpu_model(),
            "seconds": round(t, 2),
            "sample": f"first {rows} of {ffn.x.shape[0]} rows of the video FFN pair step "
                      f"(quantise, INT32 GEMM, epilogue, GELU + quantise, INT32 GEMM, epilogue)"}


if __name__ == "__main__":
    main()
