#!/usr/bin/env python3
"""Throughput of the routed-expert FP8 grouped-matmul hot path on one MI355X.

One step = one pass of every op of the path over the dropless per-device
buffer of a DeepSeek-V3-like MoE layer (G=32 local experts, static buffer of
32768 rows of which 19,661 are valid, Zipf(1.1)-skewed expert sizes with four
empty experts, Inf/NaN garbage in the stale tail):

  quantize_rows_fp8 + gmm_silu_fp8_q   wi forward, K=7168 -> 2x2048, SwiGLU
  quantize_rows_fp8 + gmm_fp8_fwd_q    wo forward, K=2048 -> 7168
  gmm_dlhs_fp8                         wo dLHS  (dout [.,7168] -> [.,2048])
  gmm_dlhs_fp8                         wi dLHS  (dout [.,4096] -> [.,7168])
  tgmm_quant (e5m2 gradient)           drhs [32, 7168, 2048] f32
  dequantize_fp8_codes                 wo codes [32, 2048, 7168]

Inputs are seeded synthetic data already resident in HBM.  `value` is the
aggregate GEMM TFLOP/s of a step (flops of the five GEMMs over valid rows,
divided by the step's wall time on the GPU, dequantization included).  HIP
events recorded between the calls on the launch stream give each op's time;
the bf16 arm (same scheduler, pre-dequantized weights) gives the FP8/bf16
ratio; the CPU oracle is timed on a bounded sample on the host cores.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 (OCP) MFMA
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E

# Bytes per launch through the L2-fabric interface from rocprofv3 FETCH_SIZE / WRITE_SIZE passes over
# this bench's step (profiles/bench_step_kernels_counters.md), scaled by a plain 1 GiB copy: FETCH_SIZE
# x 2.0, WRITE_SIZE x 1.0 (MiB read, MiB written).  Each entry holds the hash of the kernel's sources when
# the counters were taken; once the sources change the figure no longer applies and traffic is null.
MEASURED_TRAFFIC_MIB = {
    "wi_gemm": ("gmm_fwd.hip", "f0b71cf866345648", 2620, 77),
    "wo_gemm": ("gmm_fwd.hip", "f0b71cf866345648", 1307, 269),
    "wi_dlhs": ("dlhs.hip", "4745e5e8785bab26", 2814, 269),
    "wo_dlhs": ("dlhs.hip", "4745e5e8785bab26", 1427, 77),
    "tgmm": ("tgmm.hip", "2423c5c4f52c4400", 346 + 1437, 181 + 1792),
    "dequant": ("dequant.hip", "8efe77d827d0d814", 455, 896),
    "wi_quant": ("quant.hip", "924b9abefe895b12", 269, 135),
    "wo_quant": ("quant.hip", "924b9abefe895b12", 77, 39),
}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` if its sources are those the counters were taken on."""
    import hashlib
    if kernel not in MEASURED_TRAFFIC_MIB:
        return None
    src, digest, rd, wr = MEASURED_TRAFFIC_MIB[kernel]
    csrc = os.path.join(ROOT, "fp8_moe_grouped_amd", "csrc")
    h = hashlib.sha256()
    for f in (src, "common.hpp", "launch.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return (rd + wr) * 2 ** 20 if h.hexdigest()[:16] == digest else None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def make_inputs():
    import workloads as W
    t0 = time.time()
    sh = W.SHAPES[3]
    G, M, valid = sh["G"], sh["M"], sh["valid"]
    gs = W.group_sizes(3)
    d = {"gs": gs, "G": G, "M": M, "valid": valid}
    d["codes_wi"], d["scale_wi"] = W.weights(3, W.W_WI, G, sh["K_wi"], sh["N_wi"])
    log(f"[bench] wi weights {time.time() - t0:.1f}s")
    d["codes_wo"], d["scale_wo"] = W.weights(3, W.W_WO, G, sh["K_wo"], sh["N_wo"])
    log(f"[bench] wo weights {time.time() - t0:.1f}s")
    d["lhs_wi"] = W.activations(3, W.LHS_WI, M, sh["K_wi"], valid, outlier_stream=W.OUTLIERS_WI)
    d["lhs_wo"] = W.activations(3, W.LHS_WO, M, sh["K_wo"], valid, outlier_stream=W.OUTLIERS_WO)
    log(f"[bench] activations {time.time() - t0:.1f}s")
    d["dout_wi"] = W.gradients(3, W.DOUT_WI, M, sh["N_wi"], valid)
    d["dout_wo"] = W.gradients(3, W.DOUT_WO, M, sh["N_wo"], valid)
    t4 = W.make(4, "tgmm")
    d["lhs_t"], d["dout_t"] = t4["lhs"], t4["dout"]
    log(f"[bench] synthetic inputs generated in {time.time() - t0:.1f}s")
    return d


def flops_of(d):
    mv = int(np.sum(d["gs"]))
    return {
        "wi_fwd": 2.0 * mv * 7168 * 4096,
        "wo_fwd": 2.0 * mv * 2048 * 7168,
        "wo_dlhs": 2.0 * mv * 7168 * 2048,
        "wi_dlhs": 2.0 * mv * 4096 * 7168,
        "tgmm": 2.0 * mv * 7168 * 2048,
    }


def bytes_of(d):
    """Algorithmic HBM bytes per op: valid rows in and out, codes and scales of
    non-empty experts, full outputs where the op writes them."""
    mv = int(np.sum(d["gs"]))
    ne = int(np.sum(np.asarray(d["gs"]) > 0))
    G = d["G"]
    return {
        "wi_quant": mv * 7168 * (2 + 1) + mv * 4,
        "wi_gemm": mv * 7168 + mv * 4 + ne * 7168 * 4096 * 1 + ne * 4096 * 4 + mv * 2048 * 2,
        "wo_quant": mv * 2048 * (2 + 1) + mv * 4,
        "wo_gemm": mv * 2048 + mv * 4 + ne * 2048 * 7168 + ne * 7168 * 4 + mv * 7168 * 2,
        "wo_dlhs": mv * 7168 * 2 + ne * 2048 * 7168 + ne * 7168 * 4 + mv * 2048 * 2,
        "wi_dlhs": mv * 4096 * 2 + ne * 7168 * 4096 + ne * 4096 * 4 + mv * 7168 * 2,
        "tgmm": mv * (7168 + 2048) * 2 + G * 7168 * 2048 * 4,
        "dequant": G * 2048 * 7168 * (1 + 2) + G * 7168 * 4,
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(d, seconds_target):
    """The oracle as it stands, on a bounded sample: the wi forward (SwiGLU) of
    evenly spread valid rows, timed three times (median), on this host's
    cores.  Beside it, for a fairer CPU throughput figure, the same sample
    with the oracle's own quantization and an f32 BLAS contraction (not the
    oracle: its products are rounded in f32)."""
    from oracle import formats as F
    from oracle import gmm as O
    mv = int(np.sum(d["gs"]))
    # size the sample so that one run takes about seconds_target / 6 (the
    # per-expert weight decode is a fixed cost of a few seconds; the row count
    # doubles until the run is at least half that long)
    n = 1024
    while True:
        rows = np.linspace(0, mv - 1, n).astype(np.int64)
        t0 = time.time()
        O.gmm_fwd(d["lhs_wi"], d["codes_wi"], d["scale_wi"], d["gs"], swiglu_out=True, rows=rows)
        dt = time.time() - t0
        if dt * 12 > seconds_target or n >= mv:
            break
        n = min(2 * n, mv)
    runs = []
    for _ in range(3):
        t0 = time.time()
        O.gmm_fwd(d["lhs_wi"], d["codes_wi"], d["scale_wi"], d["gs"], swiglu_out=True, rows=rows)
        runs.append(time.time() - t0)

    def f32_variant():
        lay = O.layout(d["gs"], d["M"])
        gid = lay.group_of_rows(d["M"])[rows]
        for g in np.unique(gid):
            sel = rows[gid == g]
            x = F.bf16_to_f32(d["lhs_wi"][sel])
            s = O.row_scales(x)
            q = F.decode(O.quantize_rows(x, s), F.E4M3).astype(np.float32)
            c = F.decode(d["codes_wi"][g], F.E4M3).astype(np.float32)
            y = (q @ c) * s[:, None] * d["scale_wi"][g][None, :]
            F.f64_to_bf16_bits(O.swiglu(y[:, :2048].astype(np.float64), y[:, 2048:].astype(np.float64)))

    runs32 = []
    for _ in range(3):
        t0 = time.time()
        f32_variant()
        runs32.append(time.time() - t0)
    fl = 2.0 * n * 7168 * 4096
    med, med32 = float(np.median(runs)), float(np.median(runs32))
    return {"value": fl / med / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"wi forward + SwiGLU (K=7168, N=2x2048) of {n} of the {mv} valid rows, spread over the "
                      f"experts; median of 3 runs ({', '.join(f'{t:.1f}' for t in runs)} s), float64 oracle",
            "host": {"cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()},
            "f32_blas_variant": {"value": fl / med32 / 1e12, "unit": "TFLOP/s",
                                 "runs_s": [round(t, 2) for t in runs32],
                                 "what": "same sample, oracle quantization, f32 BLAS contraction (not the oracle)"}}


def sample_sclk(run_for_s, fn):
    """Shader clock while the bench step runs back to back for about
    run_for_s seconds: amd-smi is sampled in a second thread; returns the
    samples (MHz) or the error."""
    import subprocess
    import threading
    samples, errors = [], []
    stop = threading.Event()

    def find_clk(obj):
        if isinstance(obj, dict):
            for k, v in obj.items():
                if "gfx" in str(k).lower():
                    c = v.get("clk") if isinstance(v, dict) else None
                    if isinstance(c, dict) and isinstance(c.get("value"), (int, float)):
                        return float(c["value"])
                r = find_clk(v)
                if r is not None:
                    return r
        elif isinstance(obj, list):
            for v in obj:
                r = find_clk(v)
                if r is not None:
                    return r
        return None

    def sampler():
        while not stop.is_set():
            try:
                p = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True,
                                   text=True, timeout=10)
                v = find_clk(json.loads(p.stdout)) if p.returncode == 0 else None
                if v is None:
                    errors.append((p.stderr or p.stdout)[-200:])
                else:
                    samples.append(v)
            except Exception as e:   # tool missing or unparsable output: report, do not fail the bench
                errors.append(str(e)[:200])
            stop.wait(0.2)

    import torch
    t0 = time.time()
    while time.time() - t0 < 0.3:                  # the clock ramps up first; sample once it has
        fn()
        torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.time()
    while time.time() - t0 < run_for_s:
        fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if samples:
        return {"mhz_median": float(np.median(samples)), "samples": samples, "source": "amd-smi metric --clock"}
    return {"mhz_median": None, "error": errors[-1] if errors else "no sample"}


def tgmm_dense_vs_in_kernel(G, stream, lhs, dout, gs, mv):
    """The weight-gradient tgmm on the dropless buffer (32768 static rows,
    19661 valid): in-kernel per-(tile, channel) quantization of the valid
    rows (tgmm_quant) against the buffer-wide quantization baseline
    (tgmm_dense_quant: every row of the buffer quantized, then the same
    GEMM).  The garbage tail makes the baseline's gradient NaN; the timing is
    what this records."""
    import torch
    M, K = lhs.shape
    N = dout.shape[1]
    Gn = gs.shape[0]
    out = torch.empty((Gn, K, N), dtype=torch.float32, device=lhs.device)
    ws_i = torch.empty(G.workspace_bytes(G.OP_TGMM, M, K, N, Gn, 512), dtype=torch.uint8, device=lhs.device)
    ws_d = torch.empty(G.workspace_bytes(G.OP_TGMM_DENSE, M, K, N, Gn, 0), dtype=torch.uint8, device=lhs.device)

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(n):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / n

    t_i = timed(lambda: G.tgmm_quant(lhs, dout, gs, "e5m2", 512, out=out, workspace=ws_i))
    t_d = timed(lambda: G.tgmm_dense_quant(lhs, dout, gs, "e5m2", out=out, workspace=ws_d))
    del ws_d
    return {"workload": f"tgmm {K}x{N} e5m2 on the dropless buffer: {M} static rows, {mv} valid",
            "in_kernel_ms": round(t_i, 4), "dense_ms": round(t_d, 4), "dense_over_in_kernel": round(t_d / t_i, 3)}


def vendor_dense(stream, mv, wi_gemm_ms, wi_dlhs_ms):
    """Reference point for the GEMM rates: the vendor library (hipBLASLt,
    through torch) on one dense matrix with the same flops as the grouped
    GEMMs' valid rows (no experts, no ragged tails, no scales): the FP8
    forward shape (mv x 7168 by 7168 x 4096, e4m3, f32 accumulation, bf16
    out) and the bf16 dLHS shape (mv x 4096 by 4096 x 7168).  Random values;
    only the time is used.  Not part of the library's path."""
    import torch

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(n):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / n

    out = {"workload": f"one dense matrix of {mv} rows: FP8 {mv}x7168 @ 7168x4096 and bf16 {mv}x4096 @ 4096x7168"}
    fl = 2.0 * mv * 7168 * 4096
    g = torch.Generator(device="cuda").manual_seed(5)
    try:
        a8 = torch.randn(mv, 7168, device="cuda", generator=g).to(torch.float8_e4m3fn)
        b8 = torch.randn(4096, 7168, device="cuda", generator=g).to(torch.float8_e4m3fn).t()   # column-major
        one = torch.ones((), device="cuda")
        t = timed(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
        out["fp8_ms"] = round(t, 4)
        out["fp8_tflops"] = round(fl / t / 1e9, 1)
        out["wi_gemm_rate_over_vendor"] = round(t / wi_gemm_ms, 3)
        del a8, b8
    except Exception as e:   # FP8 GEMM not offered by this torch build
        out["fp8_error"] = str(e)[:200]
    a = torch.randn(mv, 4096, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(4096, 7168, device="cuda", generator=g).to(torch.bfloat16)
    t = timed(lambda: torch.mm(a, b))
    out["bf16_ms"] = round(t, 4)
    out["bf16_tflops"] = round(fl / t / 1e9, 1)
    out["wi_dlhs_rate_over_vendor"] = round(t / wi_dlhs_ms, 3)
    return out


def skinny_groups(G, stream, codes_wi, scale_wi, codes_wo, scale_wo, rows_per_expert=16):
    """Skinny groups: every one of the 32 experts gets only a few rows
    (16 = 64 tokens x top-8 / 32, a decode-like batch), so the forward and
    the dLHS are bound by reading each expert's weight codes once.  Reported
    as HBM GB/s of the algorithmic bytes: codes + scales of every expert,
    bf16 activations read, bf16 output written (the quantizer pass of the
    forward is timed with it)."""
    import torch
    Gn, K1, N1 = codes_wi.shape
    _, K2, N2 = codes_wo.shape
    M = Gn * rows_per_expert
    gs = torch.full((Gn,), rows_per_expert, dtype=torch.int32, device=codes_wi.device)
    g = torch.Generator(device="cuda").manual_seed(11)
    x1 = torch.randn(M, K1, device="cuda", generator=g).to(torch.bfloat16)
    x2 = torch.randn(M, K2, device="cuda", generator=g).to(torch.bfloat16)
    d1 = (torch.randn(M, N1, device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
    d2 = (torch.randn(M, N2, device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
    h = torch.empty(M, N1 // 2, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(M, N2, dtype=torch.bfloat16, device="cuda")
    dx1 = torch.empty(M, K1, dtype=torch.bfloat16, device="cuda")
    dx2 = torch.empty(M, K2, dtype=torch.bfloat16, device="cuda")

    def timed(fn, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(n):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / n

    def gbs(nbytes, ms):
        return round(nbytes / ms / 1e6, 1)

    w1 = Gn * K1 * N1 + Gn * N1 * 4
    w2 = Gn * K2 * N2 + Gn * N2 * 4
    out = {"workload": f"{Gn} experts x {rows_per_expert} rows ({M} rows): wi {K1} -> 2x{N1 // 2} SwiGLU, "
                       f"wo {K2} -> {N2}, and their dLHS; bytes = weight codes + scales + activations + outputs",
           "hbm_peak_gbs": HBM_PEAK_GBS}
    ws1 = torch.empty(G.workspace_bytes(G.OP_SILU, M, K1, N1, Gn), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(G.workspace_bytes(G.OP_FWD, M, K2, N2, Gn), dtype=torch.uint8, device="cuda")
    t = timed(lambda: G.gmm_silu_fp8(x1, codes_wi, scale_wi, gs, out=h, workspace=ws1))
    out["wi_fwd"] = {"ms": round(t, 4), "gbs": gbs(w1 + M * K1 * 2 + M * (N1 // 2) * 2, t)}
    t = timed(lambda: G.gmm_fp8_fwd(x2, codes_wo, scale_wo, gs, out=y, workspace=ws2))
    out["wo_fwd"] = {"ms": round(t, 4), "gbs": gbs(w2 + M * K2 * 2 + M * N2 * 2, t)}
    t = timed(lambda: G.gmm_dlhs_fp8(d1, codes_wi, scale_wi, gs, out=dx1))
    out["wi_dlhs"] = {"ms": round(t, 4), "gbs": gbs(w1 + M * N1 * 2 + M * K1 * 2, t)}
    t = timed(lambda: G.gmm_dlhs_fp8(d2, codes_wo, scale_wo, gs, out=dx2))
    out["wo_dlhs"] = {"ms": round(t, 4), "gbs": gbs(w2 + M * N2 * 2 + M * K2 * 2, t)}
    for k in ("wi_fwd", "wo_fwd", "wi_dlhs", "wo_dlhs"):
        out[k]["frac_hbm"] = round(out[k]["gbs"] / HBM_PEAK_GBS, 3)
    return out


def small_configs(G, stream):
    """The small configurations (µs-scale calls, where launches and the amax
    pass weigh): config 0 forward (G=4, M=256, K=128, N=256), config 1 wi
    forward with SwiGLU (G=8, M=8192, K=2048, N=2x768), config 2 wo forward
    and its dLHS (G=8, M=8192, K=768, N=2048), all rows valid.  Each call is
    timed with HIP events over 50 calls after 5 warmups (quantizer included in
    the forwards); the roofline time is the larger of flops at the MFMA peak
    (FP8 forward, bf16 dLHS) and the algorithmic bytes at the HBM peak."""
    import torch
    import workloads as W

    def timed(fn, n=50):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    out = {"workload": "configs 0-2 (all rows valid), 50 calls each after 5 warmups"}
    for name, cfg, op in (("cfg0_fwd", 0, "fwd"), ("cfg1_wi_fwd", 1, "wi"), ("cfg2_wo_fwd", 2, "wo"),
                          ("cfg2_wo_dlhs", 2, "dlhs_wo")):
        d = W.make(cfg, op)
        Gn, M, K, N = d["G"], len(d["lhs"]) if "lhs" in d else len(d["dout"]), d["K"], d["N"]
        gs = to_dev(np.asarray(d["group_sizes"], np.int32))
        codes, scale = to_dev(d["codes"]), to_dev(d["scale"])
        flops = 2.0 * M * K * N
        if op == "dlhs_wo":
            dout = to_dev(d["dout"])
            res = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
            fn = lambda: G.gmm_dlhs_fp8(dout, codes, scale, gs, out=res)
            nbytes = M * N * 2 + Gn * K * N + Gn * N * 4 + M * K * 2
            peak = BF16_PEAK_TFLOPS
        else:
            x = to_dev(d["lhs"])
            swiglu = op == "wi"
            res = torch.empty((M, N // 2 if swiglu else N), dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(G.workspace_bytes(G.OP_SILU if swiglu else G.OP_FWD, M, K, N, Gn), dtype=torch.uint8,
                             device="cuda")
            if swiglu:
                fn = lambda: G.gmm_silu_fp8(x, codes, scale, gs, out=res, workspace=ws)
            else:
                fn = lambda: G.gmm_fp8_fwd(x, codes, scale, gs, out=res, workspace=ws)
            nbytes = M * K * 2 + Gn * K * N + Gn * N * 4 + res.numel() * 2
            peak = FP8_PEAK_TFLOPS
        ms = timed(fn)
        roof_us = max(flops / (peak * 1e12), nbytes / (HBM_PEAK_GBS * 1e9)) * 1e6
        out[name] = {"us": round(ms * 1e3, 2), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                     "roofline_us": round(roof_us, 2), "frac_roofline": round(roof_us / (ms * 1e3), 3)}
    return out


def lhs_quant_variants(G, stream, x, codes, scale, gs, mv):
    """The forward's ops-level LHS-quantization variants on the dropless wi
    input (K = 7168, N = 4096 without SwiGLU): quantizer + GEMM per call."""
    import torch
    M, K = x.shape
    N = codes.shape[2]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    ws = torch.empty(G.workspace_bytes(G.OP_FWD_VARIANT, M, K, N, codes.shape[0], 512), dtype=torch.uint8,
                     device=x.device)
    res = {"workload": "dropless wi input: G=32, 19661 valid rows, K=7168, N=4096 (no SwiGLU)"}
    for name, kw in (("full_k_f32", {}), ("full_k_rhs_scale_first", dict(rhs_scale_first=True)),
                     ("block512_f32", dict(lhs_block=512)),
                     ("block512_bf16_scale_bf16_acc", dict(lhs_block=512, scale_bf16=True, acc_bf16=True))):
        fn = lambda: G.gmm_fp8_fwd_variant(x, codes, scale, gs, out=out, workspace=ws, **kw)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(10):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize()
        ms = e[0].elapsed_time(e[1]) / 10
        res[name] = {"ms": round(ms, 4), "tflops": round(2.0 * mv * K * N / (ms * 1e-3) / 1e12, 1)}
    return res


def pages_microbench(G, stream):
    """The pages' GMM kernel microbenchmark shape (one call at full fill, 64
    experts, 225,280 rows; wi 4096 -> 2x1024 with SwiGLU, wo 1024 -> 4096):
    the FP8 arm (row quantizer + FP8 GEMM, as the pages time the in-kernel
    activation quantization) against the bf16 arm (the same kernel on bf16
    operands, weights dequantized beforehand and not timed); plus the dLHS of
    the same weights from the codes."""
    import torch
    import workloads as W

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(n):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / n

    res = {"workload": "pages' GMM microbenchmark shape: G=64, 225280 rows at full fill (uniform routing), "
                       "wi 4096 -> 2x1024 (SwiGLU), wo 1024 -> 4096",
           "pages_tpu7x_fp8_over_bf16": {"wi": 1.635, "wo": 1.731}}
    for op in ("wi", "wo"):
        t0 = time.time()
        d = W.micro(op)
        log(f"[bench] microbenchmark {op} inputs {time.time() - t0:.1f}s")
        M, K, N = d["M"], d["K"], d["N"]
        gs = to_dev(d["group_sizes"])
        x, codes, scale = to_dev(d["lhs"]), to_dev(d["codes"]), to_dev(d["scale"])
        del d
        sw = op == "wi"
        aq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        asc = torch.empty((M,), dtype=torch.float32, device=x.device)
        out = torch.empty((M, N // 2 if sw else N), dtype=torch.bfloat16, device=x.device)
        w = G.dequantize_fp8_codes(codes, scale)
        q_fn = G.gmm_silu_fp8_q if sw else G.gmm_fp8_fwd_q
        bf_fn = G.gmm_bf16_silu if sw else G.gmm_bf16_fwd
        t_q = timed(lambda: G.quantize_rows_fp8(x, gs, codes=aq, scales=asc))
        t_g = timed(lambda: q_fn(aq, asc, codes, scale, gs, out=out))
        t_f = timed(lambda: (G.quantize_rows_fp8(x, gs, codes=aq, scales=asc),
                             q_fn(aq, asc, codes, scale, gs, out=out)))
        t_b = timed(lambda: bf_fn(x, w, gs, out=out))
        flops = 2.0 * M * K * N
        dout = torch.randn((M, N), generator=torch.Generator(device=x.device).manual_seed(7), device=x.device,
                           dtype=torch.float32).mul_(1e-3).to(torch.bfloat16)
        dl = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
        t_d = timed(lambda: G.gmm_dlhs_fp8(dout, codes, scale, gs, out=dl))
        t_db = timed(lambda: G.gmm_bf16_dlhs(dout, w, gs, out=dl))
        res[op] = {"fp8_ms": round(t_f, 4), "fp8_quant_ms": round(t_q, 4), "fp8_gemm_ms": round(t_g, 4),
                   "bf16_ms": round(t_b, 4), "fp8_over_bf16": round(t_b / t_f, 3),
                   "fp8_tflops": round(flops / (t_f * 1e-3) / 1e12, 1),
                   "fp8_gemm_tflops": round(flops / (t_g * 1e-3) / 1e12, 1),
                   "bf16_tflops": round(flops / (t_b * 1e-3) / 1e12, 1),
                   "dlhs_fp8_codes_ms": round(t_d, 4), "dlhs_bf16_weights_ms": round(t_db, 4),
                   "dlhs_tflops": round(flops / (t_d * 1e-3) / 1e12, 1)}
        del x, codes, scale, aq, asc, out, w, dout, dl
        torch.cuda.empty_cache()
    return res


def ffn_step(G, args, gs, x, wi_codes, wi_scale, wo_codes, wo_scale, dy, mv, stream):
    """One routed-expert FFN forward + backward on the same buffer (H = 7168,
    I = 2048): moe_ffn_fp8_fwd then moe_ffn_fp8_bwd (e5m2 gradients), timed
    with HIP events on the launch stream; then each backward op alone."""
    import torch
    M, H = x.shape
    I = wo_codes.shape[1]
    dev = x.device
    h = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
    pre = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    dz = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    dwi = torch.empty((32, H, 2 * I), dtype=torch.float32, device=dev)
    dwo = torch.empty((32, I, H), dtype=torch.float32, device=dev)
    ws_f = torch.empty(G.workspace_bytes(G.OP_FFN_FWD, M, H, I, 32, 0), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(G.workspace_bytes(G.OP_FFN_BWD, M, H, I, 32, 512), dtype=torch.uint8, device=dev)

    def fwd():
        G.moe_ffn_fp8_fwd(x, wi_codes, wi_scale, wo_codes, wo_scale, gs, h=h, preact=pre, y=y, workspace=ws_f)

    def bwd():
        G.moe_ffn_fp8_bwd(x, h, pre, dy, wi_codes, wi_scale, wo_codes, wo_scale, gs, "e5m2", d_preact=dz, dx=dx,
                          dwi=dwi, dwo=dwo, workspace=ws_b)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in ev:
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        bwd()
        e[2].record(stream)
    torch.cuda.synchronize()
    ms_f = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    ms_b = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    # the backward's calls one by one (same kernels, same buffers)
    parts = [
        ("dswiglu", 2.0 * mv * I * H, lambda: G.gmm_dswiglu_fp8(dy, wo_codes, wo_scale, gs, pre, out=dz)),
        ("wi_dlhs", 4.0 * mv * I * H, lambda: G.gmm_dlhs_fp8(dz, wi_codes, wi_scale, gs, out=dx)),
        ("tgmm_wo", 2.0 * mv * I * H, lambda: G.tgmm_quant(h, dy, gs, "e5m2", 512, out=dwo, workspace=ws_b)),
        ("tgmm_wi", 4.0 * mv * I * H, lambda: G.tgmm_quant(x, dz, gs, "e5m2", 512, out=dwi, workspace=ws_b)),
    ]
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(args.steps)]
    for e in pev:
        for i, (_, _, fn) in enumerate(parts):
            e[i].record(stream)
            fn()
        e[-1].record(stream)
    torch.cuda.synchronize()
    bwd_ops = {}
    for i, (name, fl, _) in enumerate(parts):
        ms = float(np.mean([e[i].elapsed_time(e[i + 1]) for e in pev]))
        bwd_ops[name] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}
    fl_f = 6.0 * mv * H * I
    fl_b = 12.0 * mv * H * I
    del dwi, dwo
    return {
        "workload": "one MoE FFN forward + backward on the dropless buffer: H=7168, I=2048, G=32, "
                    f"{mv} valid rows; e5m2 gradients",
        "ms_fwd": round(ms_f, 4), "ms_bwd": round(ms_b, 4), "ms_step": round(ms_f + ms_b, 4),
        "tflop_per_step": round((fl_f + fl_b) / 1e12, 4),
        "tflops": round((fl_f + fl_b) / ((ms_f + ms_b) * 1e-3) / 1e12, 2),
        "tflops_fwd": round(fl_f / (ms_f * 1e-3) / 1e12, 2),
        "tflops_bwd": round(fl_b / (ms_b * 1e-3) / 1e12, 2),
        "bwd_ops": bwd_ops,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=30.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16-arm", action="store_true")
    ap.add_argument("--no-ffn", action="store_true", help="skip the MoE FFN forward + backward measurement")
    ap.add_argument("--no-micro", action="store_true", help="skip the pages' microbenchmark shape")
    ap.add_argument("--no-variants", action="store_true", help="skip the LHS-quantization variants")
    ap.add_argument("--no-dense", action="store_true", help="skip the buffer-wide tgmm baseline")
    ap.add_argument("--no-vendor", action="store_true", help="skip the vendor dense-GEMM reference")
    ap.add_argument("--no-skinny", action="store_true", help="skip the skinny-groups (decode-like) measurement")
    ap.add_argument("--no-small", action="store_true", help="skip the small configurations (configs 0-2)")
    ap.add_argument("--no-sclk", action="store_true", help="skip the shader-clock sampling")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy (read MIB, write MIB) three times; used to scale "
                         "the FETCH_SIZE / WRITE_SIZE hardware counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_moe_grouped_amd as G
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    G.lib()

    if args.copy_calibration:
        n = args.copy_calibration << 18                     # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"read_bytes": 4 * n, "write_bytes": 4 * n, "launches": 3}}))
        return

    d = make_inputs()
    gs = to_dev(d["gs"])
    M = d["M"]
    lhs_wi, lhs_wo = to_dev(d["lhs_wi"]), to_dev(d["lhs_wo"])
    codes_wi, scale_wi = to_dev(d["codes_wi"]), to_dev(d["scale_wi"])
    codes_wo, scale_wo = to_dev(d["codes_wo"]), to_dev(d["scale_wo"])
    dout_wi, dout_wo = to_dev(d["dout_wi"]), to_dev(d["dout_wo"])
    lhs_t, dout_t = to_dev(d["lhs_t"]), to_dev(d["dout_t"])
    dev = lhs_wi.device
    aq_wi = torch.empty((M, 7168), dtype=torch.uint8, device=dev)
    as_wi = torch.empty((M,), dtype=torch.float32, device=dev)
    aq_wo = torch.empty((M, 2048), dtype=torch.uint8, device=dev)
    as_wo = torch.empty((M,), dtype=torch.float32, device=dev)
    h = torch.empty((M, 2048), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, 7168), dtype=torch.bfloat16, device=dev)
    dh = torch.empty((M, 2048), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, 7168), dtype=torch.bfloat16, device=dev)
    drhs = torch.empty((32, 7168, 2048), dtype=torch.float32, device=dev)
    ws_t = torch.empty(G.workspace_bytes(G.OP_TGMM, M, 7168, 2048, 32), dtype=torch.uint8, device=dev)
    wdeq = torch.empty((32, 2048, 7168), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    names = ["wi_quant", "wi_gemm", "wo_quant", "wo_gemm", "wo_dlhs", "wi_dlhs", "tgmm", "dequant"]
    calls = [
        lambda: G.quantize_rows_fp8(lhs_wi, gs, codes=aq_wi, scales=as_wi),
        lambda: G.gmm_silu_fp8_q(aq_wi, as_wi, codes_wi, scale_wi, gs, out=h),
        lambda: G.quantize_rows_fp8(lhs_wo, gs, codes=aq_wo, scales=as_wo),
        lambda: G.gmm_fp8_fwd_q(aq_wo, as_wo, codes_wo, scale_wo, gs, out=y),
        lambda: G.gmm_dlhs_fp8(dout_wo, codes_wo, scale_wo, gs, out=dh),
        lambda: G.gmm_dlhs_fp8(dout_wi, codes_wi, scale_wi, gs, out=dx),
        lambda: G.tgmm_quant(lhs_t, dout_t, gs, "e5m2", 512, out=drhs, workspace=ws_t),
        lambda: G.dequantize_fp8_codes(codes_wo, scale_wo, out=wdeq),
    ]

    def step(events=None):
        for i, c in enumerate(calls):
            if events is not None:
                events[i].record(stream)
            c()
        if events is not None:
            events[-1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(args.steps):
        step(ev[s])
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps
    op_ms = {n: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]))
             for i, n in enumerate(names)}

    fl = flops_of(d)
    by = bytes_of(d)
    total_flops = sum(fl.values())
    value = total_flops / (ms_step * 1e-3) / 1e12

    def tfs(f, ms):
        return f / (ms * 1e-3) / 1e12

    ops = {
        "wi_fwd": {"ms": op_ms["wi_quant"] + op_ms["wi_gemm"], "tflops": tfs(fl["wi_fwd"], op_ms["wi_quant"] + op_ms["wi_gemm"]),
                   "peak": FP8_PEAK_TFLOPS},
        "wo_fwd": {"ms": op_ms["wo_quant"] + op_ms["wo_gemm"], "tflops": tfs(fl["wo_fwd"], op_ms["wo_quant"] + op_ms["wo_gemm"]),
                   "peak": FP8_PEAK_TFLOPS},
        "wo_dlhs": {"ms": op_ms["wo_dlhs"], "tflops": tfs(fl["wo_dlhs"], op_ms["wo_dlhs"]), "peak": BF16_PEAK_TFLOPS},
        "wi_dlhs": {"ms": op_ms["wi_dlhs"], "tflops": tfs(fl["wi_dlhs"], op_ms["wi_dlhs"]), "peak": BF16_PEAK_TFLOPS},
        "tgmm": {"ms": op_ms["tgmm"], "tflops": tfs(fl["tgmm"], op_ms["tgmm"]),
                 "gbs": by["tgmm"] / (op_ms["tgmm"] * 1e-3) / 1e9},
        "dequant": {"ms": op_ms["dequant"], "gbs": by["dequant"] / (op_ms["dequant"] * 1e-3) / 1e9},
    }
    for k in ("wi_fwd", "wo_fwd", "wo_dlhs", "wi_dlhs"):
        ops[k]["frac_peak"] = ops[k]["tflops"] / ops[k]["peak"]
    kern = {k: {"ms": op_ms[k]} for k in names}
    for k in ("wi_gemm", "wo_gemm"):
        f = fl["wi_fwd"] if k == "wi_gemm" else fl["wo_fwd"]
        kern[k]["tflops"] = tfs(f, op_ms[k])
        kern[k]["frac_fp8_peak"] = kern[k]["tflops"] / FP8_PEAK_TFLOPS
    for k in ("wi_quant", "wo_quant", "dequant"):
        kern[k]["gbs"] = by[k] / (op_ms[k] * 1e-3) / 1e9

    # every timed item of the step against its own roofline; the dominant one (by time) is `roofline`.
    # The tgmm item is one call of two launches (the operand prep, then the GEMM), timed together.
    launched = {"wi_quant": "quant_rows_e4m3_kernel<16>", "wi_gemm": "gmm_fp8_fwd_kernel<false, true, 256>",
                "wo_quant": "quant_rows_e4m3_kernel<4>", "wo_gemm": "gmm_fp8_fwd_kernel<false, false, 256>",
                "wo_dlhs": "gmm_dlhs_kernel (wo, 256 x 256 tiles)", "wi_dlhs": "gmm_dlhs_kernel (wi, 256 x 256 tiles)",
                "tgmm": "tgmm_prep_kernel<true> + tgmm_gemm_kernel<true, 256>", "dequant": "dequant_kernel<true>"}

    def roofline_of(k):
        if k in ("wi_gemm", "wo_gemm"):
            f = fl["wi_fwd"] if k == "wi_gemm" else fl["wo_fwd"]
            r = {"bound": "mfma", "achieved": tfs(f, op_ms[k]), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s"}
        elif k in ("wi_dlhs", "wo_dlhs"):
            r = {"bound": "mfma", "achieved": tfs(fl[k], op_ms[k]), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        else:
            r = {"bound": "hbm", "achieved": by[k] / (op_ms[k] * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        r["frac"] = r["achieved"] / r["peak"]
        r["ms"] = op_ms[k]
        r["kernels"] = launched.get(k, k)
        return r

    dom = max(names, key=lambda k: op_ms[k])
    roof = {"kernel": dom, **roofline_of(dom)}
    roof["traffic"] = measured_traffic(dom)
    roof["traffic_unit"] = ("bytes per launch through the L2-fabric interface (rocprofv3 FETCH_SIZE x 2.0 + "
                            "WRITE_SIZE, calibrated on a 1 GiB copy); Infinity Cache hits included")
    roof_all = {k: {**roofline_of(k), "traffic": measured_traffic(k)} for k in names}

    # bf16 arm: same scheduler, weights dequantized beforehand (not timed)
    ratio = None
    if not args.no_bf16_arm:
        w_wi = G.dequantize_fp8_codes(codes_wi, scale_wi)
        w_wo = wdeq

        def timed(fn, n=10):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n

        t_bf_wi = timed(lambda: G.gmm_bf16_silu(lhs_wi, w_wi, gs, out=h))
        t_bf_wo = timed(lambda: G.gmm_bf16_fwd(lhs_wo, w_wo, gs, out=y))
        ratio = {"wi": t_bf_wi / ops["wi_fwd"]["ms"], "wo": t_bf_wo / ops["wo_fwd"]["ms"],
                 "bf16_wi_ms": t_bf_wi, "bf16_wo_ms": t_bf_wo,
                 "pages_tpu7x": {"wi": 1.635, "wo": 1.731}}
        del w_wi

    mv = int(np.sum(d["gs"]))
    # the tgmm with the e4m3 gradient format (the step times e5m2)
    def timed_op(fn, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n
    t_e4 = timed_op(lambda: G.tgmm_quant(lhs_t, dout_t, gs, "e4m3", 512, out=drhs, workspace=ws_t))
    t_e5 = timed_op(lambda: G.tgmm_quant(lhs_t, dout_t, gs, "e5m2", 512, out=drhs, workspace=ws_t))
    tgmm_grad = {"workload": "tgmm 7168x2048 on the dropless buffer, 10 calls each after 3 warmups",
                 "e5m2_ms": round(t_e5, 4), "e4m3_ms": round(t_e4, 4),
                 "e5m2_gbs": round(by["tgmm"] / (t_e5 * 1e-3) / 1e9, 1),
                 "e4m3_gbs": round(by["tgmm"] / (t_e4 * 1e-3) / 1e9, 1)}
    sclk = None if args.no_sclk else sample_sclk(2.5, step)
    variants = None if args.no_variants else lhs_quant_variants(G, stream, lhs_wi, codes_wi, scale_wi, gs, mv)
    dense = None if args.no_dense else tgmm_dense_vs_in_kernel(G, stream, lhs_t, dout_t, gs, mv)
    micro = None if args.no_micro else pages_microbench(G, stream)
    vendor = None if args.no_vendor else vendor_dense(stream, mv, kern["wi_gemm"]["ms"], ops["wi_dlhs"]["ms"])
    skinny = None if args.no_skinny else skinny_groups(G, stream, codes_wi, scale_wi, codes_wo, scale_wo)
    small = None if args.no_small else small_configs(G, stream)
    ffn = None if args.no_ffn else ffn_step(G, args, gs, lhs_wi, codes_wi, scale_wi, codes_wo, scale_wo, dout_wo,
                                            int(np.sum(d["gs"])), stream)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(d, args.cpu_seconds)

    line = {
        "metric": "FP8 grouped-GEMM TFLOP/s (fwd wi/wo, bwd dLHS) and % of MI355X MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16",
        "data": "synthetic",
        "config": {
            "workload": "DeepSeek-V3-like dropless per-device MoE step: G=32 experts, 32768-row buffer with "
                        "19661 valid rows (Zipf 1.1, 4 empty experts, garbage tail); wi 7168->2x2048 SwiGLU, "
                        "wo 2048->7168, dLHS wi+wo, tgmm 7168x2048 e5m2, dequantize wo codes",
            "G": 32, "M": M, "valid_rows": int(np.sum(d["gs"])),
            "gemm_tflop_per_step": round(total_flops / 1e12, 4),
        },
        "roofline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()},
        "roofline_all": {n: {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                         for n, r in roof_all.items()},
        "cpu_baseline": cpu,
        "ops": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()} for k, v in ops.items()},
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kern.items()},
        "fp8_over_bf16": ({k: (round(v, 3) if isinstance(v, float) else v) for k, v in ratio.items()}
                          if ratio else None),
        "ffn_step": ffn,
        "pages_microbench": micro,
        "lhs_quant_variants": variants,
        "tgmm_dense_baseline": dense,
        "tgmm_grad_dtypes": tgmm_grad,
        "sclk_during_steps": sclk,
        "vendor_dense": vendor,
        "skinny_groups": skinny,
        "small_configs": small,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
