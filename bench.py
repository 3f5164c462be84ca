"""Benchmark of the group-wise fake-quant linear hot path on one MI355X.

One step = one pass of every operation of the path over one batch:
  min-max init -> fake-quant forward -> straight-through backward
  (dX, dW, ds, dz) -> pack -> E2E-QP dequant-GEMM forward -> E2E-QP backward
  (dX, ds),
on the Llama-2-7B q_proj workload: fp32 W 4096x4096 ~N(0, 0.02) with 0.1% x10
outliers, w2g64, X 2048x4096 bf16 ~N(0,1) with 8 outlier channels x20,
dY ~N(0, 1e-3). Inputs are resident in HBM before the timed region.

value = counted GEMM FLOPs of the step / step time, where the count is
6*M*in*out for the fake-quant forward + backward plus 6*M*in*out for the
E2E-QP forward + dX + ds (init and pack add time, no FLOPs).

The roofline object covers the kernel with the largest share of the timed
region, timed live by the library (HIP events around each launch on its
stream). Its `traffic` comes from a committed rocprofv3 FETCH_SIZE /
WRITE_SIZE summary under profiles/, used only while the kernel sources still
hash to the value recorded there.

Prints one JSON line (N = 1 only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["weight_quantization_aware_amd/csrc/qat_gemm_kernel.h", "weight_quantization_aware_amd/csrc/qat_dma.h",
                  "weight_quantization_aware_amd/csrc/qat_gemm.hip",
                  "weight_quantization_aware_amd/csrc/qat_elementwise.hip",
                  "weight_quantization_aware_amd/csrc/qat_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_q_proj_w2g64.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=512, help="weight rows of the bounded oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region run one 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--deploy-only", action="store_true",
                    help="only the inference linear on the deployment format (Llama-2-70B block, M = 1 and 16)")
    ap.add_argument("--block-only", action="store_true",
                    help="only one Block-AP step on a Llama-2-7B block (2 x 2048 tokens, w2g64)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the context measurements (practical peaks, cold HBM, the C3 block)")
    return ap.parse_args()


def sources_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def work_per_launch(label, M, out, inp, bits):
    """Algorithmic work of one launch: ('mfma', flops) or ('hbm', bytes)."""
    G = inp // 64
    n = out * inp
    if label.startswith("gemm"):
        return "mfma", 2.0 * M * inp * out
    if label == "init_minmax":
        return "hbm", n * 4 + 2 * out * G * 4
    if label in ("quant_w_hat", "quant_w_hat_t"):
        return "hbm", n * (4 + 2) + 2 * out * G * 4
    if label == "pack":
        return "hbm", n * (4 + bits / 8) + 3 * out * G * 4
    if label in ("dequant", "dequant_t"):
        return "hbm", n * (bits / 8 + 2) + 2 * out * G * 4
    return "hbm", float("nan")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from weight_quantization_aware_amd import _lib as Q
    from weight_quantization_aware_amd import synth

    dev = torch.device("cuda:0")
    if args.deploy_only:
        print(json.dumps({"inference_linear_70b_block":
                          deploy_measurements(Q, torch, dev, torch.cuda.current_stream(dev))}), flush=True)
        return
    if args.block_only:
        print(json.dumps({"block_ap_step_7b": block_step_measurements(Q, torch, dev, torch.cuda.current_stream(dev))}),
              flush=True)
        return
    lin = synth.config(2)[0]
    M, out, inp, bits = lin.m, lin.out, lin.inp, lin.bits
    G = inp // 64
    W_np, X_np, dY_np = lin.W(), lin.X(), lin.dY()

    W = torch.from_numpy(W_np).to(dev)
    X = torch.from_numpy(X_np.view(np.int16)).view(torch.bfloat16).to(dev)
    dY = torch.from_numpy(dY_np.view(np.int16)).view(torch.bfloat16).to(dev)
    s = torch.empty(out, G, device=dev)
    z = torch.empty_like(s)
    Y = torch.empty(M, out, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, inp, dtype=torch.bfloat16, device=dev)
    dW = torch.empty(out, inp, device=dev)
    ds = torch.empty_like(s)
    dz = torch.empty_like(s)
    Wq = torch.empty(out, inp * bits // 8, dtype=torch.uint8, device=dev)
    zp = torch.empty_like(s)
    Y2 = torch.empty_like(Y)
    dX2 = torch.empty_like(dX)
    ds2 = torch.empty_like(s)
    ws = Q.workspace(max(Q.fakequant_ws_bytes(out, inp, bits), Q.dequant_ws_bytes(out, inp, bits)), dev)

    calls = [
        ("init", lambda: Q.qat_init_minmax(W, bits, s, z)),
        ("fq_fwd", lambda: Q.qat_fakequant_linear_fwd(X, W, s, z, bits, Y, ws=ws)),
        # the backwards read the W_hat their forward left in ws (autograd's saved tensor)
        ("fq_bwd", lambda: Q.qat_fakequant_linear_bwd_saved(dY, X, W, s, z, ws, bits, dX=dX, dW=dW, ds=ds, dz=dz)),
        ("pack", lambda: Q.qat_pack(W, s, z, bits, Wq, zp)),
        ("e2e_fwd", lambda: Q.qat_dequant_gemm_fwd(X, Wq, s, zp, bits, Y2, ws=ws)),
        ("e2e_bwd", lambda: Q.qat_dequant_gemm_bwd_s_saved(dY, X, Wq, s, zp, ws, bits, ds2, dX=dX2)),
    ]

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize(dev)

    def run_steps(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            for _, f in calls:
                f()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / n

    def kernel_times(label=None):
        Q.timing_select(label)
        Q.timing_enable(True)
        ms = run_steps(args.steps)
        Q.timing_enable(False)
        Q.timing_select(None)
        return ms, Q.timing_report()

    # ---- per-kernel table: every launch of K steps bracketed by HIP events
    ms_step_all_events, kernels = kernel_times()
    dom = max(kernels, key=lambda k: kernels[k][0])      # most device time per step

    # ---- timed region: K whole steps; only the dominant kernel's launches
    # carry HIP events (recorded by the library on the launch stream)
    Q.timing_select(dom)
    Q.timing_enable(True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    ms_step = run_steps(args.steps)
    wall = time.perf_counter() - t0
    Q.timing_enable(False)
    Q.timing_select(None)
    dom_ms, dom_n = Q.timing_report()[dom]

    # ---- the same steps with no kernel events at all
    ms_step_clean = run_steps(args.steps)

    # ---- per-call breakdown: events between the six calls of a step
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record(stream)
        for i, (_, f) in enumerate(calls):
            f()
            ev[k][i + 1].record(stream)
    torch.cuda.synchronize(dev)
    per_call = {name: float(np.mean([ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)]))
                for i, (name, _) in enumerate(calls)}

    flops_fq = 6.0 * M * inp * out
    flops_e2e = 6.0 * M * inp * out
    value = (flops_fq + flops_e2e) / (ms_step * 1e-3) / 1e12

    # ---- per-kernel table (from the all-events pass)
    ktab = {}
    for label, (tot_ms, n) in kernels.items():
        kind, work = work_per_launch(label, M, out, inp, bits)
        avg_s = tot_ms / n * 1e-3
        rate = work / avg_s / (1e12 if kind == "mfma" else 1e9)
        ktab[label] = {"launches_per_step": n / args.steps, "avg_us": round(avg_s * 1e6, 2),
                       ("tflops" if kind == "mfma" else "gbs"): round(rate, 1),
                       "share": round(tot_ms / (ms_step_all_events * args.steps), 4)}

    # ---- the dominant kernel's roofline, from its launches in the timed region
    kind, work = work_per_launch(dom, M, out, inp, bits)
    avg_s = dom_ms / dom_n * 1e-3
    if kind == "mfma":
        achieved, peak, unit = work / avg_s / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = work / avg_s / 1e9, HBM_PEAK_GBS, "GB/s"
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("sources_hash") == sources_hash() and dom in tr.get("kernels", {}):
            traffic = tr["kernels"][dom]["bytes_per_launch"]
    roofline = {"kernel": dom, "bound": "mfma" if kind == "mfma" else "hbm", "achieved": round(achieved, 2),
                "peak": peak, "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
                "avg_us": round(avg_s * 1e6, 2), "launches_timed": dom_n, "work_per_launch": work}

    # ---- the fused fp32 forward (no workspace), timed on its own as evidence
    Yf = torch.empty_like(Y)
    for _ in range(3):
        Q.qat_fakequant_linear_fwd(X, W, s, z, bits, Yf, ws=None)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        Q.qat_fakequant_linear_fwd(X, W, s, z, bits, Yf, ws=None)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    t_fused = e0.elapsed_time(e1) / 10
    fused_same = bool(torch.equal(Yf, Y))

    if args.copy_calibration:            # a plain copy of known size for the HBM counters
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize(dev)

    breakdown = {name: {"ms": round(t, 4)} for name, t in per_call.items()}
    breakdown["fq_fwd"]["tflops"] = round(2 * M * inp * out / (per_call["fq_fwd"] * 1e-3) / 1e12, 1)
    breakdown["fq_bwd"]["tflops"] = round(4 * M * inp * out / (per_call["fq_bwd"] * 1e-3) / 1e12, 1)
    breakdown["e2e_fwd"]["tflops"] = round(2 * M * inp * out / (per_call["e2e_fwd"] * 1e-3) / 1e12, 1)
    breakdown["e2e_bwd"]["tflops"] = round(4 * M * inp * out / (per_call["e2e_bwd"] * 1e-3) / 1e12, 1)
    breakdown["init"]["gbs"] = round(out * inp * 4.125 / (per_call["init"] * 1e-3) / 1e9, 1)
    breakdown["pack"]["gbs"] = round(out * inp * (4.125 + bits / 8) / (per_call["pack"] * 1e-3) / 1e9, 1)
    breakdown["fq_fwd_fused_no_ws"] = {"ms": round(t_fused, 4),
                                       "tflops": round(2 * M * inp * out / (t_fused * 1e-3) / 1e12, 1),
                                       "bit_identical_to_staged": fused_same}
    fq_only = flops_fq / ((per_call["fq_fwd"] + per_call["fq_bwd"]) * 1e-3) / 1e12

    extras = None
    if not args.no_extras:
        extras = context_measurements(Q, torch, dev, stream, W, s, z, Wq, zp, bits, out, inp, X, dY)
        extras["inference_linear_70b_block"] = deploy_measurements(Q, torch, dev, stream)
        extras["block_ap_step_7b"] = block_step_measurements(Q, torch, dev, stream)
        roofline["frac_of_measured_peak"] = round(
            achieved / (extras["measured_peaks"]["mfma_bf16_tflops"] if kind == "mfma"
                        else extras["measured_peaks"]["hbm_read_gbs"]), 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(lin, W_np, X_np, dY_np, args.cpu_rows)

    line = {
        "metric": "fake-quant linear fwd+bwd TFLOP/s (w2g64, Llama-2-7B shapes); % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_without_kernel_events": round(ms_step_clean, 4),
        "ms_per_step_with_all_kernel_events": round(ms_step_all_events, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama2-7b q_proj 4096x4096, 2048 tokens, w2g64: init + fake-quant "
                               "fwd/bwd + pack + E2E-QP fwd/bwd", "M": M, "out": out, "in": inp,
                   "bits": bits, "group": 64},
        "fq_fwd_bwd_tflops": round(fq_only, 2),
        "mfma_peak_frac_fq": round(fq_only / MFMA_BF16_PEAK_TFLOPS, 4),
        "breakdown": breakdown,
        "kernels": ktab,
        "wall_s": round(wall, 3),
        "roofline": roofline,
        "context": extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _clocks():
    """SCLK / MCLK as rocm-smi reports them (best effort; None if unavailable)."""
    import shutil
    import subprocess
    exe = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe, "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
        card = next(iter(d.values()))
        return {k: v for k, v in card.items() if "clock" in k.lower() and ("sclk" in k.lower() or "mclk" in k.lower())}
    except Exception:
        return None


def context_measurements(Q, torch, dev, stream, W, s, z, Wq, zp, bits, out, inp, X, dY):
    """Context beside the headline (not part of `value`):
    - practical peaks on this GPU: a register-resident bf16 MFMA loop and a
      read stream over 1 GiB (beyond the 256 MiB MALL);
    - init and pack with cold caches: before each timed call a 1 GiB buffer is
      read (not written, so no dirty lines are left to write back), which
      evicts W from L2 and the MALL (median of 10); at the q_proj weight
      (64 MiB) and at the Llama-2-70B gate weight (896 MiB);
    - the q_proj fake-quant forward + backward at groups of 32, 64, 128 and
      channel-wise (one group per row);
    - the Llama-2-7B block of seven w3g64 linears (q, k, v, o 4096x4096; gate,
      up 11008x4096; down 4096x11008; 2048 tokens): fake-quant forward +
      backward of all seven, 2486.79 GFLOP counted;
    - the clocks rocm-smi reports."""
    from weight_quantization_aware_amd import synth

    def ev_time(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize(dev)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / reps * 1e-3

    # practical peaks
    blocks = 256
    scratch = torch.empty(max(Q.lib().qat_peak_scratch_bytes(2048) // 4, 2048 * 256), device=dev)
    flops = Q.lib().qat_peak_mfma_flops(blocks, 4096)
    t = ev_time(lambda: Q.peak_mfma(blocks, 4096, scratch), 5)
    mfma_peak = flops / t / 1e12
    big = torch.ones(1 << 28, dtype=torch.float32, device=dev)          # 1 GiB
    t = ev_time(lambda: Q.peak_read(big, 2048, scratch), 10)
    read_peak = (1 << 30) / t / 1e9

    # cold init / pack
    def cold(fn):
        ts = []
        for _ in range(10):
            Q.peak_read(big, 2048, scratch)
            torch.cuda.synchronize(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))
    s2, z2 = torch.empty_like(s), torch.empty_like(z)
    Wq2, zp2 = torch.empty_like(Wq), torch.empty_like(zp)
    t_init = cold(lambda: Q.qat_init_minmax(W, bits, s2, z2))
    t_pack = cold(lambda: Q.qat_pack(W, s, z, bits, Wq2, zp2))
    n = out * inp
    init_bytes = n * 4 + 2 * out * (inp // 64) * 4
    pack_bytes = n * (4 + bits / 8) + 3 * out * (inp // 64) * 4
    del s2, z2, Wq2, zp2

    # the same at the Llama-2-70B gate weight (28672 x 8192 fp32, 896 MiB, w2)
    lin5 = synth.config(5, 2)[0]
    W5 = torch.from_numpy(lin5.W()).to(dev)
    G5 = lin5.inp // 64
    s5 = torch.empty(lin5.out, G5, device=dev)
    z5 = torch.empty_like(s5)
    Wq5 = torch.empty(lin5.out, lin5.inp * 2 // 8, dtype=torch.uint8, device=dev)
    zp5 = torch.empty_like(s5)
    Q.qat_init_minmax(W5, 2, s5, z5)
    t_init5 = cold(lambda: Q.qat_init_minmax(W5, 2, s5, z5))
    t_pack5 = cold(lambda: Q.qat_pack(W5, s5, z5, 2, Wq5, zp5))
    n5 = lin5.out * lin5.inp
    init5_bytes = n5 * 4 + 2 * lin5.out * G5 * 4
    pack5_bytes = n5 * (4 + 2 / 8) + 3 * lin5.out * G5 * 4
    del W5, s5, z5, Wq5, zp5, big

    # the q_proj step's fake-quant forward + backward at the other group sizes
    groups = {}
    M2, out2, in2 = X.shape[0], W.shape[0], W.shape[1]
    ws2 = Q.workspace(Q.fakequant_ws_bytes(out2, in2, bits), dev)
    Y2 = torch.empty(M2, out2, dtype=torch.bfloat16, device=dev)
    dX2 = torch.empty(M2, in2, dtype=torch.bfloat16, device=dev)
    dW2 = torch.empty(out2, in2, device=dev)
    for gname, gsize in (("32", 32), ("64", 64), ("128", 128), ("row", in2)):
        sg = torch.empty(out2, in2 // gsize, device=dev)
        zg = torch.empty_like(sg)
        dsg, dzg = torch.empty_like(sg), torch.empty_like(sg)
        Q.qat_init_minmax(W, bits, sg, zg, group=gsize)

        def fq(sg=sg, zg=zg, dsg=dsg, dzg=dzg, gsize=gsize):
            Q.qat_fakequant_linear_fwd(X, W, sg, zg, bits, Y2, ws=ws2, group=gsize)
            Q.qat_fakequant_linear_bwd_saved(dY, X, W, sg, zg, ws2, bits, dX=dX2, dW=dW2, ds=dsg, dz=dzg,
                                             group=gsize)
        tg = ev_time(fq, 10)
        groups[gname] = {"ms": round(tg * 1e3, 4), "tflops": round(6.0 * M2 * in2 * out2 / tg / 1e12, 1)}
    del ws2, Y2, dX2, dW2

    # the C3 block
    c3 = []
    for lin in synth.config(3):
        Wc = torch.from_numpy(lin.W()).to(dev)
        Xc = torch.from_numpy(lin.X().view(np.int16)).view(torch.bfloat16).to(dev)
        dYc = torch.from_numpy(lin.dY().view(np.int16)).view(torch.bfloat16).to(dev)
        sc = torch.empty(lin.out, lin.inp // 64, device=dev)
        zc = torch.empty_like(sc)
        Q.qat_init_minmax(Wc, lin.bits, sc, zc)
        c3.append((lin, Wc, Xc, dYc, sc, zc))
    M3 = c3[0][0].m
    ws3 = Q.workspace(max(Q.fakequant_ws_bytes(l.out, l.inp, l.bits) for l, *_ in c3), dev)
    Y3 = torch.empty(M3 * max(l.out for l, *_ in c3), dtype=torch.bfloat16, device=dev)
    dX3 = torch.empty(M3 * max(l.inp for l, *_ in c3), dtype=torch.bfloat16, device=dev)
    dW3 = torch.empty(max(l.out * l.inp for l, *_ in c3), device=dev)
    ds3 = torch.empty(max(l.out * (l.inp // 64) for l, *_ in c3), device=dev)
    dz3 = torch.empty_like(ds3)

    def block():
        for lin, Wc, Xc, dYc, sc, zc in c3:
            o, i = lin.out, lin.inp
            Q.qat_fakequant_linear_fwd(Xc, Wc, sc, zc, lin.bits, Y3[:M3 * o].view(M3, o), ws=ws3)
            Q.qat_fakequant_linear_bwd_saved(dYc, Xc, Wc, sc, zc, ws3, lin.bits, dX=dX3[:M3 * i].view(M3, i),
                                             dW=dW3[:o * i].view(o, i), ds=ds3[:o * (i // 64)].view(o, i // 64),
                                             dz=dz3[:o * (i // 64)].view(o, i // 64))
    t_c3 = ev_time(block, 5)
    gflop = sum(6.0 * lin.m * lin.inp * lin.out for lin, *_ in c3) / 1e9
    return {
        "measured_peaks": {"mfma_bf16_tflops": round(mfma_peak, 1), "hbm_read_gbs": round(read_peak, 1),
                           "what": "register-resident v_mfma_f32_16x16x32_bf16 loop, 8 waves per CU; "
                                   "grid-stride read of 1 GiB"},
        "init_cold": {"us": round(t_init * 1e6, 2), "gbs": round(init_bytes / t_init / 1e9, 1)},
        "pack_cold": {"us": round(t_pack * 1e6, 2), "gbs": round(pack_bytes / t_pack / 1e9, 1)},
        "init_cold_70b_gate": {"us": round(t_init5 * 1e6, 2), "gbs": round(init5_bytes / t_init5 / 1e9, 1)},
        "pack_cold_70b_gate_w2": {"us": round(t_pack5 * 1e6, 2), "gbs": round(pack5_bytes / t_pack5 / 1e9, 1)},
        "c3_block_w3g64": {"gflop": round(gflop, 2), "ms": round(t_c3 * 1e3, 4),
                           "tflops": round(gflop / t_c3 / 1e3, 1)},
        "q_proj_fwd_bwd_by_group": groups,
        "clocks": _clocks(),
    }


def deploy_measurements(Q, torch, dev, stream):
    """The inference linear on the deployment format (fp16 step sizes, N-bit
    zero points) for one token (M = 1) and for 16, over the seven linears of a
    Llama-2-70B block at w2g64 and w4g64, against torch's fp16 linear on the
    same shapes (the comparison the EfficientQAT pages make for INT2). Each
    figure is the median GPU time of 20 calls, every call between its own
    event pair, all queued behind a GPU sleep so that host launch overhead
    does not enter; TB/s counts codes, s16, zq, X and Y."""
    from weight_quantization_aware_amd import synth

    def gpu_med_us(fn, reps=20):
        fn()
        torch.cuda.synchronize(dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda._sleep(5_000_000)
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize(dev)
        t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        return t[len(t) // 2] * 1e3

    res = {"what": "deployed Llama-2-70B block, group 64; us = median GPU time per call", "linears": {}}
    tot = {}
    for name, out, inp in synth.DEPLOY_SHAPES["70b"]:
        row = {"out": out, "in": inp}
        for M in (1, 16):
            X = torch.randn(M, inp, device=dev).half()
            Y = torch.empty(M, out, dtype=torch.float16, device=dev)
            W16 = torch.randn(out, inp, device=dev).half()
            t16 = gpu_med_us(lambda: torch.nn.functional.linear(X, W16))
            del W16
            row[f"fp16_M{M}_us"] = round(t16, 2)
            tot[f"fp16_M{M}"] = tot.get(f"fp16_M{M}", 0.0) + t16
            for bits in (2, 4):
                Wq = torch.randint(0, 256, (out, inp * bits // 8), dtype=torch.uint8, device=dev)
                s16 = (torch.rand(out, inp // 64, device=dev) * 0.05 + 0.002).half()
                zq = torch.randint(0, 256, (out, Q.deploy_zq_stride(inp, bits)), dtype=torch.uint8, device=dev)
                t = gpu_med_us(lambda: Q.qat_deploy_gemv(X, Wq, s16, zq, bits, Y))
                nbytes = Wq.numel() + s16.numel() * 2 + zq.numel() + X.numel() * 2 + Y.numel() * 2
                row[f"w{bits}_M{M}"] = {"us": round(t, 2), "tbs": round(nbytes / t / 1e6, 2)}
                tot[f"w{bits}_M{M}"] = tot.get(f"w{bits}_M{M}", 0.0) + t
        res["linears"][name] = row
    res["block"] = {k: round(v, 1) for k, v in tot.items()}
    for M in (1, 16):
        for bits in (2, 4):
            res["block"][f"speedup_w{bits}_M{M}_vs_fp16"] = round(tot[f"fp16_M{M}"] / tot[f"w{bits}_M{M}"], 2)
    return res


def block_step_flops(H, nh, I, T, Bn):
    """GEMM FLOPs of one Block-AP step as the kernels compute them: the seven
    linears' forward and weight-gradient products, the dX products of o, gate,
    up and down (the block input's gradient is not needed), and the six
    attention products per (sequence, head) over full T x T score tiles."""
    from weight_quantization_aware_amd import synth
    shapes = synth.block_linear_shapes(H, I)
    BT = Bn * T
    lin = 2.0 * BT * sum(o * i for _, o, i in shapes)
    dx = 2.0 * BT * sum(o * i for n, o, i in shapes if n not in ("q_proj", "k_proj", "v_proj"))
    attn = 6 * 2.0 * Bn * nh * T * T * (H // nh)
    return {"linears": 2 * lin + dx, "attention": attn}


def block_step_measurements(Q, torch, dev, stream, steps=10):
    """One Block-AP step (include/qat_block.h) on a Llama-2-7B block: 2
    sequences of 2048 tokens, w2g64, seeded synthetic inputs (synth.block_inputs),
    s and z from the library's min-max init, no dW buffer (W's AdamW runs in
    the epilogue of its gradient product). Whole steps between events
    (parameters and moments advance from step to step, as in training), then
    one step with the library's per-launch events for the kernel table."""
    from weight_quantization_aware_amd import synth
    H, nh, I, T, Bn = synth.BLOCK_7B
    bits, group = 2, 64
    d = synth.block_inputs(6, H, I, Bn * T)
    shape = Q.block_shape(H, nh, I, T, Bn, bits, group)
    lins = []
    for n, o, i in synth.block_linear_shapes(H, I):
        W = torch.from_numpy(d["W"][n]).to(dev)
        sz = torch.empty(o, i // group, device=dev)
        zz = torch.empty_like(sz)
        Q.qat_init_minmax(W, bits, sz, zz, group=group)
        e = {"W": W, "s": sz, "z": zz}
        for k in ("W", "s", "z"):
            if k != "W":             # dW is not needed by the update at group 64
                e["d" + k] = torch.empty_like(e[k])
            e["m_" + k] = torch.zeros_like(e[k])
            e["v_" + k] = torch.zeros_like(e[k])
        lins.append(e)
    del d["W"]
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    tgt = torch.from_numpy(d["target"].view(np.int16)).view(torch.bfloat16).to(dev)
    g1, g2 = torch.from_numpy(d["g1"]).to(dev), torch.from_numpy(d["g2"]).to(dev)
    ws = Q.workspace(Q.block_ws_bytes(shape), dev)
    loss = torch.empty(1, device=dev)
    opt = {"lr_weight": 2e-5, "lr_quant": 1e-4, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.0,
           "step": 0, "total_steps": 4096}
    k = [0]

    def step():
        opt["step"] = k[0]
        Q.qat_block_ap_step(shape, lins, g1, g2, x, tgt, opt, loss, ws=ws)
        k[0] += 1

    for _ in range(2):
        step()
    torch.cuda.synchronize(dev)
    loss0 = float(loss.item())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    Q.timing_enable(True)
    step()
    torch.cuda.synchronize(dev)
    rep = Q.timing_report()
    Q.timing_enable(False)
    fl = block_step_flops(H, nh, I, T, Bn)
    ktab = {lab: {"ms": round(t, 4), "launches": n} for lab, (t, n) in sorted(rep.items(), key=lambda kv: -kv[1][0])}
    ksum = sum(t for t, _ in rep.values())
    for lab in ktab:
        ktab[lab]["share"] = round(ktab[lab]["ms"] / ksum, 4)
    nparam = sum(o * i + 2 * o * (i // group) for _, o, i in synth.block_linear_shapes(H, I))
    nqp = sum(2 * o * (i // group) for _, o, i in synth.block_linear_shapes(H, I))
    if "adamw" in ktab:                  # s and z only
        ktab["adamw"]["gbs"] = round(28.0 * nqp / (ktab["adamw"]["ms"] * 1e-3) / 1e9, 1)
    return {"what": "Llama-2-7B block (hidden 4096, 32 heads, inter 11008), 2 x 2048 tokens, w2g64: forward, "
                    "MSE, straight-through backward, AdamW (two groups, cosine)",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(Bn * T / (ms * 1e-3)),
            "gemm_tflop": round((fl["linears"] + fl["attention"]) / 1e12, 4),
            "gemm_tflops": round((fl["linears"] + fl["attention"]) / (ms * 1e-3) / 1e12, 1),
            "linear_gemm_tflop": round(fl["linears"] / 1e12, 4),
            "loss_after_two_steps": round(loss0, 6), "kernels_one_step": ktab,
            "kernel_sum_ms": round(ksum, 4), "params": nparam}


def cpu_baseline(lin, W_np, X_np, dY_np, rows):
    """The fp64 oracle timed on the host on a bounded sample: the same step
    restricted to the first `rows` weight rows (all tokens, all inputs)."""
    from oracle import qat_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    M, inp, bits = lin.m, lin.inp, lin.bits
    W = W_np[:rows]
    dY = dY_np[:, :rows].copy()

    def step():
        s, z = O.init_minmax(W, bits)
        O.fakequant_fwd(X_np, W, s, z, bits)
        O.fakequant_bwd(dY, X_np, W, s, z, bits)
        Wq, zp = O.pack(W, s, z, bits)
        O.dequant_gemm_fwd(X_np, Wq, s, zp, inp, bits)
        O.dequant_gemm_bwd_s(dY, X_np, Wq, s, zp, inp, bits)

    t0 = time.perf_counter()
    step()
    t1 = time.perf_counter()
    reps = 1
    while time.perf_counter() - t0 < 10.0 and reps < 5:
        step()
        reps += 1
    dt = (time.perf_counter() - t1) / max(reps - 1, 1) if reps > 1 else t1 - t0
    flops = 12.0 * M * inp * rows
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"same step on the first {rows} of {lin.out} weight rows (all {M} tokens, all {inp} "
                      f"inputs), {reps} runs, mean of the timed ones; fp64 numpy"}


if __name__ == "__main__":
    main()
