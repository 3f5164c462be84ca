"""Benchmark of the group-wise fake-quant linear hot path on one MI355X.

One step = one pass of every operation of the path over one batch:
  min-max init -> fake-quant forward -> straight-through backward
  (dX, dW, ds, dz) -> pack -> E2E-QP dequant-GEMM forward -> E2E-QP backward
  (dX, ds),
on the Llama-2-7B q_proj workload: fp32 W 4096x4096 ~N(0, 0.02) with 0.1% x10
outliers, w2g64, X 2048x4096 bf16 ~N(0,1) with 8 outlier channels x20,
dY ~N(0, 1e-3). Inputs are resident in HBM before the timed region.

value = the metric as named: the fake-quant linear's forward + backward,
6*M*in*out = 206.16 GFLOP, divided by the median over the timed steps of the
GPU time from the start of the forward to the end of the backward (events
between the calls of each step). The whole step (all rows, with init, pack
and the E2E-QP pair) is reported beside it.

Per-kernel times come from the library's timing, whose events are bound to
each kernel's own dispatch (no extra packets on the stream), so they agree
with a rocprofv3 kernel trace. The roofline object covers the kernel with the
most device time per step, timed that way inside the timed region. Its
`traffic` comes from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
under profiles/, used only while the kernel sources still hash to the value
recorded there.

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
TARGET_MFMA_FRAC = 0.60        # the GEMM target: 60% of the dense bf16 peak
TARGET_HBM_FRAC = 0.70         # the HBM target for init, pack and the staging kernels
KERNEL_SOURCES = ["weight_quantization_aware_amd/csrc/qat_gemm_kernel.h", "weight_quantization_aware_amd/csrc/qat_dma.h",
                  "weight_quantization_aware_amd/csrc/qat_gemm.hip",
                  "weight_quantization_aware_amd/csrc/qat_elementwise.hip",
                  "weight_quantization_aware_amd/csrc/qat_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_q_proj_w2g64.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="least host time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region run one 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--deploy-only", action="store_true",
                    help="only the inference linear on the deployment format (Llama-2-70B block, M = 1 and 16)")
    ap.add_argument("--deploy-gate", action="store_true",
                    help="only the inference linear on the Llama-2-70B gate (28672 x 8192) at M = 1, w2 and w4, "
                         "8 calls each (the shape its counters in profiles/ cover)")
    ap.add_argument("--block-only", action="store_true",
                    help="only one Block-AP step on a Llama-2-7B block (2 x 2048 tokens, w2g64)")
    ap.add_argument("--configs-only", action="store_true",
                    help="only the other workloads (C1 latency, C3 block, C4 E2E-QP MLP, C5 70B gate + down)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the context measurements (practical peaks, the other workloads, cold HBM, "
                         "group sizes, inference linear, Block-AP step)")
    return ap.parse_args()


def note(msg: str) -> None:
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sources_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stats_ms(ts):
    """median, min and interquartile range of times in ms."""
    a = np.asarray(ts, np.float64)
    q25, q50, q75 = np.percentile(a, [25, 50, 75])
    return {"median_ms": round(float(q50), 5), "min_ms": round(float(a.min()), 5),
            "iqr_ms": round(float(q75 - q25), 5), "n": int(a.size)}


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


class Gpu:
    """Event timing helpers on one stream."""

    def __init__(self, torch, dev, stream, Q):
        self.torch, self.dev, self.stream, self.Q = torch, dev, stream, Q
        self._flush_buf = None

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def sync(self):
        self.torch.cuda.synchronize(self.dev)

    def per_call(self, fn, reps):
        """GPU time of each of `reps` calls (ms), each between its own event pair,
        queued back to back."""
        fn()
        self.sync()
        evs = [(self.ev(), self.ev()) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
        self.sync()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    def flush(self):
        """Evict L2 and the 256 MiB MALL: read a 1 GiB buffer (no dirty lines left)."""
        if self._flush_buf is None:
            self._flush_buf = self.torch.ones(1 << 28, dtype=self.torch.float32, device=self.dev)
            self._flush_scratch = self.torch.empty(2048 * 256, device=self.dev)
        self.Q.peak_read(self._flush_buf, 2048, self._flush_scratch)

    def kernel_ms(self, label, fn, reps, cold):
        """Duration of the library kernel `label` inside fn(), from events bound to
        its dispatch; cold: caches flushed before every call."""
        Q = self.Q
        ts = []
        fn()
        self.sync()
        for _ in range(reps):
            if cold:
                self.flush()
            self.sync()
            Q.timing_select(label)
            Q.timing_enable(True)
            fn()
            self.sync()
            Q.timing_enable(False)
            Q.timing_select(None)
            ms, n = Q.timing_report()[label]
            ts.append(ms / n)
        return ts

    def release(self):
        self._flush_buf = None
        self._flush_scratch = None


def bf16_dev(torch, dev, bits_np):
    return torch.from_numpy(np.ascontiguousarray(bits_np).view(np.int16)).view(torch.bfloat16).to(dev)


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
    stream = torch.cuda.current_stream(dev)
    g = Gpu(torch, dev, stream, Q)
    if args.deploy_gate:
        print(json.dumps({"inference_linear_70b_gate_m1": deploy_gate(Q, torch, dev, args.copy_calibration)}),
              flush=True)
        return
    if args.deploy_only:
        print(json.dumps({"inference_linear_70b_block": deploy_measurements(Q, torch, dev, stream)}), flush=True)
        if args.copy_calibration:        # a plain copy of known size for the HBM counters
            a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
            torch.empty_like(a).copy_(a)
            torch.cuda.synchronize(dev)
        return
    if args.block_only:
        print(json.dumps({"block_ap_step_7b": block_step_measurements(Q, torch, dev, stream)}), flush=True)
        return
    if args.configs_only:
        print(json.dumps(other_workloads(Q, torch, dev, g, synth)), flush=True)
        return

    lin = synth.config(2)[0]
    M, out, inp, bits = lin.m, lin.out, lin.inp, lin.bits
    G = inp // 64
    W_np, X_np, dY_np = lin.W(), lin.X(), lin.dY()

    W = torch.from_numpy(W_np).to(dev)
    X = bf16_dev(torch, dev, X_np)
    dY = bf16_dev(torch, dev, dY_np)
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

    def step():
        for _, f in calls:
            f()

    for _ in range(args.warmup):
        step()
    g.sync()
    note(f"warm-up done ({args.warmup} steps)")

    # ---- per-kernel table: every launch of K steps timed by its own dispatch
    Q.timing_enable(True)
    for _ in range(args.steps):
        step()
    g.sync()
    Q.timing_enable(False)
    kernels = Q.timing_report()
    dom = max(kernels, key=lambda k: kernels[k][0])      # most device time per step

    # ---- timed region: K whole steps between two events; inside each step two
    # events around the fake-quant forward + backward; the dominant kernel's
    # launches carry dispatch-bound events (no extra packets)
    e_fq = [(g.ev(), g.ev()) for _ in range(args.steps)]
    e0, e1 = g.ev(), g.ev()
    Q.timing_select(dom)
    Q.timing_enable(True)
    g.sync()
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(args.steps):
        calls[0][1]()
        e_fq[k][0].record(stream)
        calls[1][1]()
        calls[2][1]()
        e_fq[k][1].record(stream)
        for _, f in calls[3:]:
            f()
    e1.record(stream)
    g.sync()
    wall = time.perf_counter() - t0
    Q.timing_enable(False)
    Q.timing_select(None)
    dom_ms, dom_n = Q.timing_report()[dom]
    ms_step = e0.elapsed_time(e1) / args.steps
    fq_ms = [a.elapsed_time(b) for a, b in e_fq]
    fq_stats = stats_ms(fq_ms)

    flops_fq = 6.0 * M * inp * out
    flops_step = flops_fq + 6.0 * M * inp * out                # + E2E-QP forward, dX and ds
    value = flops_fq / (fq_stats["median_ms"] * 1e-3) / 1e12
    note(f"timed region: {ms_step:.4f} ms per step, fake-quant fwd+bwd {value:.1f} TFLOP/s")

    # ---- per-call breakdown: events between the calls of each step
    ev = [[g.ev() for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record(stream)
        for i, (_, f) in enumerate(calls):
            f()
            ev[k][i + 1].record(stream)
    g.sync()
    breakdown = {name: stats_ms([ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)])
                 for i, (name, _) in enumerate(calls)}
    for name, fl in (("fq_fwd", 2), ("fq_bwd", 4), ("e2e_fwd", 2), ("e2e_bwd", 4)):
        breakdown[name]["tflops"] = round(fl * M * inp * out / (breakdown[name]["median_ms"] * 1e-3) / 1e12, 1)

    # ---- per-kernel table (dispatch-bound events)
    ktab = {}
    for label, (tot_ms, n) in kernels.items():
        kind, work = work_per_launch(label, M, out, inp, bits)
        avg_s = tot_ms / n * 1e-3
        rate = work / avg_s / (1e12 if kind == "mfma" else 1e9)
        ktab[label] = {"launches_per_step": n / args.steps, "avg_us": round(avg_s * 1e6, 2),
                       ("tflops" if kind == "mfma" else "gbs_warm"): round(rate, 1),
                       "frac_of_peak": round(rate / (MFMA_BF16_PEAK_TFLOPS if kind == "mfma" else HBM_PEAK_GBS), 4),
                       "share": round(tot_ms / sum(t for t, _ in kernels.values()), 4)}

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
                "avg_us": round(avg_s * 1e6, 2), "launches_timed": dom_n, "work_per_launch": work,
                "timing": "events bound to the kernel's dispatch (hipExtLaunchKernel), live in the timed region"}

    # ---- HBM-bound kernels with cold caches (the result) and warm (context)
    hbm = {}
    for label, fn in (("init_minmax", calls[0][1]), ("quant_w_hat", calls[1][1]), ("pack", calls[3][1]),
                      ("dequant", calls[4][1])):
        _, nbytes = work_per_launch(label, M, out, inp, bits)
        cold = stats_ms(g.kernel_ms(label, fn, 100, True))
        warm_us = ktab[label]["avg_us"]
        hbm[label] = {"cold": cold, "gbs": round(nbytes / (cold["median_ms"] * 1e-3) / 1e9, 1),
                      "frac_of_peak": round(nbytes / (cold["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "warm_us": warm_us, "gbs_warm": round(nbytes / (warm_us * 1e-6) / 1e9, 1),
                      "bytes": nbytes}

    note("cold HBM kernels done")
    # ---- the no-workspace variants at the same workload (bit-identical outputs)
    nows = {}
    Yf = torch.empty_like(Y)
    t = stats_ms(g.per_call(lambda: Q.qat_fakequant_linear_fwd(X, W, s, z, bits, Yf, ws=None), 100))
    nows["fq_fwd_fused_fp32"] = dict(t, tflops=round(2 * M * inp * out / (t["median_ms"] * 1e-3) / 1e12, 1),
                                     bit_identical=bool(torch.equal(Yf, Y)))
    dXf = torch.empty_like(dX)
    t = stats_ms(g.per_call(lambda: Q.qat_fakequant_linear_bwd(dY, X, W, s, z, bits, dX=dXf), 100))
    nows["fq_dx_fused_fp32"] = dict(t, tflops=round(2 * M * inp * out / (t["median_ms"] * 1e-3) / 1e12, 1),
                                    bit_identical=bool(torch.equal(dXf, dX)))
    Q.qat_dequant_gemm_fwd(X, Wq, s, zp, bits, Y2, ws=ws)
    t = stats_ms(g.per_call(lambda: Q.qat_dequant_gemm_fwd(X, Wq, s, zp, bits, Yf), 100))
    nows["e2e_fwd_fused_packed"] = dict(t, tflops=round(2 * M * inp * out / (t["median_ms"] * 1e-3) / 1e12, 1),
                                        bit_identical=bool(torch.equal(Yf, Y2)))
    Q.qat_dequant_gemm_bwd_s_saved(dY, X, Wq, s, zp, ws, bits, ds2, dX=dX2)
    t = stats_ms(g.per_call(lambda: Q.qat_dequant_gemm_bwd_s(dY, X, Wq, s, zp, bits, ds2, dX=dXf), 100))
    nows["e2e_dx_ds_fused_packed"] = dict(t, tflops=round(4 * M * inp * out / (t["median_ms"] * 1e-3) / 1e12, 1),
                                          bit_identical=bool(torch.equal(dXf, dX2)))
    del Yf, dXf

    if args.copy_calibration:            # a plain copy of known size for the HBM counters
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        g.sync()
        del a, b

    extras = None
    if not args.no_extras:
        extras = {"measured_peaks": measured_peaks(Q, torch, dev, g)}
        note("measured peaks done")
        extras["q_proj_fwd_bwd_by_group"] = by_group(Q, torch, dev, g, W, X, dY, bits)
        del W, X, dY, dW, Wq, ws, Y, Y2, dX, dX2
        torch.cuda.empty_cache()
        extras.update(other_workloads(Q, torch, dev, g, synth))
        extras["inference_linear_70b_block"] = deploy_measurements(Q, torch, dev, stream)
        note("inference linear done")
        extras["block_ap_step_7b"] = block_step_measurements(Q, torch, dev, stream)
        note("Block-AP step done")
        extras["clocks"] = _clocks()
        roofline["frac_of_measured_peak"] = round(
            achieved / (extras["measured_peaks"]["mfma_bf16_tflops"] if kind == "mfma"
                        else extras["measured_peaks"]["hbm_read_gbs"]), 4)
        # each HBM-bound kernel against the time its reads and writes take at
        # the measured stream rates (reads at the read peak, writes at the write peak)
        pk = extras["measured_peaks"]
        for label, row in hbm.items():
            rd, wr = rw_bytes(label, out, inp, bits)
            t_floor = rd / (pk["hbm_read_gbs"] * 1e9) + wr / (pk["hbm_write_gbs"] * 1e9)
            row["frac_of_measured_rw"] = round(t_floor / (row["cold"]["median_ms"] * 1e-3), 4)
            row["frac_of_measured_rw_warm"] = round(t_floor / (row["warm_us"] * 1e-6), 4)
    g.release()

    cpu = None
    if not args.no_cpu_baseline:
        note("oracle on the host")
        cpu = cpu_baseline(lin, W_np, X_np, dY_np, args.cpu_seconds)

    line = {
        "metric": "fake-quant linear fwd+bwd TFLOP/s (w2g64, Llama-2-7B shapes); % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Llama-2-7B q_proj shapes, no dataset or checkpoint)",
        "config": {"workload": "llama2-7b q_proj 4096x4096, 2048 tokens, w2g64: init + fake-quant "
                               "fwd/bwd + pack + E2E-QP fwd/bwd per step; value over the fake-quant fwd+bwd",
                   "M": M, "out": out, "in": inp, "bits": bits, "group": 64},
        "value_frac_of_mfma_peak": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "fq_fwd_bwd": dict(fq_stats, gflop=round(flops_fq / 1e9, 2),
                           budget_ms_at_60pct=round(flops_fq / (TARGET_MFMA_FRAC * MFMA_BF16_PEAK_TFLOPS * 1e9), 4)),
        "step_all_rows_tflops": round(flops_step / (ms_step * 1e-3) / 1e12, 2),
        "breakdown": breakdown,
        "kernels": ktab,
        "hbm_kernels": hbm,
        "no_workspace": nows,
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


def measured_peaks(Q, torch, dev, g):
    """Practical peaks on this GPU: a register-resident bf16 MFMA loop, and a
    read stream and a write stream over 1 GiB (beyond the 256 MiB MALL);
    medians of 5 / 10 / 10."""
    blocks = 256
    scratch = torch.empty(max(Q.lib().qat_peak_scratch_bytes(2048) // 4, 2048 * 256), device=dev)
    flops = Q.lib().qat_peak_mfma_flops(blocks, 4096)
    t = np.median(g.per_call(lambda: Q.peak_mfma(blocks, 4096, scratch), 5)) * 1e-3
    big = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    tr = np.median(g.per_call(lambda: Q.peak_read(big, 2048, scratch), 10)) * 1e-3
    tw = np.median(g.per_call(lambda: Q.peak_write(big, 2048), 10)) * 1e-3
    return {"mfma_bf16_tflops": round(flops / t / 1e12, 1), "hbm_read_gbs": round((1 << 30) / tr / 1e9, 1),
            "hbm_write_gbs": round((1 << 30) / tw / 1e9, 1),
            "what": "register-resident v_mfma_f32_16x16x32_bf16 loop, 8 waves per CU; grid-stride read and "
                    "grid-stride write of 1 GiB"}


def rw_bytes(label, out, inp, bits):
    """(read, written) bytes of one launch of an HBM-bound kernel; they add up
    to work_per_launch's bytes."""
    G = inp // 64
    n = out * inp
    if label == "init_minmax":
        return n * 4, 2 * out * G * 4
    if label in ("quant_w_hat", "quant_w_hat_t"):
        return n * 4 + 2 * out * G * 4, n * 2
    if label == "pack":
        return n * 4 + 2 * out * G * 4, n * bits / 8 + out * G * 4
    if label in ("dequant", "dequant_t"):
        return n * bits / 8 + 2 * out * G * 4, n * 2
    raise KeyError(label)


def by_group(Q, torch, dev, g, W, X, dY, bits):
    """The q_proj fake-quant forward + backward at groups of 32, 64, 128 and
    channel-wise (one group per row)."""
    M, out, inp = X.shape[0], W.shape[0], W.shape[1]
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits), dev)
    Y = torch.empty(M, out, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, inp, dtype=torch.bfloat16, device=dev)
    dW = torch.empty(out, inp, device=dev)
    res = {}
    for gname, gsize in (("32", 32), ("64", 64), ("128", 128), ("row", inp)):
        sg = torch.empty(out, inp // gsize, device=dev)
        zg = torch.empty_like(sg)
        dsg, dzg = torch.empty_like(sg), torch.empty_like(sg)
        Q.qat_init_minmax(W, bits, sg, zg, group=gsize)

        def fq(sg=sg, zg=zg, dsg=dsg, dzg=dzg, gsize=gsize):
            Q.qat_fakequant_linear_fwd(X, W, sg, zg, bits, Y, ws=ws, group=gsize)
            Q.qat_fakequant_linear_bwd_saved(dY, X, W, sg, zg, ws, bits, dX=dX, dW=dW, ds=dsg, dz=dzg, group=gsize)
        t = stats_ms(g.per_call(fq, 100))
        res[gname] = dict(t, tflops=round(6.0 * M * inp * out / (t["median_ms"] * 1e-3) / 1e12, 1))
    return res


def _rate(flops, t):
    tf = flops / (t["median_ms"] * 1e-3) / 1e12
    return {"tflops": round(tf, 1), "frac_of_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "budget_ms_at_60pct": round(flops / (TARGET_MFMA_FRAC * MFMA_BF16_PEAK_TFLOPS * 1e9), 4)}


def other_workloads(Q, torch, dev, g, synth):
    """The other workloads, each pass between its own event pair (medians,
    min and IQR over the passes), GEMM FLOPs counted as 6 M in out for a
    forward + backward and 4 M in out for the E2E-QP forward + ds:
    - C1 (256 x 256, 128 tokens, w2g64): GPU time of each call, and the host
      time to issue one (launch latency);
    - C3 (the seven w3g64 linears of a Llama-2-7B block, 2048 tokens):
      fake-quant forward + backward of all seven (staged W_hat, saved for dX);
    - C4 (E2E-QP Llama-2-7B MLP at 4096 tokens, w2g64): forward + dX + ds of
      gate, up and down, with the W_hat workspace and without (fused packed);
    - C5 (Llama-2-70B gate 28672x8192 and down 8192x28672, 4096 tokens) at
      2, 3 and 4 bits: Block-AP fake-quant forward + backward of both, and the
      E2E-QP forward + ds of their packed weights. The same seeded W, X, dY
      serve every bit width (a bit-width sweep of one weight)."""
    res = {}
    # ---- C1: latency
    lin = synth.config(1)[0]
    M, out, inp, b = lin.m, lin.out, lin.inp, lin.bits
    W = torch.from_numpy(lin.W()).to(dev)
    X, dY = bf16_dev(torch, dev, lin.X()), bf16_dev(torch, dev, lin.dY())
    s = torch.empty(out, inp // 64, device=dev)
    z, ds, dz, zp, ds2 = (torch.empty_like(s) for _ in range(5))
    Y, Y2 = (torch.empty(M, out, dtype=torch.bfloat16, device=dev) for _ in range(2))
    dX, dX2 = (torch.empty(M, inp, dtype=torch.bfloat16, device=dev) for _ in range(2))
    dW = torch.empty(out, inp, device=dev)
    Wq = torch.empty(out, inp * b // 8, dtype=torch.uint8, device=dev)
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, b), dev)
    c1 = [("init", lambda: Q.qat_init_minmax(W, b, s, z)),
          ("fq_fwd", lambda: Q.qat_fakequant_linear_fwd(X, W, s, z, b, Y, ws=ws)),
          ("fq_bwd", lambda: Q.qat_fakequant_linear_bwd_saved(dY, X, W, s, z, ws, b, dX=dX, dW=dW, ds=ds, dz=dz)),
          ("pack", lambda: Q.qat_pack(W, s, z, b, Wq, zp)),
          ("e2e_fwd", lambda: Q.qat_dequant_gemm_fwd(X, Wq, s, zp, b, Y2, ws=ws)),
          ("e2e_bwd", lambda: Q.qat_dequant_gemm_bwd_s_saved(dY, X, Wq, s, zp, ws, b, ds2, dX=dX2))]
    r1 = {}
    for name, f in c1:
        t = stats_ms(g.per_call(f, 100))
        g.sync()
        h0 = time.perf_counter()
        for _ in range(200):
            f()
        h1 = time.perf_counter()
        g.sync()
        r1[name] = {"gpu_us_median": round(t["median_ms"] * 1e3, 2), "gpu_us_min": round(t["min_ms"] * 1e3, 2),
                    "host_us_per_call": round((h1 - h0) / 200 * 1e6, 2)}
    step = stats_ms(g.per_call(lambda: [f() for _, f in c1], 100))
    note("C1 latency done")
    res["c1_latency"] = {"what": "256x256 linear, 128 tokens, w2g64; GPU time per call (event pairs) and "
                                 "host time to issue it", "calls": r1,
                         "step_us_median": round(step["median_ms"] * 1e3, 2)}
    del W, X, dY, s, z, ds, dz, zp, ds2, Y, Y2, dX, dX2, dW, Wq, ws

    # ---- C3: the 7B block's seven w3g64 linears
    c3 = []
    for lin in synth.config(3):
        Wc = torch.from_numpy(lin.W()).to(dev)
        Xc, dYc = bf16_dev(torch, dev, lin.X()), bf16_dev(torch, dev, lin.dY())
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
    t = stats_ms(g.per_call(block, 20))
    fl = sum(6.0 * lin.m * lin.inp * lin.out for lin, *_ in c3)
    note("C3 block done")
    res["c3_block_w3g64"] = dict(t, gflop=round(fl / 1e9, 2), **_rate(fl, t))
    del c3, ws3, Y3, dX3, dW3, ds3, dz3
    torch.cuda.empty_cache()

    # ---- C4: E2E-QP MLP at 4096 tokens
    c4 = []
    for lin in synth.config(4):
        c4.append((lin, torch.from_numpy(lin.Wq()).to(dev), torch.from_numpy(lin.s_e2e()).to(dev),
                   torch.from_numpy(lin.z_e2e()).to(dev), bf16_dev(torch, dev, lin.X()),
                   bf16_dev(torch, dev, lin.dY())))
    M4 = c4[0][0].m
    ws4 = Q.workspace(max(Q.dequant_ws_bytes(l.out, l.inp, l.bits) for l, *_ in c4), dev)
    Y4 = torch.empty(M4 * max(l.out for l, *_ in c4), dtype=torch.bfloat16, device=dev)
    dX4 = torch.empty(M4 * max(l.inp for l, *_ in c4), dtype=torch.bfloat16, device=dev)
    ds4 = torch.empty(max(l.out * (l.inp // 64) for l, *_ in c4), device=dev)

    def mlp(staged):
        for lin, Wq4, s4, z4, X4, dY4 in c4:
            o, i = lin.out, lin.inp
            dsv = ds4[:o * (i // 64)].view(o, i // 64)
            if staged:
                Q.qat_dequant_gemm_fwd(X4, Wq4, s4, z4, lin.bits, Y4[:M4 * o].view(M4, o), ws=ws4)
                Q.qat_dequant_gemm_bwd_s_saved(dY4, X4, Wq4, s4, z4, ws4, lin.bits, dsv, dX=dX4[:M4 * i].view(M4, i))
            else:
                Q.qat_dequant_gemm_fwd(X4, Wq4, s4, z4, lin.bits, Y4[:M4 * o].view(M4, o))
                Q.qat_dequant_gemm_bwd_s(dY4, X4, Wq4, s4, z4, lin.bits, dsv, dX=dX4[:M4 * i].view(M4, i))
    fl = sum(6.0 * lin.m * lin.inp * lin.out for lin, *_ in c4)
    t = stats_ms(g.per_call(lambda: mlp(True), 20))
    tf = stats_ms(g.per_call(lambda: mlp(False), 20))
    note("C4 E2E-QP MLP done")
    res["c4_e2e_mlp_w2g64"] = {"gflop": round(fl / 1e9, 2), "staged": dict(t, **_rate(fl, t)),
                               "fused_no_workspace": dict(tf, **_rate(fl, tf))}
    del c4, ws4, Y4, dX4, ds4
    torch.cuda.empty_cache()

    # ---- C5: the 70B gate and down at 2, 3, 4 bits
    lins = synth.config(5, 2)
    data = []
    for lin in lins:
        data.append((lin, torch.from_numpy(lin.W()).to(dev), bf16_dev(torch, dev, lin.X()),
                     bf16_dev(torch, dev, lin.dY())))
    M5 = lins[0].m
    big_o = max(l.out for l in lins)
    big_i = max(l.inp for l in lins)
    ws5 = Q.workspace(max(Q.fakequant_ws_bytes(l.out, l.inp, 4) for l in lins), dev)
    Y5 = torch.empty(M5 * big_o, dtype=torch.bfloat16, device=dev)
    dX5 = torch.empty(M5 * big_i, dtype=torch.bfloat16, device=dev)
    dW5 = torch.empty(max(l.out * l.inp for l in lins), device=dev)
    c5 = {}
    fl_bap = sum(6.0 * l.m * l.inp * l.out for l in lins)
    fl_e2e = sum(4.0 * l.m * l.inp * l.out for l in lins)
    for b in (2, 3, 4):
        qp = []
        for lin, W5, X5, dY5 in data:
            o, i = lin.out, lin.inp
            s5 = torch.empty(o, i // 64, device=dev)
            z5, ds5, dz5, zp5 = (torch.empty_like(s5) for _ in range(4))
            Q.qat_init_minmax(W5, b, s5, z5)
            Wq5 = torch.empty(o, i * b // 8, dtype=torch.uint8, device=dev)
            Q.qat_pack(W5, s5, z5, b, Wq5, zp5)
            qp.append((lin, W5, X5, dY5, s5, z5, ds5, dz5, zp5, Wq5))

        def block_ap(b=b, qp=qp):
            for lin, W5, X5, dY5, s5, z5, ds5, dz5, zp5, Wq5 in qp:
                o, i = lin.out, lin.inp
                Q.qat_fakequant_linear_fwd(X5, W5, s5, z5, b, Y5[:M5 * o].view(M5, o), ws=ws5)
                Q.qat_fakequant_linear_bwd_saved(dY5, X5, W5, s5, z5, ws5, b, dX=dX5[:M5 * i].view(M5, i),
                                                 dW=dW5[:o * i].view(o, i), ds=ds5, dz=dz5)

        def e2e(b=b, qp=qp):
            for lin, W5, X5, dY5, s5, z5, ds5, dz5, zp5, Wq5 in qp:
                o, i = lin.out, lin.inp
                Q.qat_dequant_gemm_fwd(X5, Wq5, s5, zp5, b, Y5[:M5 * o].view(M5, o), ws=ws5)
                Q.qat_dequant_gemm_bwd_s_saved(dY5, X5, Wq5, s5, zp5, ws5, b, ds5)
        tb = stats_ms(g.per_call(block_ap, 20))
        te = stats_ms(g.per_call(e2e, 20))
        note(f"C5 at {b} bits done")
        c5[f"w{b}g64"] = {"block_ap_fwd_bwd": dict(tb, **_rate(fl_bap, tb)), "e2e_fwd_ds": dict(te, **_rate(fl_e2e, te))}
        del qp
    # init and pack of the 896 MiB gate weight, cold
    lin, W5 = data[0][0], data[0][1]
    s5 = torch.empty(lin.out, lin.inp // 64, device=dev)
    z5, zp5 = torch.empty_like(s5), torch.empty_like(s5)
    Wq5 = torch.empty(lin.out, lin.inp * 2 // 8, dtype=torch.uint8, device=dev)
    for label, fn in (("init_minmax", lambda: Q.qat_init_minmax(W5, 2, s5, z5)),
                      ("pack", lambda: Q.qat_pack(W5, s5, z5, 2, Wq5, zp5))):
        _, nbytes = work_per_launch(label, lin.m, lin.out, lin.inp, 2)
        t = stats_ms(g.kernel_ms(label, fn, 20, True))
        c5[f"{label}_cold_gate_w2"] = dict(t, gbs=round(nbytes / (t["median_ms"] * 1e-3) / 1e9, 1),
                                          frac_of_peak=round(nbytes / (t["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    res["c5_70b_gate_down"] = dict(c5, gflop_block_ap=round(fl_bap / 1e9, 2), gflop_e2e_fwd_ds=round(fl_e2e / 1e9, 2))
    del data, ws5, Y5, dX5, dW5, W5, s5, z5, zp5, Wq5
    torch.cuda.empty_cache()
    return res


def deploy_gate(Q, torch, dev, copy_calibration):
    """The inference linear on the Llama-2-70B gate shape (28672 x 8192) at one
    token, w2g64 and w4g64, 8 calls each (mean GPU time per call from an event
    pair around the 8); with copy_calibration a plain 1 GiB device copy follows
    (the reference for FETCH_SIZE)."""
    out, inp = 28672, 8192
    X = torch.randn(1, inp, device=dev).half()
    Y = torch.empty(1, out, dtype=torch.float16, device=dev)
    res = {}
    for bits in (2, 4):
        Wq = torch.randint(0, 256, (out, inp * bits // 8), dtype=torch.uint8, device=dev)
        s16 = (torch.rand(out, inp // 64, device=dev) * 0.05 + 0.002).half()
        zq = torch.randint(0, 256, (out, Q.deploy_zq_stride(inp, bits)), dtype=torch.uint8, device=dev)
        Q.qat_deploy_gemv(X, Wq, s16, zq, bits, Y)
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(8):
            Q.qat_deploy_gemv(X, Wq, s16, zq, bits, Y)
        e1.record()
        torch.cuda.synchronize(dev)
        us = e0.elapsed_time(e1) / 8 * 1e3
        nbytes = Wq.numel() + s16.numel() * 2 + zq.numel() + X.numel() * 2 + Y.numel() * 2
        res[f"w{bits}"] = {"us": round(us, 2), "tbs": round(nbytes / us / 1e6, 2)}
        del Wq, s16, zq
    if copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize(dev)
    return res


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
    # one step with timing on first, so that the event pool holds every
    # label's events before the step that is reported (an event created in
    # the step made its first launch read ~1 ms)
    Q.timing_enable(True)
    step()
    torch.cuda.synchronize(dev)
    Q.timing_enable(True)                # clears the records, keeps the events
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


def cpu_baseline(lin, W_np, X_np, dY_np, seconds):
    """The fp64 oracle timed on the host on the same workload: the fake-quant
    forward + backward of the whole q_proj linear (what `value` measures on
    the GPU), repeated until `seconds` have passed (at least twice); the
    median run is reported."""
    from oracle import qat_oracle as O
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:
        threads = len(os.sched_getaffinity(0))
    M, out, inp, bits = lin.m, lin.out, lin.inp, lin.bits
    s, z = O.init_minmax(W_np, bits)

    def step():
        O.fakequant_fwd(X_np, W_np, s, z, bits)
        O.fakequant_bwd(dY_np, X_np, W_np, s, z, bits)

    ts = []
    t0 = time.perf_counter()
    while len(ts) < 2 or (time.perf_counter() - t0 < seconds and len(ts) < 20):
        a = time.perf_counter()
        step()
        ts.append(time.perf_counter() - a)
    dt = float(np.median(ts))
    flops = 6.0 * M * inp * out
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "blas": blas, "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"the fake-quant forward + backward of the whole q_proj workload ({out}x{inp}, {M} tokens, "
                      f"w2g64), fp64 numpy oracle, {len(ts)} runs, median {dt:.2f} s"}


if __name__ == "__main__":
    main()
