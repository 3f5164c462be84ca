"""Summaries of rocprofv3 result databases for profiles/.

    python profile_summary.py stats <results.db> [--cmd "..."]
        per-kernel dispatch count and mean / min / max duration (kernel trace)

    python profile_summary.py traffic <fetch.db> <write.db> \
            --copy-bytes N [--cmd "..."]
        per-kernel HBM bytes per launch from a FETCH_SIZE run and a WRITE_SIZE
        run, each scaled by what the same counter reads for the largest
        non-library dispatch of the run (a plain device copy of N bytes), as
        JSON keyed by the library's kernel labels, with the hash of the kernel
        sources it was measured on.

    python profile_summary.py pmc <results.db> [--cmd "..."]
        per-kernel means of the collected counters (summed over dimensions per
        dispatch) and, when present, MFMA utilisation =
        SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) and
        the LDS bank-conflict share SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.
        (GRBM_GUI_ACTIVE is summed over the 8 XCDs: it reads 8x the kernel's
        duration in cycles.)

Reads SQLite databases written by rocprofv3 (ROCm 7); prints to stdout. It
sits beside bench.py, whose runs it summarises; the library does not use it.
"""
from __future__ import annotations

import argparse
import collections
import json
import re
import sqlite3
import sys

# rocprofv3 kernel symbol -> the label the library's own timing uses
# k_gemm<BM, BN, BK, STAGES, WGM, WGN, GM, AMN, BMN, EP, NB>: the last four
# template arguments name it (AMN / BMN: 0, 2 K-contiguous; 1, 3
# MN-contiguous; EP the epilogue; NB the bit width or a tag).
GEMM_RE = re.compile(r"k_gemm<(?:\s*\d+\s*,){7}\s*(\d+)\s*,\s*(\d+)\s*,\s*(\d+)\s*,\s*(\d+)\s*>")
# k_gemm_fused_dx<BM, BN, BL, NB, ADW> (dX), k_gemm_fused_fwd<BM, BN, BL, NB> (forward); BL 1: fp32
# master weight, 2: packed codes
FUSED_DX_RE = re.compile(r"k_gemm_fused_dx<(?:\s*\d+\s*,){2}\s*(\d+)\s*,\s*(\d+)\s*,\s*(\d+)\s*>")
FUSED_FWD_RE = re.compile(r"k_gemm_fused_fwd<(?:\s*\d+\s*,){2}\s*(\d+)\s*,\s*(\d+)\s*>")
LABELS = [
    (r"k_attn_rowdot", "attn_rowdot"),
    (r"k_flash_fwd", "attn_fwd"),
    (r"k_flash_bwd_kv", "attn_bwd_kv"),
    (r"k_init_minmax|k_init_rows", "init_minmax"),
    (r"k_quant_codes", "quant_w_hat"),
    (r"k_w_hat_t<0,", "quant_w_hat_t"),
    (r"k_w_hat_t<1,", "dequant_t"),
    (r"k_pack<", "pack"),
    (r"k_dequant<", "dequant"),
    # inference linear on the deployment format: k_deploy_gemv_lds<N, RW, NB>, k_deploy_gemv<N>
    (r"k_deploy_gemv_lds<2,", "deploy_gemv_w2"),
    (r"k_deploy_gemv_lds<3,", "deploy_gemv_w3"),
    (r"k_deploy_gemv_lds<4,", "deploy_gemv_w4"),
    (r"k_deploy_gemv_xchunk<", "deploy_gemv_xchunk"),
    (r"k_deploy_gemv<2>", "deploy_gemv_xreg_w2"),
    (r"k_deploy_gemv<3>", "deploy_gemv_xreg_w3"),
    (r"k_deploy_gemv<4>", "deploy_gemv_xreg_w4"),
    (r"k_deploy_qparams", "deploy_qparams"),
    # the Block-AP step's row kernels and optimiser
    (r"k_rmsnorm_fwd", "rmsnorm_fwd"),
    (r"k_rmsnorm_bwd", "rmsnorm_bwd"),
    (r"k_rope_table", "rope_table"),
    (r"k_rope\(", "rope"),
    (r"k_swiglu_fwd", "swiglu_fwd"),
    (r"k_swiglu_bwd", "swiglu_bwd"),
    (r"k_loss_final", "loss"),
    (r"k_adamw", "adamw"),
    (r"k_fill_zero", "fill_zero"),
]


def label_of(name: str):
    m = FUSED_FWD_RE.search(name)
    if m:
        return "gemm_fwd_fused_fp32" if int(m.group(1)) == 1 else "gemm_fwd_packed"
    m = FUSED_DX_RE.search(name)
    if m:
        return "gemm_dx_fused_fp32" if int(m.group(1)) == 1 else "gemm_dx_packed"
    m = GEMM_RE.search(name)
    if m:
        amn, bmn, ep, nb = (int(v) for v in m.groups())
        if ep == 1:
            return "gemm_ste_grads"
        if ep == 4:
            return "gemm_ste_grads_adamw"
        if ep == 2:
            return "gemm_e2e_grads"
        if ep == 5:
            return "gemm_fwd_mse"
        if ep == 3:
            return "gemm_fwd_f32"
        if nb == 5:
            return "attn_gemm_bf16"
        return "gemm_dx" if nb == 1 else "gemm_fwd"
    for pat, lab in LABELS:
        if re.search(pat, name):
            return lab
    return None


def stats(db: str, cmd: str) -> None:
    c = sqlite3.connect(db)
    durs = collections.defaultdict(list)
    for name, d in c.execute("select name, end-start from kernels"):
        durs[name].append(d)
    print(f"# rocprofv3 kernel trace summary\n# command: {cmd}\n#")
    print(f"{'label':22s} {'calls':>6s} {'mean_us':>9s} {'median_us':>9s} {'min_us':>9s} {'max_us':>9s} "
          f"{'total_us':>10s}  kernel")
    for name, ds in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        ds = sorted(ds)
        n, tot = len(ds), sum(ds)
        med = ds[n // 2] if n % 2 else (ds[n // 2 - 1] + ds[n // 2]) / 2
        lab = label_of(name) or "-"
        short = re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", ""))[:80]
        print(f"{lab:22s} {n:6d} {tot / n / 1e3:9.2f} {med / 1e3:9.2f} {ds[0] / 1e3:9.2f} {ds[-1] / 1e3:9.2f} "
              f"{tot / 1e3:10.1f}  {short}")


def _counter(db: str, counter: str):
    c = sqlite3.connect(db)
    rows = c.execute("select kernel_name, dispatch_id, sum(value) from counters_collection "
                     "where counter_name = ? group by dispatch_id", (counter,)).fetchall()
    per = collections.defaultdict(list)
    calib = 0.0
    for name, _, kib in rows:
        lab = label_of(name)
        if lab:
            per[lab].append(kib)
        elif "qat::" not in name:
            calib = max(calib, kib)
    return per, calib


def traffic(fetch_db: str, write_db: str, copy_bytes: int, cmd: str) -> None:
    sys.path.insert(0, ".")
    from bench import sources_hash

    fetch, cf = _counter(fetch_db, "FETCH_SIZE")
    write, cw = _counter(write_db, "WRITE_SIZE")
    if cf <= 0 or cw <= 0:
        raise SystemExit("no calibration copy found in the counter runs")
    sf = copy_bytes / (cf * 1024.0)
    sw = copy_bytes / (cw * 1024.0)
    out = {"command": cmd, "sources_hash": sources_hash(),
           "calibration": {"copy_bytes": copy_bytes, "fetch_kib": cf, "write_kib": cw,
                           "fetch_scale": sf, "write_scale": sw},
           "kernels": {}}
    for lab in sorted(set(fetch) | set(write)):
        f = sum(fetch.get(lab, [0])) / max(len(fetch.get(lab, [])), 1) * 1024.0 * sf
        w = sum(write.get(lab, [0])) / max(len(write.get(lab, [])), 1) * 1024.0 * sw
        out["kernels"][lab] = {"fetch_bytes": round(f), "write_bytes": round(w), "bytes_per_launch": round(f + w),
                               "dispatches": max(len(fetch.get(lab, [])), len(write.get(lab, [])))}
    print(json.dumps(out, indent=1))


def pmc(db: str, cmd: str) -> None:
    c = sqlite3.connect(db)
    rows = c.execute("select kernel_name, dispatch_id, counter_name, sum(value) from counters_collection "
                     "group by dispatch_id, counter_name").fetchall()
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for name, _, cn, v in rows:
        lab = label_of(name)
        if lab:
            agg[lab][cn].append(v)
    print(f"# rocprofv3 counter summary (mean per dispatch)\n# command: {cmd}\n#")
    for lab in sorted(agg):
        d = {cn: sum(v) / len(v) for cn, v in agg[lab].items()}
        n = max(len(v) for v in agg[lab].values())
        extra = []
        if "SQ_VALU_MFMA_BUSY_CYCLES" in d and d.get("GRBM_GUI_ACTIVE"):
            util = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / 8 * 1024)
            extra.append(f"mfma_util={util:.3f}")
        if "SQ_LDS_BANK_CONFLICT" in d and d.get("SQ_LDS_IDX_ACTIVE"):
            extra.append(f"lds_conflict_share={d['SQ_LDS_BANK_CONFLICT'] / d['SQ_LDS_IDX_ACTIVE']:.3f}")
        vals = "  ".join(f"{cn}={v:.4g}" for cn, v in sorted(d.items()))
        print(f"{lab:22s} dispatches={n}  {'  '.join(extra)}\n    {vals}")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("db")
    a.add_argument("--cmd", default="")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_db")
    b.add_argument("write_db")
    b.add_argument("--copy-bytes", type=int, default=1 << 30)
    b.add_argument("--cmd", default="")
    c = sub.add_parser("pmc")
    c.add_argument("db")
    c.add_argument("--cmd", default="")
    args = ap.parse_args()
    if args.what == "stats":
        stats(args.db, args.cmd)
    elif args.what == "pmc":
        pmc(args.db, args.cmd)
    else:
        traffic(args.fetch_db, args.write_db, args.copy_bytes, args.cmd)


if __name__ == "__main__":
    main()
