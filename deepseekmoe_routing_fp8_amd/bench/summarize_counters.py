"""Summarise rocprofv3 counter and trace runs of bench/moe_counters into a short text file.

Each run directory holds rocprofv3's CSV output of one pass over the same driver command:
  --fetch  FETCH_SIZE        --write  WRITE_SIZE
  --util   MfmaUtil, VALUBusy, LdsUtil, LDSBankConflict, SQ_INSTS_VALU_MFMA_MOPS_F8,
           SQ_INSTS_VALU_MFMA_MOPS_F6F4, GRBM_GUI_ACTIVE
  --trace  --kernel-trace --stats
  --sq     optional: two passes of SQ wave-state counters (SQ_WAVE_CYCLES, SQ_WAIT_ANY,
           SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_{ANY,VALU,LDS,VMEM,SCA}; SQ_INSTS_{VALU,MFMA,
           LDS,SALU}, SQ_WAIT_INST_LDS, SQ_VALU_MFMA_BUSY_CYCLES, SQ_LDS_IDX_ACTIVE,
           SQ_WAVES, GRBM_GUI_ACTIVE)
The copy kernel's readings calibrate the byte counters (its bytes are known from the
driver's log). Per kernel: the mean per dispatch of every counter, HBM bytes, the
kernel-trace average duration, and from these GB/s and the MFMA figures.

Usage: python summarize_counters.py --workload v3_prefill --log driver.log --fetch D
         --write D --util D --trace D [--sq D1 D2] --cmd "<commands>" [--sources f1 f2 ...]
       python summarize_counters.py --trace-only --trace D --title T --cmd "<command>"
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
from collections import defaultdict

HBM_PEAK = 8000.0      # GB/s
FP8_PEAK = 5000.0      # TFLOP/s, dense


def short(name: str) -> str:
    n = re.sub(r"^void ", "", name)
    n = re.sub(r"moe::|\(anonymous namespace\)::", "", n)
    n = re.sub(r"\(.*$", "", n)
    return n.strip()


def rows(d: str, suffix: str):
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f, newline="") as fh:
            out += list(csv.DictReader(fh))
    return out


def counters(d: str):
    """{kernel: {counter: [value per dispatch]}}"""
    acc = defaultdict(lambda: defaultdict(dict))
    for r in rows(d, "counter_collection.csv"):
        k = short(r["Kernel_Name"])
        acc[k][r["Counter_Name"]][int(r["Dispatch_Id"])] = float(r["Counter_Value"])
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in acc.items()}


def mean(v):
    return sum(v) / len(v) if v else float("nan")


def trace_table(trace: str, title: str, cmd: str, note: str):
    """Markdown table of a --kernel-trace --stats run (kernel, calls, average/min/max us,
    share of GPU time)."""
    st = rows(trace, "kernel_stats.csv")
    print(f"# Kernel trace: {title}\n")
    if note:
        print(note + "\n")
    print("Command (repository root `$R`; library built with "
          "`python deepseekmoe_routing_fp8_amd/build.py --tools`):\n")
    print("```\ncd /tmp && export TMPDIR=/tmp")
    for c in cmd.split(" ;; "):
        print(c)
    print("```\n")
    # steady state: every dispatch of a kernel but its first (the first call of a kernel
    # in a process also loads its code object)
    per = defaultdict(list)
    for r in rows(trace, "kernel_trace.csv"):
        per[short(r["Kernel_Name"])].append(
            (int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    print("| kernel | calls | average us | average us without the first call | min us | max us | "
          "share of GPU time |")
    print("|---|---|---|---|---|---|---|")
    for r in sorted(st, key=lambda r: -float(r["TotalDurationNs"])):
        k = short(r["Name"])
        d = [v for _, v in sorted(per.get(k, []))][1:]
        steady = f"{sum(d) / len(d):.1f}" if d else "-"
        print(f"| `{k}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {steady} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
              f"{float(r['Percentage']):.2f}% |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace-only", action="store_true",
                    help="print only the kernel-trace table of --trace (with --title, --note)")
    ap.add_argument("--title", default="")
    ap.add_argument("--note", default="")
    ap.add_argument("--workload")
    ap.add_argument("--log")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--util")
    ap.add_argument("--trace", required=True)
    ap.add_argument("--cmd", required=True)
    ap.add_argument("--flops", nargs="*", default=[],
                    help="kernel=FLOPs per dispatch (algorithmic), for the MFMA rows")
    ap.add_argument("--bytes", nargs="*", default=[],
                    help="kernel=bytes per dispatch (algorithmic), for the traffic ratio")
    ap.add_argument("--sources", nargs="*", default=[])
    ap.add_argument("--sq", nargs="*", default=[],
                    help="run directories of the SQ wave-state passes (printed for the FFN kernels)")
    a = ap.parse_args()
    if a.trace_only:
        trace_table(a.trace, a.title, a.cmd, a.note)
        return

    log = open(a.log).read()
    m = re.search(r"copy_kernel: (\d+) bytes read \+ (\d+) bytes written", log)
    copy_r, copy_w = int(m.group(1)), int(m.group(2))
    fe, wr, ut = counters(a.fetch), counters(a.write), counters(a.util)
    rscale = copy_r / (mean(fe["copy_kernel"]["FETCH_SIZE"]) * 1024)
    wscale = copy_w / (mean(wr["copy_kernel"]["WRITE_SIZE"]) * 1024)
    dur = {}
    for r in rows(a.trace, "kernel_stats.csv"):
        dur[short(r["Name"])] = (float(r["AverageNs"]) / 1e3, int(r["Calls"]), float(r["MinNs"]) / 1e3)
    alg_f = {k: float(v) for k, v in (s.split("=") for s in a.flops)}
    alg_b = {k: float(v) for k, v in (s.split("=") for s in a.bytes)}
    # the grouped FFN's algorithmic figures from the driver's shape and expert loads: every
    # touched expert's codes and block scales once, every token's 1x128 codes and scales
    # once, the 1x128 intermediate written and read once per row, bf16 rows out
    w = re.search(r"T=(\d+) H=(\d+) I=(\d+) routed=(\d+) shared=(\d+) top_k=(\d+) rows=(\d+)", log)
    ld = re.search(r"expert loads:([ \d]+)", log)
    if w and ld:
        T, H, I, N, S, k, nrows = (int(v) for v in w.groups())
        touched = sum(1 for v in ld.group(1).split() if int(v) > 0) + S
        mat = I * H + (I // 128) * (H // 128) * 4
        inter = nrows * (I + (I // 128) * 4)
        alg_b.setdefault("ffn_kernel<1, unsigned short, false>", touched * 2 * mat + T * (H + H // 32) + inter)
        alg_b.setdefault("ffn_kernel<2, unsigned short, false>", touched * mat + inter + nrows * H * 2)
        alg_f.setdefault("ffn_kernel<1, unsigned short, false>", 4.0 * H * I * nrows)
        alg_f.setdefault("ffn_kernel<2, unsigned short, false>", 2.0 * H * I * nrows)

    print(f"# Counter summary of one MoE-layer step, workload {a.workload}")
    for line in log.splitlines():
        if line.startswith("workload") or line.startswith("copy_kernel"):
            print(f"# {line}")
    print("#\n# Commands (repository root $R, drivers built by "
          "`python deepseekmoe_routing_fp8_amd/build.py --tools`):")
    for c in a.cmd.split(" ;; "):
        print(f"#   {c}")
    print(f"#\n# Calibration (copy_kernel): read scale {rscale:.4f} x FETCH_SIZE, write scale "
          f"{wscale:.4f} x WRITE_SIZE")
    print("# Per kernel, mean per dispatch. bytes = 1024 * (FETCH_SIZE * read scale + WRITE_SIZE * "
          "write scale); time = kernel-trace average; MfmaUtil = busy MFMA cycles / (GPU cycles x "
          "SIMDs); f8 TFLOP/s = 512 * (MOPS_F8 + MOPS_F6F4) / time.")
    hdr = (f"# {'kernel':44s} {'calls':>5s} {'avg us':>9s} {'read GB':>8s} {'write GB':>8s} "
           f"{'GB/s':>7s} {'%HBM':>5s} {'alg x':>6s} {'Mfma%':>6s} {'VALU%':>6s} {'LDS%':>5s} "
           f"{'bank%':>5s} {'f8 TF/s':>8s} {'%FP8':>5s}")
    print(hdr)
    out = {}
    for k in sorted(dur, key=lambda k: -dur[k][0] * dur[k][1]):
        if k.startswith("copy_kernel") or k.startswith("fill_"):
            continue
        us, calls, _ = dur[k]
        rb = mean(fe.get(k, {}).get("FETCH_SIZE", [])) * 1024 * rscale
        wb = mean(wr.get(k, {}).get("WRITE_SIZE", [])) * 1024 * wscale
        u = ut.get(k, {})
        mops = mean(u.get("SQ_INSTS_VALU_MFMA_MOPS_F8", [0.0])) + mean(u.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", [0.0]))
        tf = 512 * mops / (us * 1e-6) / 1e12
        gbs = (rb + wb) / (us * 1e-6) / 1e9
        ratio = (rb + wb) / alg_b[k] if k in alg_b else float("nan")
        print(f"  {k:44s} {calls:5d} {us:9.1f} {rb / 1e9:8.4f} {wb / 1e9:8.4f} {gbs:7.0f} "
              f"{100 * gbs / HBM_PEAK:5.1f} {ratio:6.3f} {mean(u.get('MfmaUtil', [float('nan')])):6.1f} "
              f"{mean(u.get('VALUBusy', [float('nan')])):6.1f} {mean(u.get('LdsUtil', [float('nan')])):5.1f} "
              f"{mean(u.get('LDSBankConflict', [float('nan')])):5.1f} {tf:8.1f} {100 * tf / FP8_PEAK:5.1f}")
        out[k] = (rb + wb, us, mops)
        if k in alg_b:
            print(f"      algorithmic {alg_b[k] / 1e9:.4f} GB per dispatch -> "
                  f"{alg_b[k] / (us * 1e-6) / 1e9:.0f} GB/s algorithmic ({alg_b[k] / (us * 1e-6) / 1e9 / HBM_PEAK:.3f} of 8 TB/s)")
        if k in alg_f:
            print(f"      algorithmic {alg_f[k] / 1e12:.4f} TFLOP per dispatch; counted "
                  f"{512 * mops / 1e12:.4f} TFLOP (x{512 * mops / alg_f[k]:.3f}); "
                  f"{alg_f[k] / (us * 1e-6) / 1e12:.1f} TFLOP/s algorithmic")
    if a.sq:
        sq = {}
        for d in a.sq:
            for k, cs in counters(d).items():
                sq.setdefault(k, {}).update(cs)
        print("#\n# Wave states of the FFN kernels (SQ counters, mean per dispatch). Wave time is "
              "SQ_WAVE_CYCLES (quad-cycles summed over waves) = 100%: SQ_ACTIVE_INST_ANY (issuing or "
              "executing an instruction), SQ_WAIT_INST_ANY (waiting for an instruction to issue: "
              "dependencies, issue arbitration), SQ_WAIT_ANY (waiting at s_waitcnt or s_barrier); "
              "the active time by instruction type (VALU includes the MFMA issue). MFMA busy = "
              "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs): GRBM_GUI_ACTIVE as "
              "collected sums the 8 XCDs' counts, so this matches the Mfma% column. Instructions "
              "per MFMA from SQ_INSTS_*.")
        for k in sorted(sq):
            if not k.startswith("ffn_kernel"):
                continue
            c = {n: mean(v) for n, v in sq[k].items()}
            wc = c.get("SQ_WAVE_CYCLES", float("nan"))
            pct = lambda n: 100.0 * c.get(n, float("nan")) / wc
            mf = c.get("SQ_INSTS_MFMA", float("nan"))
            busy = 100.0 * c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (
                c.get("GRBM_GUI_ACTIVE", float("nan")) / 8 * 1024)
            print(f"  {k}: active {pct('SQ_ACTIVE_INST_ANY'):.1f}%, waiting to issue "
                  f"{pct('SQ_WAIT_INST_ANY'):.1f}%, waiting at waitcnt/barrier {pct('SQ_WAIT_ANY'):.1f}%; "
                  f"active on VALU {pct('SQ_ACTIVE_INST_VALU'):.1f}%, LDS {pct('SQ_ACTIVE_INST_LDS'):.1f}%, "
                  f"VMEM {pct('SQ_ACTIVE_INST_VMEM'):.1f}%, scalar {pct('SQ_ACTIVE_INST_SCA'):.1f}%; "
                  f"waiting for LDS issue {pct('SQ_WAIT_INST_LDS'):.1f}%; MFMA busy {busy:.1f}%; per MFMA "
                  f"{(c.get('SQ_INSTS_VALU', 0) - mf) / mf:.2f} other VALU, {c.get('SQ_INSTS_LDS', 0) / mf:.2f} LDS, "
                  f"{c.get('SQ_INSTS_SALU', 0) / mf:.2f} SALU instructions; {c.get('SQ_WAVES', 0):.0f} waves")
    if a.sources:
        h = hashlib.sha256()
        for f in a.sources:
            h.update(open(f, "rb").read())
        print("#\n# Values read by bench.py (traffic is reported only while the kernel sources hash "
              "to this value):")
        print(f"kernel_sources_sha256 = {h.hexdigest()}")
        print(f"read_scale = {rscale:.6f}")
        print(f"write_scale = {wscale:.6f}")
        for k, (b, us, _) in out.items():
            if k.startswith("ffn_kernel<1"):
                print(f"traffic_bytes_per_launch = {b:.0f}")
            if k.startswith("ffn_kernel<2"):
                print(f"down_traffic_bytes_per_launch = {b:.0f}")


if __name__ == "__main__":
    main()
