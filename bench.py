"""Benchmark of the DSA token-selection hot path with IndexShare on one MI355X.

One step = one IndexShare group pass over one synthetic batch: the Full layer's fused
indexer + top-k (k = 2048) once, then the sparse MLA attention of all 4 layers (1 Full +
3 Shared) with that index set.  Headline workload: 131072-token prefill, FP8 indexer
(H_I = 64, d_I = 128, per-token scales), bf16 576-d latent KV with 32 query heads.
Inputs are resident in HBM before the timed region starts.

Also reported (same JSON line): decode at 64 x 200K (1 new token per sequence) step and
per-token latency, the all-layers-Full comparator (every layer runs its own indexer),
per-kernel HIP-event timings with their roofline fractions, an 80-layer stack run one call
per layer under the FSSS, released (freq 4, offset 3) and all-Full schedules, the per-token
E4M3 quantization of the indexer operands (prefill q^I, decode k^I cache append), and the
CPU oracle timed on a bounded sample of query rows.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu] [--no-stack] [--no-quant]
"""
import argparse
import csv
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                 # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}
# what bounds each compute dtype of the path, and its datasheet peak: fp8 and bf16 run on the
# matrix cores; the fp32 reference-size path (the Tiny config) runs on the vector ALU, whose
# fp32 peak is 256 CUs x 4 SIMDs x 64 flops per clock (32 FMA lanes) x 2.4 GHz = 157.3 TFLOP/s
COMPUTE_PEAK = {"fp8": ("mfma", 5000.0), "bf16": ("mfma", 2500.0), "f32": ("alu", 157.3)}

# Memory traffic per launch comes from two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE)
# summarised under profiles/.  Both count the L2's requests to the memory side (its misses
# and write-backs), which the Infinity Cache or HBM serves: an upper bound of the DRAM bytes.
# A summary is used only while the kernel's sources still hash to the digest it records;
# otherwise the traffic is reported as null.
PKG = os.path.join(ROOT, "dsa_lightning_indexer_scores_amd")
KERNEL_SOURCES = {"mla_attn32_kernel": ["csrc/attn.hip", "csrc/mla_blocks.hpp"],
                  "mla_combine_kernel": ["csrc/attn.hip", "csrc/mla_blocks.hpp"],
                  "indexer_topk_kernel": ["csrc/indexer.hip"]}
COMMON_SOURCES = ["csrc/dsa_common.hpp", "csrc/dsa_launch.hpp", "build_lib.py"]
TRAFFIC_SUMMARY = {"sparse_attn": ("mla_attn32_kernel", "profiles/mla_attn32_kernel_prefill128k_memtraffic.txt"),
                   "indexer_topk": ("indexer_topk_kernel", "profiles/indexer_topk_kernel_prefill128k_memtraffic.txt")}
PMC_COMMAND = ('rocprofv3 --pmc {counter} --kernel-include-regex "dsa::|copyBuffer" --output-format csv '
               '-d {dir} -o run -- {bench}')
BENCH_ONE_STEP = ("python3 bench.py --workload {workload} --steps 1 --warmup 0 --no-cpu --no-allfull --no-decode "
                  "--no-prefill16k --no-stack --no-chunk1m --no-quant --no-train --no-attainable")
COPY_BYTES = 1 << 30
# Counter passes for the execution profile of a kernel (each within one rocprofv3 pass's
# limits on gfx950: at most 8 SQ, 4 TCC, 4 TCP, 2 TA and 2 GRBM counters).
PMC_PASSES = {
    "sq_issue": "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
                "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE",
    "sq_wait": "SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_ANY SQ_INSTS_VALU_MFMA_MOPS_BF16 "
               "SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_VALU_MFMA_COEXEC_CYCLES SQ_INST_CYCLES_VMEM_RD GRBM_GUI_ACTIVE",
    "l2": "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_DRAM_32B_sum TCC_EA0_WRREQ_WRITE_DRAM_32B_sum GRBM_GUI_ACTIVE",
    "l1": "TCP_TCC_READ_REQ_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_PENDING_STALL_CYCLES_sum "
          "TCP_TCP_TA_DATA_STALL_CYCLES_sum TA_TA_BUSY_sum TA_ADDR_STALLED_BY_TC_CYCLES_sum GRBM_GUI_ACTIVE",
}
N_XCD, N_CU, N_SIMD = 8, 256, 1024


class Work:
    """Algorithmic work of the path: causal (query, key) pairs the indexer scores and
    selected pairs the sparse attention reads, and their flops."""

    @staticmethod
    def causal_pairs(L, Lq):
        # queries at positions L-Lq .. L-1 see L-Lq+1 .. L keys
        return (2 * L - Lq + 1) * Lq // 2

    @staticmethod
    def selected_pairs(L, k, Lq):
        # a query at position p reads min(k, p + 1) keys
        first = L - Lq + 1
        if first > k:
            return Lq * k
        small = min(k, L)                      # counts first .. small are below or at k
        return (first + small) * (small - first + 1) // 2 + (L - small) * k

    @staticmethod
    def indexer_flops(pairs, H_I, d_I):
        return 2 * H_I * d_I * pairs

    @staticmethod
    def attention_flops(pairs, H, Dqk, Dv):
        return 2 * H * (Dqk + Dv) * pairs


def kernel_sources(kernel):
    """The library sources a kernel is built from: the csrc file that defines it, plus the
    shared headers and build flags."""
    if kernel in KERNEL_SOURCES:
        return KERNEL_SOURCES[kernel]
    found = []
    for f in sorted(os.listdir(os.path.join(PKG, "csrc"))):
        if f.endswith(".hip") and re.search(r"\b" + re.escape(kernel) + r"\s*\(", open(os.path.join(PKG, "csrc", f)).read()):
            found.append("csrc/" + f)
    return found


def source_digest(kernel):
    h = hashlib.sha256()
    for rel in sorted(kernel_sources(kernel) + COMMON_SOURCES):
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(rel.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(name):
    """HBM bytes per launch from the committed counter summary, or None when absent or stale."""
    kernel, rel = TRAFFIC_SUMMARY[name]
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("source_digest") != source_digest(kernel):
        return None
    return int(fields["traffic_bytes_per_launch"])


def summarize_trace(trace_csv):
    """Per (kernel, grid size) launch statistics of a rocprofv3 kernel trace: the same
    kernel is launched with different grids by the workloads of one benchmark run."""
    groups = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "dsa::" not in name:
                continue
            grid = (r.get("Grid_Size_X") or r.get("Grid_Size") or "?", r.get("Grid_Size_Y", "1"))
            dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            groups.setdefault((name, grid), []).append(dur)
    # launches under 5% of the longest of their group (the fused indexer's near-empty
    # recompute pass, for one) get a row of their own, marked "short"
    rows = []
    for (name, grid), d in groups.items():
        top = max(d)
        long_d = [x for x in d if x >= 0.05 * top]
        short_d = [x for x in d if x < 0.05 * top]
        rows.append((name, grid, "", long_d))
        if short_d:
            rows.append((name, grid, "short", short_d))
    lines = ["kernel,grid_x,grid_y,launches,calls,avg_us,min_us,max_us"]
    for name, grid, tag, d in sorted(rows, key=lambda r: -sum(r[3])):
        lines.append(f'"{name}",{grid[0]},{grid[1]},{tag or "work"},{len(d)},{sum(d) / len(d) / 1e3:.2f},'
                     f'{min(d) / 1e3:.2f},{max(d) / 1e3:.2f}')
    return "\n".join(lines)


def summarize_counters(fetch_csv, write_csv, kernel, template, workload):
    """Summary text of the two counter runs for one kernel.  FETCH_SIZE and WRITE_SIZE are
    KiB per dispatch of L2-to-memory-side traffic; each is scaled by what it reads for the
    1 GiB device copy that the same run makes (the copy whose WRITE_SIZE is 1 GiB)."""
    def load(path):
        out = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                out[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
        return out
    fetch, write = load(fetch_csv), load(write_csv)
    copies = [d for d, (n, v) in write.items()
              if "copyBuffer" in n and abs(v * 1024 - COPY_BYTES) < 0.005 * COPY_BYTES]
    if not copies:
        raise SystemExit("no 1 GiB calibration copy in the WRITE_SIZE run")
    cid = copies[-1]
    if cid not in fetch or "copyBuffer" not in fetch[cid][0]:
        raise SystemExit("the FETCH_SIZE run does not have the calibration copy at the same dispatch")
    f_scale = COPY_BYTES / (fetch[cid][1] * 1024)
    w_scale = COPY_BYTES / (write[cid][1] * 1024)
    sel = [d for d, (n, v) in fetch.items() if kernel in n and template in n]
    if not sel or any(d not in write for d in sel):
        raise SystemExit(f"no dispatches of {kernel}{template} in both runs")
    # launches that do the work: dispatches reading under 1% of the largest one (the fused
    # indexer's recompute pass when no item failed) are left out of the per-launch figures
    n_all = len(sel)
    top = max(fetch[d][1] for d in sel)
    sel = [d for d in sel if fetch[d][1] >= 0.01 * top]
    f_kib = sum(fetch[d][1] for d in sel) / len(sel)
    w_kib = sum(write[d][1] for d in sel) / len(sel)
    read_b = f_kib * 1024 * f_scale
    write_b = w_kib * 1024 * w_scale
    bench_cmd = BENCH_ONE_STEP.format(workload=workload) + " --copy-calibration"
    lines = [
        f"# memory-side traffic (L2 misses and write-backs: FETCH_SIZE, WRITE_SIZE; served by the",
        f"# Infinity Cache or HBM) of dsa::{kernel}{template}, workload {workload}",
        "# commands, from the repository root on one MI355X (cd /tmp && export TMPDIR=/tmp first):",
        "#   " + PMC_COMMAND.format(counter="FETCH_SIZE", dir="<fetch_dir>", bench=bench_cmd),
        "#   " + PMC_COMMAND.format(counter="WRITE_SIZE", dir="<write_dir>", bench=bench_cmd),
        f"#   python3 bench.py --summarize-counters <fetch_dir>/run_counter_collection.csv "
        f"<write_dir>/run_counter_collection.csv --kernel {kernel} --template '{template}' --workload {workload}",
        f"calibration_copy_bytes: {COPY_BYTES}",
        f"calibration_fetch_kib: {fetch[cid][1]:.2f}",
        f"calibration_write_kib: {write[cid][1]:.2f}",
        f"read_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        "# launches: the dispatches that do the work (those reading under 1% of the largest are left out)",
        f"dispatches: {n_all}",
        f"launches: {len(sel)}",
        f"fetch_kib_per_launch: {f_kib:.1f}",
        f"write_kib_per_launch: {w_kib:.1f}",
        f"read_bytes_per_launch: {int(read_b)}",
        f"write_bytes_per_launch: {int(write_b)}",
        f"traffic_bytes_per_launch: {int(read_b + write_b)}",
        f"source_digest: {source_digest(kernel)}",
    ]
    return "\n".join(lines)


def summarize_pmc(csvs, kernel, template, workload, command):
    """Execution profile of one kernel from rocprofv3 counter runs (PMC_PASSES): the mean per
    launch of every counter, then the fractions derived from them.  Launches are matched by
    their order among the kernel's dispatches in each run; dispatches with a duration under
    5% of the longest (the fused indexer's recompute pass when nothing failed) are left out."""
    per_run = []
    for path in csvs:
        rows = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                if kernel not in name or template not in name:
                    continue
                d = rows.setdefault(int(r["Dispatch_Id"]), {"name": name, "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
        per_run.append([rows[d] for d in sorted(rows)])
    if not per_run or not per_run[0]:
        raise SystemExit(f"no dispatches of {kernel}{template}")
    n = min(len(r) for r in per_run)
    top = max(d["ns"] for r in per_run for d in r[:n])
    keep = [i for i in range(n) if all(r[i]["ns"] >= 0.05 * top for r in per_run)]
    vals, ns = {}, []
    for i in keep:
        for r in per_run:
            ns.append(r[i]["ns"])
            for c, v in r[i].items():
                if c not in ("name", "ns"):
                    vals.setdefault(c, []).append(v)
    mean = {c: sum(v) / len(v) for c, v in vals.items()}
    lines = [f"# rocprofv3 counters of dsa::{kernel}{template}, workload {workload}",
             "# commands, from the repository root on one MI355X (cd /tmp && export TMPDIR=/tmp first), one per pass:"]
    for pname, ctrs in PMC_PASSES.items():
        lines.append("#   " + command.format(counters=ctrs, dir=f"<{pname}_dir>"))
    lines.append(f"#   python3 bench.py --summarize-pmc <each pass dir>/run_counter_collection.csv ... "
                 f"--kernel {kernel} --template '{template}' --workload {workload}")
    lines.append(f"dispatches_per_run: {n}")
    lines.append(f"launches: {len(keep)}")
    lines.append(f"mean_duration_us_under_counters: {sum(ns) / len(ns) / 1e3:.1f}")
    for c in sorted(mean):
        lines.append(f"{c}: {mean[c]:.6g}")
    # derived fractions; GRBM_GUI_ACTIVE is summed over the XCDs by the CSV, so the busy
    # clock of the launch is that sum / XCDs; SQ_ACTIVE_* and SQ_WAVE_CYCLES count quad-cycles
    gui = mean.get("GRBM_GUI_ACTIVE")
    def put(name, v, note):
        lines.append(f"{name}: {v:.4f}    # {note}")
    if gui:
        clk = gui / N_XCD
        lines.append(f"busy_cycles_per_xcd: {clk:.6g}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            put("mfma_busy_frac", mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (clk * N_SIMD), "SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)")
        if "SQ_ACTIVE_INST_VALU" in mean:
            put("valu_busy_frac", 4 * mean["SQ_ACTIVE_INST_VALU"] / (clk * N_SIMD), "4 x SQ_ACTIVE_INST_VALU / (cycles x 1024 SIMDs)")
        if "SQ_LDS_IDX_ACTIVE" in mean:
            put("lds_active_frac", mean["SQ_LDS_IDX_ACTIVE"] / (clk * N_CU), "SQ_LDS_IDX_ACTIVE / (cycles x 256 CUs)")
        if "SQ_LDS_BANK_CONFLICT" in mean:
            put("lds_bank_conflict_frac", mean["SQ_LDS_BANK_CONFLICT"] / (clk * N_CU), "SQ_LDS_BANK_CONFLICT / (cycles x 256 CUs)")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in mean:
            put("mfma_valu_coexec_frac", mean["SQ_VALU_MFMA_COEXEC_CYCLES"] / (clk * N_SIMD), "SQ_VALU_MFMA_COEXEC_CYCLES / (cycles x 1024 SIMDs)")
        if "TA_TA_BUSY_sum" in mean:
            put("ta_busy_frac", mean["TA_TA_BUSY_sum"] / (clk * N_CU), "TA_TA_BUSY_sum / (cycles x 256 CUs)")
        if "TCP_PENDING_STALL_CYCLES_sum" in mean:
            put("l1_pending_stall_frac", mean["TCP_PENDING_STALL_CYCLES_sum"] / (clk * N_CU), "TCP_PENDING_STALL_CYCLES_sum / (cycles x 256 CUs)")
    if "SQ_WAVE_CYCLES" in mean and "SQ_WAIT_INST_ANY" in mean:
        put("wave_wait_inst_frac", mean["SQ_WAIT_INST_ANY"] / mean["SQ_WAVE_CYCLES"], "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES")
    if "SQ_WAVE_CYCLES" in mean and "SQ_ACTIVE_INST_ANY" in mean:
        put("wave_issue_frac", mean["SQ_ACTIVE_INST_ANY"] / mean["SQ_WAVE_CYCLES"], "SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES")
    if "TCC_HIT_sum" in mean and "TCC_MISS_sum" in mean:
        put("l2_hit_frac", mean["TCC_HIT_sum"] / max(1.0, mean["TCC_HIT_sum"] + mean["TCC_MISS_sum"]), "TCC_HIT / (TCC_HIT + TCC_MISS)")
    if "TCC_EA0_RDREQ_DRAM_32B_sum" in mean:
        lines.append(f"l2_miss_read_bytes_per_launch: {int(32 * mean['TCC_EA0_RDREQ_DRAM_32B_sum'])}    "
                     f"# 32 x TCC_EA0_RDREQ_DRAM_32B: L2 misses to the memory side (served by the Infinity Cache or HBM)")
    if "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum" in mean:
        lines.append(f"l2_write_bytes_per_launch: {int(32 * mean['TCC_EA0_WRREQ_WRITE_DRAM_32B_sum'])}    "
                     f"# 32 x TCC_EA0_WRREQ_WRITE_DRAM_32B")
    if "TCP_TCC_READ_REQ_sum" in mean and "TCP_TCC_READ_REQ_LATENCY_sum" in mean:
        put("l1_to_l2_read_latency_cycles", mean["TCP_TCC_READ_REQ_LATENCY_sum"] / max(1.0, mean["TCP_TCC_READ_REQ_sum"]),
            "TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum")
    if "SQ_INSTS_MFMA" in mean and "SQ_INSTS_VALU" in mean:
        put("valu_insts_per_mfma", (mean["SQ_INSTS_VALU"] - mean["SQ_INSTS_MFMA"]) / max(1.0, mean["SQ_INSTS_MFMA"]),
            "(SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA (SQ_INSTS_VALU includes the MFMAs)")
    for dt in ("BF16", "F8"):
        c = f"SQ_INSTS_VALU_MFMA_MOPS_{dt}"
        if mean.get(c):
            lines.append(f"mfma_flops_{dt.lower()}_per_launch: {mean[c] * 512:.6g}    # 512 x {c}")
    lines.append(f"source_digest: {source_digest(kernel)}")
    return "\n".join(lines)


def main_roofline(cfg, L, idx_ms, attn_ms, idx_flop, attn_flop, attn_gather_gb):
    """Roofline object of the main line: the kernel with the larger share of the step
    (the indexer once against the attention of every layer), priced by what bounds it.
    With fewer than 16 queries per sequence (decode) neither part reuses keys, so both are
    priced in HBM bytes: the k^I cache with its scales, the gathered latent rows.  Otherwise
    both are dense contractions priced against the peak of their arithmetic type.  Returns
    (roofline, extra indexer fields or None)."""
    idx_tfs = idx_flop / (idx_ms * 1e-3) / 1e12
    attn_tfs = attn_flop / (attn_ms * 1e-3) / 1e12
    idx_first = idx_ms >= attn_ms * cfg.n_layers
    if cfg.Lq < 16:
        code_bytes = {"fp8": 1, "bf16": 2, "f32": 4}[cfg.idx_dtype]
        kI_gb = cfg.B * L * (cfg.d_I * code_bytes + (4 if cfg.idx_dtype == "fp8" else 0)) / 1e9
        idx_gbs, attn_gbs = kI_gb / (idx_ms * 1e-3), attn_gather_gb / (attn_ms * 1e-3)
        name, gbs = ("indexer_topk", idx_gbs) if idx_first else ("sparse_attn", attn_gbs)
        roof = {"kernel": name, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
        return roof, {"hbm_gb": round(kI_gb, 3), "hbm_gbs": round(idx_gbs, 1)}
    if idx_first:
        (bound, peak), name, tfs = COMPUTE_PEAK[cfg.idx_dtype], "indexer_topk", idx_tfs
    else:
        (bound, peak), name, tfs = COMPUTE_PEAK[cfg.attn_dtype], "sparse_attn", attn_tfs
    return {"kernel": name, "bound": bound, "achieved": round(tfs, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(tfs / peak, 4)}, None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill128k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill16k", action="store_true", help="skip the 16384-token bf16 prefill group line")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-allfull", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the 80-layer stack at the prefill workload")
    ap.add_argument("--no-chunk1m", action="store_true")
    ap.add_argument("--no-train", action="store_true", help="skip the indexer-training (centroid, KL backward) measurement")
    ap.add_argument("--no-quant", action="store_true", help="skip the step-before-the-path measurements (projections, per-token E4M3 quantization)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device-to-device copy (HBM counter scale)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of two rocprofv3 counter runs and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_CSV",
                    help="print per (kernel, grid) launch statistics of a rocprofv3 kernel trace and exit")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="print the execution profile (PMC_PASSES counter runs) of --kernel and exit")
    ap.add_argument("--pmc-command", default="",
                    help="the benchmark command the counter runs profiled (recorded in the summary)")
    ap.add_argument("--no-attainable", action="store_true",
                    help="skip the library GEMM and device-copy reference measurements")
    ap.add_argument("--kernel", default="mla_attn32_kernel")
    ap.add_argument("--template", default="")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, args.kernel, args.template, args.workload))
        return
    if args.summarize_pmc:
        cmd = ('rocprofv3 --pmc {counters} --kernel-include-regex "dsa::" --output-format csv -d {dir} -o run -- '
               + (args.pmc_command or BENCH_ONE_STEP.format(workload=args.workload)))
        print(summarize_pmc(args.summarize_pmc, args.kernel, args.template, args.workload, cmd))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the library and this benchmark run on one GPU; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import dsa_lightning_indexer_scores_amd as dsa
    accounting = Work

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.get_config(args.workload)
    L, k = cfg.L, cfg.topk
    log(f"[bench] generating {cfg.name}: L={L} k={k} H_I={cfg.H_I} d_I={cfg.d_I} {cfg.idx_dtype}")
    t0 = time.time()
    ind = synth.indexer_inputs(cfg, device=dev)
    layers = [synth.attention_inputs(cfg, layer=l, device=dev) for l in range(cfg.n_layers)]
    idx = torch.empty((cfg.B, cfg.Lq, k), dtype=torch.int32, device=dev)
    out_dtype = torch.float32 if cfg.attn_dtype == "f32" else torch.bfloat16
    outs = [torch.empty((cfg.B, cfg.Lq, cfg.H, cfg.Dv), dtype=out_dtype, device=dev)
            for _ in range(cfg.n_layers)]
    ws = dsa.Workspace()
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, q_scale=ind["q_scale"], k_scale=ind["k_scale"],
                         ws=ws, out=idx)
        if ev is not None:
            ev[1].record(stream)
        for l in range(cfg.n_layers):
            dsa.sparse_attn(layers[l], idx, ws=ws, out=outs[l])
            if ev is not None:
                ev[2 + l].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + cfg.n_layers)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for s in range(args.steps):
        step(evs[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    idx_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    attn_ms = float(np.mean([e[1 + l].elapsed_time(e[2 + l]) for e in evs for l in range(cfg.n_layers)]))
    log(f"[bench] step {ms_step:.2f} ms  (indexer+topk {idx_ms:.2f} ms, attention {attn_ms:.2f} ms/layer)")

    tokens = cfg.B * cfg.Lq
    pairs = accounting.causal_pairs(L, cfg.Lq) * cfg.B
    sel = accounting.selected_pairs(L, k, cfg.Lq) * cfg.B
    idx_flop = accounting.indexer_flops(pairs, cfg.H_I, cfg.d_I)
    attn_flop = accounting.attention_flops(sel, cfg.H, cfg.Dqk, cfg.Dv)
    idx_tfs = idx_flop / (idx_ms * 1e-3) / 1e12
    attn_tfs = attn_flop / (attn_ms * 1e-3) / 1e12
    # gathered latent rows (algorithmic bytes of the attention: each selected row once per query)
    attn_gather_gb = sel * cfg.Dqk * 2 / 1e9
    idx_bound, idx_peak = COMPUTE_PEAK[cfg.idx_dtype]
    attn_bound, attn_peak = COMPUTE_PEAK[cfg.attn_dtype]
    kernels = {
        "indexer_topk": {"ms": round(idx_ms, 4), "algorithmic_tflop": round(idx_flop / 1e12, 3),
                         "tflops": round(idx_tfs, 1), "bound": idx_bound, "peak_tflops": idx_peak,
                         "frac": round(idx_tfs / idx_peak, 4)},
        "sparse_attn": {"ms_per_layer": round(attn_ms, 4), "algorithmic_tflop": round(attn_flop / 1e12, 3),
                        "tflops": round(attn_tfs, 1), "bound": attn_bound, "peak_tflops": attn_peak,
                        "frac": round(attn_tfs / attn_peak, 4),
                        "gathered_gb": round(attn_gather_gb, 2),
                        "gather_gbs": round(attn_gather_gb / (attn_ms * 1e-3), 1)},
    }
    if cfg.attn == "mla" and not args.no_decode:
        # one layer over an FP8 latent cache (E4M3 codes + per-row scales) at the same shapes
        lay8 = synth.fp8_latent(layers[1])
        dsa.sparse_attn(lay8, idx, ws=ws, out=outs[1])
        torch.cuda.synchronize()
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for _ in range(3):
            dsa.sparse_attn(lay8, idx, ws=ws, out=outs[1])
        f1.record(stream)
        torch.cuda.synchronize()
        kernels["sparse_attn_fp8_latent"] = {"ms_per_layer": round(f0.elapsed_time(f1) / 3, 4)}
        log(f"[bench] fp8 latent attention {f0.elapsed_time(f1) / 3:.2f} ms/layer")
        del lay8
        torch.cuda.empty_cache()
    # roofline object: the kernel with the larger share of the step
    roof, idx_hbm = main_roofline(cfg, L, idx_ms, attn_ms, idx_flop, attn_flop, attn_gather_gb)
    if idx_hbm is not None:
        kernels["indexer_topk"].update(idx_hbm)
    # measured HBM bytes per launch (counters), only for the workload they were taken on
    roof["traffic"] = recorded_traffic(roof["kernel"]) if cfg.name == "prefill128k" else None

    result = {
        "metric": "indexed prefill tokens/s per 4-layer group @128K; decode us/token @200K; %roofline",
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-indexer/bf16-attention" if cfg.idx_dtype == "fp8" else cfg.idx_dtype,
        "data": "synthetic (seeded Gaussian, 5% planted 3x keys)",
        "config": {"workload": cfg.name, "L": L, "B": cfg.B, "topk": k, "H_I": cfg.H_I, "d_I": cfg.d_I,
                   "indexer_dtype": cfg.idx_dtype, "attention": f"{cfg.attn.upper()} {cfg.H} heads, {cfg.Dqk}/{cfg.Dv}",
                   "group": "1 Full + 3 Shared", "parallelism": "single GPU"},
        "kernels": kernels,
        "roofline": roof,
    }

    if not args.no_allfull:
        # comparator: every layer runs its own indexer + top-k (4 indexers per group)
        others = [synth.indexer_inputs(cfg, device=dev, layer=l) for l in range(1, cfg.n_layers)]
        inds = [ind] + others
        idxs = [torch.empty_like(idx) for _ in range(cfg.n_layers)]

        def step_all_full():
            for l in range(cfg.n_layers):
                d = inds[l]
                dsa.indexer_topk(d["q"], d["k"], d["w"], k, q_scale=d["q_scale"], k_scale=d["k_scale"],
                                 ws=ws, out=idxs[l])
                dsa.sparse_attn(layers[l], idxs[l], ws=ws, out=outs[l])

        step_all_full()
        torch.cuda.synchronize()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        n_af = max(1, min(args.steps, 3))
        a0.record(stream)
        for _ in range(n_af):
            step_all_full()
        a1.record(stream)
        torch.cuda.synchronize()
        ms_af = a0.elapsed_time(a1) / n_af
        result["indexshare"] = {"group_ms": round(ms_step, 3), "all_full_ms": round(ms_af, 3),
                                "speedup": round(ms_af / ms_step, 3),
                                "indexer_calls_per_group": {"indexshare": 1, "all_full": cfg.n_layers},
                                "pages_context": "1.82x prefill / 1.48x decode end-to-end at 200K (30B model); "
                                                 ">=1.3x for 744B above 100K; hardware not stated"}
        log(f"[bench] all-Full group {ms_af:.2f} ms vs IndexShare {ms_step:.2f} ms")
        if not args.no_stack:
            result["stack80"] = bench_stack(dsa, torch, inds, layers, outs, ws, k, stream)
        del others, inds, idxs

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 1 << 30
        del a, b

    # free the prefill working set before decode
    del ind, layers, outs, idx
    torch.cuda.empty_cache()

    if not args.no_prefill16k and cfg.name != "prefill16k":
        result["prefill16k"] = bench_prefill16k(dsa, synth, accounting, torch, np, dev, stream)

    if not args.no_decode:
        result["decode"] = bench_decode(args, dsa, synth, accounting, torch, np, dev, stream)

    if not args.no_chunk1m:
        result["chunk1m"] = bench_chunk1m(args, dsa, synth, accounting, torch, np, dev, stream)

    if not args.no_quant:
        result["quantize"] = bench_quantize(dsa, torch, np, dev, stream)
        result["projections"] = bench_projections(dsa, torch, np, dev, stream)
    if not args.no_attainable:
        # context only: what torch's library GEMMs and a device copy reach on this GPU (the
        # roofline fractions are taken against the datasheet peaks, never against these)
        result["library_reference"] = bench_attainable(torch, dev, stream)
    if not args.no_train:
        result["indexer_training"] = bench_objective(dsa, synth, torch, dev, stream)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(cfg)

    print(json.dumps(result), flush=True)


def bench_prefill16k(dsa, synth, accounting, torch, np, dev, stream, steps=3):
    """The 16384-token prefill group with a bf16 indexer (H_I = 64, d_I = 128), k = 2048:
    one fused indexer + top-k, then the 4 layers' sparse MLA attention, timed like the
    headline step."""
    cfg = synth.get_config("prefill16k")
    L, k = cfg.L, cfg.topk
    ind = synth.indexer_inputs(cfg, device=dev)
    layers = [synth.attention_inputs(cfg, layer=l, device=dev) for l in range(cfg.n_layers)]
    idx = torch.empty((1, L, k), dtype=torch.int32, device=dev)
    outs = [torch.empty((1, L, cfg.H, cfg.Dv), dtype=torch.bfloat16, device=dev) for _ in range(cfg.n_layers)]
    ws = dsa.Workspace()

    def step(ev):
        ev[0].record(stream)
        dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, ws=ws, out=idx)
        ev[1].record(stream)
        for l in range(cfg.n_layers):
            dsa.sparse_attn(layers[l], idx, ws=ws, out=outs[l])
        ev[2].record(stream)

    step([torch.cuda.Event(enable_timing=True) for _ in range(3)])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    step_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in evs]))
    idx_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) / cfg.n_layers
    idx_flop = accounting.indexer_flops(accounting.causal_pairs(L, L), cfg.H_I, cfg.d_I)
    attn_flop = accounting.attention_flops(accounting.selected_pairs(L, k, L), cfg.H, cfg.Dqk, cfg.Dv)
    out = {"workload": cfg.name, "L": L, "topk": k, "indexer_dtype": "bf16", "step_ms": round(step_ms, 3),
           "tokens_per_s": round(L / (step_ms * 1e-3), 1),
           "indexer_topk_ms": round(idx_ms, 4),
           "indexer_frac": round(idx_flop / (idx_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
           "attn_ms_per_layer": round(attn_ms, 4),
           "attn_frac": round(attn_flop / (attn_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4)}
    log(f"[bench] prefill16k group {step_ms:.2f} ms (indexer+topk {idx_ms:.3f} ms, attention {attn_ms:.3f} ms/layer)")
    del ind, layers, outs, idx, ws
    torch.cuda.empty_cache()
    return out


def bench_stack(dsa, torch, inds, layers, outs, ws, k, stream, n=80):
    """An n-layer stack run one call per layer (dsa.LayerStack), under three schedules:
    20 x FSSS (freq 4, offset 0), the released configuration (freq 4, offset 3) and
    all-Full (every layer runs its own indexer).  Layer l uses the operands of group
    position l % 4 (the workload's four layers), so the stack needs no more memory."""
    res = {"layers": n, "workload_layers_reused": len(layers)}
    sched = {"fsss": dsa.layer_schedule(n, freq=4, offset=0),
             "released_freq4_offset3": dsa.layer_schedule(n, freq=4, offset=3),
             "all_full": dsa.layer_schedule(n, freq=1, offset=0)}
    for name, anchors in sched.items():
        st = dsa.LayerStack(anchors, k, ws=ws)
        m = len(layers)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for l in range(n):
            st.layer(l, layers[l % m], indexer=inds[l % m] if st.is_full(l) else None, out=outs[l % m])
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = {"full_layers": st.n_full, "s": round(e0.elapsed_time(e1) / 1e3, 3)}
        log(f"[bench] {n}-layer stack, {name}: {st.n_full} Full layers, {res[name]['s']:.3f} s")
        del st
    res["all_full_over_fsss"] = round(res["all_full"]["s"] / res["fsss"]["s"], 3)
    return res


def bench_decode(args, dsa, synth, accounting, torch, np, dev, stream):
    cfg = synth.get_config("decode200k")
    k = cfg.topk
    log(f"[bench] decode: B={cfg.B} Lk={cfg.L} fp8 indexer, {cfg.n_layers} layers")
    ind = synth.indexer_inputs(cfg, device=dev)
    layers = [synth.attention_inputs(cfg, layer=l, device=dev) for l in range(cfg.n_layers)]
    idx = torch.empty((cfg.B, 1, k), dtype=torch.int32, device=dev)
    outs = [torch.empty((cfg.B, 1, cfg.H, cfg.Dv), dtype=torch.bfloat16, device=dev) for _ in range(cfg.n_layers)]
    ws = dsa.Workspace()
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, q_scale=ind["q_scale"], k_scale=ind["k_scale"],
                         ws=ws, out=idx)
        if ev is not None:
            ev[1].record(stream)
        for l in range(cfg.n_layers):
            dsa.sparse_attn(layers[l], idx, ws=ws, out=outs[l])
        if ev is not None:
            ev[2].record(stream)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    n = max(args.steps, 5)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for s in range(n):
        step(evs[s])
    torch.cuda.synchronize()
    step_ms = float(np.median([e[0].elapsed_time(e[2]) for e in evs]))
    idx_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    attn_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs])) / cfg.n_layers
    kI_bytes = cfg.B * cfg.L * (cfg.d_I + 4)               # fp8 keys + fp32 scale
    gather_bytes = cfg.B * k * cfg.Dqk * 2                 # selected latent rows per layer
    log(f"[bench] decode step {step_ms * 1e3:.1f} us (indexer+topk {idx_ms * 1e3:.1f} us, "
        f"attention {attn_ms * 1e3:.1f} us/layer)")
    # the same caches as a variable-length batch: sequence b holds its first lens[b] keys,
    # lengths seeded uniform in [Lk/2, Lk]; bandwidth over the keys actually held
    lens_np = np.random.default_rng(5).integers(cfg.L // 2, cfg.L + 1, cfg.B).astype(np.int32)
    lens = torch.from_numpy(lens_np).to(dev)

    def step_varlen(ev):
        ev[0].record(stream)
        dsa.indexer_topk_varlen(ind["q"], ind["k"], ind["w"], k, lens, q_scale=ind["q_scale"],
                                k_scale=ind["k_scale"], ws=ws, out=idx)
        ev[1].record(stream)
        for l in range(cfg.n_layers):
            dsa.sparse_attn(layers[l], idx, ws=ws, out=outs[l])
        ev[2].record(stream)

    step_varlen([torch.cuda.Event(enable_timing=True) for _ in range(3)])
    torch.cuda.synchronize()
    evv = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for s_ in range(n):
        step_varlen(evv[s_])
    torch.cuda.synchronize()
    v_step = float(np.median([e[0].elapsed_time(e[2]) for e in evv]))
    v_idx = float(np.median([e[0].elapsed_time(e[1]) for e in evv]))
    v_bytes = int(lens_np.astype(np.int64).sum()) * (cfg.d_I + 4)
    varlen = {"lengths": f"seeded uniform in [{cfg.L // 2}, {cfg.L}]", "mean_len": round(float(lens_np.mean()), 1),
              "step_us": round(v_step * 1e3, 1), "indexer_topk_us": round(v_idx * 1e3, 1),
              "indexer_hbm_gbs": round(v_bytes / (v_idx * 1e-3) / 1e9, 1),
              "indexer_hbm_frac": round(v_bytes / (v_idx * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"[bench] decode varlen (mean {lens_np.mean():.0f} keys) step {v_step * 1e3:.1f} us "
        f"(indexer+topk {v_idx * 1e3:.1f} us)")
    # MTP draft step: 4 draft queries per sequence attend with the first step's index row
    # (idx_q_stride = 0); the indexer does not run again, each layer gathers the shared rows
    n_mtp = cfg.mtp
    g4 = torch.Generator(device=dev)
    g4.manual_seed(cfg.seed * 1000 + 77)
    layers_mtp = [{**lay, "q": torch.randn((cfg.B, n_mtp, cfg.H, cfg.Dqk), generator=g4, device=dev,
                                          dtype=torch.float32).to(torch.bfloat16)} for lay in layers]
    outs_mtp = [torch.empty((cfg.B, n_mtp, cfg.H, cfg.Dv), dtype=torch.bfloat16, device=dev) for _ in layers]

    def step_mtp(ev):
        ev[0].record(stream)
        for l in range(cfg.n_layers):
            dsa.sparse_attn(layers_mtp[l], idx, idx_q_stride=0, ws=ws, out=outs_mtp[l])
        ev[1].record(stream)

    step_mtp([torch.cuda.Event(enable_timing=True) for _ in range(2)])
    torch.cuda.synchronize()
    evm = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for s_ in range(n):
        step_mtp(evm[s_])
    torch.cuda.synchronize()
    m_step = float(np.median([e[0].elapsed_time(e[1]) for e in evm]))
    mtp = {"draft_queries": n_mtp, "reuses_index_row": True, "step_us": round(m_step * 1e3, 1),
           "attn_us_per_layer": round(m_step * 1e3 / cfg.n_layers, 1),
           "us_per_draft_token": round(m_step * 1e3 / (cfg.B * n_mtp), 3)}
    log(f"[bench] decode MTP ({n_mtp} draft queries sharing the index row) step {m_step * 1e3:.1f} us "
        f"(attention {m_step * 1e3 / cfg.n_layers:.1f} us/layer)")
    del layers_mtp, outs_mtp
    # FP8 latent caches (E4M3 codes + one fp32 scale per row): the same step with every
    # layer's attention reading 580 bytes per selected row instead of 1152
    layers8 = [synth.fp8_latent(lay) for lay in layers]

    def step_kv8(ev):
        ev[0].record(stream)
        dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, q_scale=ind["q_scale"], k_scale=ind["k_scale"],
                         ws=ws, out=idx)
        ev[1].record(stream)
        for l in range(cfg.n_layers):
            dsa.sparse_attn(layers8[l], idx, ws=ws, out=outs[l])
        ev[2].record(stream)

    step_kv8([torch.cuda.Event(enable_timing=True) for _ in range(3)])
    torch.cuda.synchronize()
    ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for s_ in range(n):
        step_kv8(ev8[s_])
    torch.cuda.synchronize()
    k8_step = float(np.median([e[0].elapsed_time(e[2]) for e in ev8]))
    k8_attn = float(np.median([e[1].elapsed_time(e[2]) for e in ev8])) / cfg.n_layers
    g8 = cfg.B * k * (cfg.Dqk + 4)
    fp8_kv = {"step_us": round(k8_step * 1e3, 1), "attn_us_per_layer": round(k8_attn * 1e3, 1),
              "gathered_mb": round(g8 / 1e6, 1), "attn_gather_gbs": round(g8 / (k8_attn * 1e-3) / 1e9, 1),
              "attn_gather_frac": round(g8 / (k8_attn * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"[bench] decode fp8 latent step {k8_step * 1e3:.1f} us (attention {k8_attn * 1e3:.1f} us/layer)")
    del layers8
    torch.cuda.empty_cache()
    paged = bench_decode_paged(dsa, torch, np, cfg, ind, layers, ws, stream, n, k, dev)
    out = {"workload": cfg.name, "B": cfg.B, "Lk": cfg.L, "step_us": round(step_ms * 1e3, 1),
           "us_per_token": round(step_ms * 1e3 / cfg.B, 2),
           "indexer_topk_us": round(idx_ms * 1e3, 1),
           "indexer_hbm_gbs": round(kI_bytes / (idx_ms * 1e-3) / 1e9, 1),
           "indexer_hbm_frac": round(kI_bytes / (idx_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "attn_us_per_layer": round(attn_ms * 1e3, 1),
           "attn_gather_gbs": round(gather_bytes / (attn_ms * 1e-3) / 1e9, 1),
           "attn_gather_frac": round(gather_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "varlen": varlen, "mtp": mtp, "fp8_latent": fp8_kv, "paged": paged}
    del ind, layers, outs, idx
    torch.cuda.empty_cache()
    return out


def bench_attainable(torch, dev, stream):
    """Measured ceilings on this GPU, for context beside the datasheet peaks: a large bf16
    GEMM and, where torch provides it, an fp8 one (hipBLASLt through torch; measurement only,
    never on the library's path), a 2 GiB device copy (read + write bytes) and a 2 GiB
    reduction (read bytes)."""
    def timed(fn, n=5):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n = 8192
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    a = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    out = {"gemm_shape": [n, n, n]}
    ms = timed(lambda: torch.matmul(a, b))
    out["bf16_gemm_tflops"] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
    try:
        a8 = a.to(torch.float8_e4m3fn)
        b8 = b.to(torch.float8_e4m3fn).t().contiguous().t()      # column-major right operand
        one = torch.ones((), device=dev, dtype=torch.float32)
        ms8 = timed(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
        out["fp8_gemm_tflops"] = round(2.0 * n ** 3 / (ms8 * 1e-3) / 1e12, 1)
        del a8, b8
    except Exception as e:                                     # not provided by this torch build
        out["fp8_gemm_tflops"] = None
        out["fp8_gemm_note"] = f"unavailable: {type(e).__name__}"
    del a, b
    x = torch.empty(1 << 29, device=dev, dtype=torch.float32)
    y = torch.empty_like(x)
    x.fill_(1.0)
    msc = timed(lambda: y.copy_(x))
    out["copy_gbs"] = round(2.0 * x.numel() * 4 / (msc * 1e-3) / 1e9, 1)
    # a read-only stream (a library reduction over 2 GiB, as int64 words): the reference for
    # read-bound kernels
    x64 = x.view(torch.int64)
    msr = timed(lambda: torch.sum(x64))
    out["read_gbs"] = round(x.numel() * 4 / (msr * 1e-3) / 1e9, 1)
    del x, y, x64
    torch.cuda.empty_cache()
    log(f"[bench] attainable: bf16 GEMM {out['bf16_gemm_tflops']} TFLOP/s, fp8 GEMM {out['fp8_gemm_tflops']} "
        f"TFLOP/s, device copy {out['copy_gbs']} GB/s, read {out['read_gbs']} GB/s")
    return out


def bench_quantize(dsa, torch, np, dev, stream):
    """Per-token E4M3 quantization (the step before the path): the q^I of a 131072-token
    prefill (64 heads x 128 dims, bf16 in, codes + per-token scales out; HBM-bound), and
    one decode step's k^I append (64 sequences, one 128-dim row each, written straight
    into their cache slots; launch-bound)."""
    T, H, D = 131072, 64, 128
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    x = torch.randn((T, H * D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    codes = torch.empty((T, H * D), dtype=torch.uint8, device=dev)
    scales = torch.empty(T, dtype=torch.float32, device=dev)

    def timed(fn, n=10):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed(lambda: dsa.quantize_e4m3(x, codes=codes, scales=scales))
    nbytes = T * H * D * 2 + T * H * D + T * 4
    del x, codes, scales
    B, Lmax, p = 64, 200001, 200000
    cache = torch.zeros((B, Lmax, D), dtype=torch.uint8, device=dev)
    sc_cache = torch.zeros((B, Lmax), dtype=torch.float32, device=dev)
    new = torch.randn((B, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    us_app = timed(lambda: dsa.quantize_e4m3(new, codes=cache[:, p], scales=sc_cache[:, p]), n=50) * 1e3
    del cache, sc_cache
    torch.cuda.empty_cache()
    log(f"[bench] quantize: q^I prefill {ms:.3f} ms ({nbytes / (ms * 1e-3) / 1e9:.0f} GB/s), decode append {us_app:.1f} us")
    return {"prefill_qI_tokens": T, "prefill_ms": round(ms, 4), "prefill_hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "prefill_hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_append_rows": B, "decode_append_us": round(us_app, 2)}


def bench_projections(dsa, torch, np, dev, stream):
    """The indexer's projections (the step before the path) for one 4096-token prefill
    chunk: q^I = h W_Q (64 x 128 outputs), k^I = h W_K (128) and w = h W_w (64) from
    hidden states of width D = 6144 (a stand-in: the pages give no width), bf16 in, fp32
    out, then the per-token E4M3 quantization of q^I and k^I.  The q^I map is the
    MFMA-bound part; its rate is reported against the bf16 peak."""
    T, D, H_I, d_I = 4096, 6144, 64, 128
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    h = torch.randn((T, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    wq = (torch.randn((H_I * d_I, D), generator=g, device=dev, dtype=torch.float32) * D ** -0.5).to(torch.bfloat16)
    wk = (torch.randn((d_I, D), generator=g, device=dev, dtype=torch.float32) * D ** -0.5).to(torch.bfloat16)
    ww = (torch.randn((H_I, D), generator=g, device=dev, dtype=torch.float32) * D ** -0.5).to(torch.bfloat16)
    yq = torch.empty((T, H_I * d_I), dtype=torch.float32, device=dev)

    def timed(fn, n=10):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_q = timed(lambda: dsa.linear_bf16(h, wq, out=yq))
    ms_all = timed(lambda: dsa.indexer_projections(h, wq, wk, ww, H_I))
    fl_q = 2.0 * T * H_I * d_I * D
    tf_q = fl_q / (ms_q * 1e-3) / 1e12
    del h, wq, wk, ww, yq
    torch.cuda.empty_cache()
    log(f"[bench] projections: q^I map {ms_q:.3f} ms ({tf_q:.0f} TFLOP/s, {tf_q / MFMA_PEAK_TFLOPS['bf16'] * 100:.1f}% "
        f"of bf16 peak); q^I + k^I + w with quantization {ms_all:.3f} ms per {T} tokens")
    return {"tokens": T, "hidden": D, "qI_map_ms": round(ms_q, 4), "qI_map_tflops": round(tf_q, 1),
            "qI_map_frac": round(tf_q / MFMA_PEAK_TFLOPS["bf16"], 4), "all_ms": round(ms_all, 4)}


def bench_objective(dsa, synth, torch, dev, stream):
    """Training of the kept indexer at the 16K bf16 prefill (L = 16384, H_I = 64, d_I = 128,
    k = 2048, 4 MLA layers of 32 heads): the group centroid of the 4 layers' head-averaged
    distributions on each index row (dsa_attn_probs per layer, from the lse of its sparse
    attention), then the KL backward of the indexer (loss, dq, dw, dk).  Work: the centroid
    rescores every selected (query, key) pair per layer, 2 * 32 * 576 flops; the backward
    scores each pair twice and runs the dq and dk contractions, 4 * 2 * 64 * 128 flops."""
    cfg = synth.get_config("prefill16k")
    ind = synth.indexer_inputs(cfg, device=dev)
    layers = [synth.attention_inputs(cfg, layer=l, device=dev) for l in range(cfg.n_layers)]
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], cfg.topk)
    lses = [dsa.sparse_attn(lay, idx, return_lse=True)[1] for lay in layers]
    pbar = torch.zeros(idx.shape, dtype=torch.float32, device=dev)
    dk = torch.zeros(ind["k"].shape, dtype=torch.float32, device=dev)
    ws = dsa.Workspace()

    def centroid():
        pbar.zero_()
        dsa.attention_centroid(layers, idx, lses, out=pbar)

    def backward():
        dk.zero_()
        return dsa.indexer_kl_backward(ind["q"], ind["k"], ind["w"], idx, pbar, dk=dk, ws=ws)

    def timed(fn, n=3):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_c = timed(centroid)
    ms_b = timed(backward)
    sel = int((idx >= 0).sum())
    fl_c = 2.0 * cfg.H * cfg.Dqk * sel * len(layers)
    fl_b = 4 * 2.0 * cfg.H_I * cfg.d_I * sel
    tf_c, tf_b = fl_c / (ms_c * 1e-3) / 1e12, fl_b / (ms_b * 1e-3) / 1e12
    loss = float(backward()["loss"].mean())
    del ind, layers, idx, lses, pbar, dk
    torch.cuda.empty_cache()
    log(f"[bench] indexer training (16K bf16): centroid of 4 layers {ms_c:.2f} ms ({tf_c:.0f} TFLOP/s), "
        f"KL backward {ms_b:.2f} ms ({tf_b:.0f} TFLOP/s), mean loss {loss:.4f}")
    return {"workload": cfg.name, "selected_pairs": sel, "centroid_ms": round(ms_c, 3),
            "centroid_tflops": round(tf_c, 1), "kl_backward_ms": round(ms_b, 3), "kl_backward_tflops": round(tf_b, 1),
            "bf16_frac_centroid": round(tf_c / MFMA_PEAK_TFLOPS["bf16"], 4),
            "bf16_frac_kl_backward": round(tf_b / MFMA_PEAK_TFLOPS["bf16"], 4)}


def bench_decode_paged(dsa, torch, np, cfg, ind, layers, ws, stream, n, k, dev, page=64):
    """The decode step over paged caches: every sequence's k^I, key scales and latent rows
    in 64-position pages of shared pools, pages placed by a seeded random permutation; the
    Full layer's positions are translated to pool rows once (dsa_paged_rows) and the 4
    attention layers gather from their pools.  The layers' contiguous caches are replaced by
    their pools one by one (the work per step is that of the contiguous step)."""
    B, L = cfg.B, cfg.L
    max_pages = (L + page - 1) // page
    pool_pages = B * max_pages
    perm = torch.from_numpy(np.random.default_rng(9).permutation(pool_pages).astype(np.int64)).to(dev)
    table = perm.view(B, max_pages).to(torch.int32).contiguous()
    # pool row of (b, position): table[b, pos / page] * page + pos % page; inverse map by scatter
    pos = torch.arange(max_pages * page, device=dev)
    src = torch.full((pool_pages * page,), -1, dtype=torch.int64, device=dev)
    for b in range(B):
        prow = perm[b * max_pages + pos // page] * page + pos % page
        valid = pos < L
        src[prow[valid]] = b * L + pos[valid]
    del pos

    def to_pool(cache):
        flat = cache.reshape(B * L, -1)
        out = flat[src.clamp(min=0)]
        out[src < 0] = 0
        return out.reshape((pool_pages * page,) + tuple(cache.shape[2:]))

    kpool = to_pool(ind["k"])
    spool = to_pool(ind["k_scale"][..., None])[:, 0].contiguous()
    pools = []
    for l in range(len(layers)):
        kv = layers[l].pop("kv")
        pl = dict(layers[l])
        pl["q"] = layers[l]["q"].reshape(1, B, cfg.H, cfg.Dqk)
        pl["kv"] = to_pool(kv)[None]
        del kv
        torch.cuda.empty_cache()
        pools.append(pl)
    del src
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    rows = torch.empty_like(idx)
    outs = [torch.empty((1, B, cfg.H, cfg.Dv), dtype=torch.bfloat16, device=dev) for _ in pools]

    def step(ev):
        ev[0].record(stream)
        dsa.indexer_topk_paged(ind["q"], kpool, ind["w"], k, lens, table, page, q_scale=ind["q_scale"],
                               k_scale_pool=spool, ws=ws, out=idx)
        dsa.paged_rows(idx, table, page, pool_pages, out=rows)
        ev[1].record(stream)
        for l, pl in enumerate(pools):
            dsa.sparse_attn(pl, rows.view(1, B, k), ws=ws, out=outs[l])
        ev[2].record(stream)

    step([torch.cuda.Event(enable_timing=True) for _ in range(3)])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for s_ in range(n):
        step(evs[s_])
    torch.cuda.synchronize()
    st = float(np.median([e[0].elapsed_time(e[2]) for e in evs]))
    ix = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    at = float(np.median([e[1].elapsed_time(e[2]) for e in evs])) / len(pools)
    log(f"[bench] decode paged (page {page}) step {st * 1e3:.1f} us (indexer+topk+rows {ix * 1e3:.1f} us, "
        f"attention {at * 1e3:.1f} us/layer)")
    del kpool, spool, pools, outs, idx, rows
    torch.cuda.empty_cache()
    return {"page": page, "placement": "seeded random page permutation", "step_us": round(st * 1e3, 1),
            "indexer_topk_rows_us": round(ix * 1e3, 1), "attn_us_per_layer": round(at * 1e3, 1)}


def bench_chunk1m(args, dsa, synth, accounting, torch, np, dev, stream):
    """1,048,576-token prefill in 4096-query chunks, timed once over all 256 chunks: per
    chunk the Full layer's fused indexer + top-k against the (c+1)*4096 keys so far, then
    the sparse attention of the group's 4 layers.  The attention queries of one chunk are
    drawn once per layer and reused by every chunk (the work per chunk is unchanged); the
    indexer queries, keys and weights cover the whole sequence."""
    cfg = synth.get_config("chunk1m")
    L, C, k = cfg.L, cfg.chunk, cfg.topk
    n_chunks = L // C
    log(f"[bench] chunk1m: L={L} in {n_chunks} chunks of {C}, fp8 indexer, {cfg.n_layers} layers")
    ind = synth.indexer_inputs(cfg, device=dev, Lq=L)
    layers = [synth.attention_inputs(cfg, layer=l, device=dev, Lq=C) for l in range(cfg.n_layers)]
    idx = torch.empty((1, C, k), dtype=torch.int32, device=dev)
    out = torch.empty((1, C, cfg.H, cfg.Dv), dtype=torch.bfloat16, device=dev)
    ws = dsa.Workspace()
    torch.cuda.synchronize()

    def chunk(c, ev=None):
        lo, hi = c * C, (c + 1) * C
        if ev is not None:
            ev[0].record(stream)
        dsa.indexer_topk(ind["q"][:, lo:hi], ind["k"][:, :hi], ind["w"][:, lo:hi], k,
                         q_scale=ind["q_scale"][:, lo:hi], k_scale=ind["k_scale"][:, :hi], ws=ws, out=idx)
        if ev is not None:
            ev[1].record(stream)
        for lay in layers:
            dsa.sparse_attn({**lay, "kv": lay["kv"][:, :hi]}, idx, ws=ws, out=out)
        if ev is not None:
            ev[2].record(stream)

    for c in (0, n_chunks - 1):                       # warm-up: smallest and largest chunk
        chunk(c)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_chunks)]
    t0 = time.time()
    for c in range(n_chunks):
        chunk(c, evs[c])
    torch.cuda.synchronize()
    wall = time.time() - t0
    idx_ms = [e[0].elapsed_time(e[1]) for e in evs]
    attn_ms = [e[1].elapsed_time(e[2]) / cfg.n_layers for e in evs]
    t_idx = sum(idx_ms) / 1e3                      # one Full layer's indexer over the sequence
    t_attn = sum(attn_ms) / 1e3                    # one layer's attention over the sequence
    group = t_idx + cfg.n_layers * t_attn
    last_pairs = accounting.causal_pairs(L, C)
    last_tfs = accounting.indexer_flops(last_pairs, cfg.H_I, cfg.d_I) / (idx_ms[-1] * 1e-3) / 1e12
    all_pairs = accounting.causal_pairs(L, L)
    idx_tfs = accounting.indexer_flops(all_pairs, cfg.H_I, cfg.d_I) / t_idx / 1e12
    log(f"[bench] chunk1m: indexer+topk {t_idx:.2f} s/layer, attention {t_attn * 1e3:.1f} ms/layer, "
        f"group {group:.2f} s (wall {wall:.1f} s)")
    out_d = {"workload": cfg.name, "L": L, "chunk": C, "chunks": n_chunks,
             "indexer_topk_s_per_full_layer": round(t_idx, 4),
             "indexer_tflops": round(idx_tfs, 1), "indexer_frac": round(idx_tfs / MFMA_PEAK_TFLOPS["fp8"], 4),
             "last_chunk_indexer_ms": round(idx_ms[-1], 3),
             "last_chunk_indexer_tflops": round(last_tfs, 1),
             "attn_s_per_layer": round(t_attn, 4),
             "group_s": round(group, 3), "tokens_per_s": round(L / group, 1),
             "all_full_group_s_derived": round(cfg.n_layers * (t_idx + t_attn), 3),
             "stack80": {"indexshare_20_full_s": round(20 * group, 1),
                         "all_80_full_s": round(80 * (t_idx + t_attn), 1),
                         "note": "derived from the measured per-layer indexer and attention times"}}
    del ind, layers, idx, out
    torch.cuda.empty_cache()
    return out_d


def cpu_baseline(cfg, target_s=15.0):
    """The fp64 oracle on a bounded sample of query rows of the same workload (full group:
    indexer scores, top-k, 4 dense-masked attentions), timed on the host cores."""
    import numpy as np
    import torch
    import oracle
    import synth
    from tests._helpers import to_f64, attn_to_oracle
    from threadpoolctl import threadpool_limits

    cores = len(os.sched_getaffinity(0))
    log(f"[bench] cpu oracle on {cores} host cores")
    rng = np.random.default_rng(0)
    cand = sorted(cfg.Lq - 1 - int(x) for x in rng.integers(0, cfg.Lq // 2, 64))
    ind = synth.indexer_inputs(cfg, device="cuda:0")
    qI = to_f64(ind["q"][0, cand])
    wI = to_f64(ind["w"][0, cand])
    qs = None if ind["q_scale"] is None else to_f64(ind["q_scale"][0, cand])
    kI = to_f64(ind["k"][0])
    ks = None if ind["k_scale"] is None else to_f64(ind["k_scale"][0])
    del ind
    ol = []
    for l in range(cfg.n_layers):
        lay = synth.attention_inputs(cfg, layer=l, device="cuda:0")
        ol.append(attn_to_oracle({**lay, "q": lay["q"][:, cand]}))
        del lay
        torch.cuda.empty_cache()
    done = 0
    with threadpool_limits(limits=cores):
        t0 = time.time()
        for r_i, r in enumerate(cand):
            p = cfg.L - cfg.Lq + r                      # absolute position of this query
            # a single query at position p: pass it as the last of (L - p) queries
            sc = oracle.indexer_scores_rows(qI[r_i:r_i + 1], kI, wI[r_i:r_i + 1], [0], cfg.L,
                                            None if qs is None else qs[r_i:r_i + 1], ks, cfg.L - p)
            sel = oracle.topk_rows(sc, [p + 1], cfg.topk)
            for lay in ol:
                oracle.sparse_attention_rows(lay["q"][0][[r_i]], lay["k"][0], lay["v"][0], sel,
                                             lay["sm_scale"], 1)
            done += 1
            if time.time() - t0 > target_s:
                break
        dt = time.time() - t0
    return {"value": round(done / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} query rows (from the last half of the {cfg.L}-token sequence) through the "
                      f"whole group: fp64 indexer scores over all causal keys, exact top-{cfg.topk}, "
                      f"{cfg.n_layers} dense-masked attentions; {dt:.1f} s"}


if __name__ == "__main__":
    main()
