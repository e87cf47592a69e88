"""Summaries of rocprofv3 output for the attention kernels.

Reads the CSV files rocprofv3 writes (``-f csv``): ``*_kernel_stats.csv``
from ``--kernel-trace --stats`` and ``*_counter_collection.csv`` from
``--pmc``.  Writes a short text summary and the measured HBM traffic per
launch, which bench.py reports next to the algorithmic bytes.

HBM traffic per launch comes from two separate ``--pmc`` runs of the same
command:
  * reads: the L2-to-memory read requests by size, TCC_EA0_RDREQ_32B,
    _64B and _128B (bytes = 32 n32 + 64 n64 + 128 n128).  The derived
    FETCH_SIZE of this ROCm counts 128-byte requests through TCC_BUBBLE,
    which does not see them: a contiguous 1 GiB copy reads as 0.5 GiB there
    and as 1.000 GiB from the request counters;
  * writes: WRITE_SIZE (KiB).
Each is scaled by what it reads for a plain copy of known size, bench.py
``--calib-copy``: y = -x over 2^28 fp32 (1 GiB read, 1 GiB written).  The
same run also holds the library's interleaved window gather of a
16x512x512x32 bf16 grid (every token's 64 bytes read on its own) and its
scatter, which show the 128-byte line granularity: the gather of 256 MiB
fetches 512 MiB.

Usage (on the files a GPU run wrote):
    python -m vision_transformer_windowed_partition_amd.profiling \\
        --stats DIR --fetch DIR --write DIR --kernel attn_small_kernel \\
        --workload NAME --bench-json FILE --command-stats "..." \\
        --command-fetch "..." --command-write "..." --out-md F.md --out-json F.json
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics

# torch's elementwise kernel (names truncated by rocprofv3 -T); the zero fill
# of the source comes first, the three negations last
LINE_KERNEL, LINE_BYTES = "vectorized_elementwise_kernel", 2 ** 30
# the library's window copy: three gathers (64-byte reads) then three scatters
# (64-byte writes), 2^28 bytes each way
PIECE_KERNEL, PIECE_BYTES = "window_copy_kernel", 2 ** 28
CALIB_LAUNCHES = 3
RDREQ = {"TCC_EA0_RDREQ_32B_sum": 32, "TCC_EA0_RDREQ_64B_sum": 64, "TCC_EA0_RDREQ_128B_sum": 128}


def _one(pattern: str) -> str:
    files = sorted(glob.glob(pattern))
    if not files:
        raise FileNotFoundError(pattern)
    return files[0]


def kernel_stats(stats_dir: str, kernel: str) -> dict:
    """Row of *_kernel_stats.csv whose name contains `kernel` (the largest
    total if several template instances match, their calls summed)."""
    rows = [r for r in csv.DictReader(open(_one(os.path.join(stats_dir, "*kernel_stats.csv"))))
            if kernel in r["Name"]]
    if not rows:
        raise KeyError(f"{kernel} not in kernel stats of {stats_dir}")
    calls = sum(int(r["Calls"]) for r in rows)
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    return {"name": kernel, "calls": calls, "total_ns": total, "avg_ns": total / calls,
            "min_ns": min(float(r["MinNs"]) for r in rows), "max_ns": max(float(r["MaxNs"]) for r in rows),
            "percentage": sum(float(r["Percentage"]) for r in rows)}


def counter_per_dispatch(pmc_dir: str, counter: str, kernel: str) -> list[float]:
    """Values of `counter` for every dispatch of a kernel whose name contains
    `kernel`, in dispatch order (summed over the rows of one dispatch)."""
    per = {}
    for r in csv.DictReader(open(_one(os.path.join(pmc_dir, "*counter_collection.csv")))):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            d = int(r["Dispatch_Id"])
            per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    if not per:
        raise KeyError(f"no {counter} for {kernel} in {pmc_dir}")
    return [per[d] for d in sorted(per)]


def read_bytes_per_dispatch(pmc_dir: str, kernel: str) -> list[float]:
    """L2-to-memory read bytes of every dispatch of `kernel`, from the read
    requests by size."""
    per = [counter_per_dispatch(pmc_dir, c, kernel) for c in RDREQ]
    return [sum(RDREQ[c] * v[i] for c, v in zip(RDREQ, per)) for i in range(len(per[0]))]


def traffic(rdreq_dir: str, write_dir: str, kernel: str) -> dict:
    """Calibrated HBM bytes per launch of `kernel` (median over dispatches)."""
    med = statistics.median
    r_k = med(read_bytes_per_dispatch(rdreq_dir, kernel))
    w_k = med(counter_per_dispatch(write_dir, "WRITE_SIZE", kernel)) * 1024.0
    r_line = med(read_bytes_per_dispatch(rdreq_dir, LINE_KERNEL)[-CALIB_LAUNCHES:])
    w_line = med(counter_per_dispatch(write_dir, "WRITE_SIZE", LINE_KERNEL)[-CALIB_LAUNCHES:]) * 1024.0
    r_gather = med(read_bytes_per_dispatch(rdreq_dir, PIECE_KERNEL)[-2 * CALIB_LAUNCHES:-CALIB_LAUNCHES])
    read_scale = LINE_BYTES / r_line
    write_scale = LINE_BYTES / w_line
    return {"read_bytes_raw": r_k, "write_bytes_raw": w_k,
            "copy_read_bytes": r_line, "copy_write_bytes": w_line,
            "read_scale": read_scale, "write_scale": write_scale,
            "gather64_read_bytes": r_gather, "gather64_useful_bytes": PIECE_BYTES,
            "read_bytes": r_k * read_scale, "write_bytes": w_k * write_scale,
            "hbm_bytes_per_launch": r_k * read_scale + w_k * write_scale}


# Matrix-core counters of one --pmc run: what each kernel issued and how long
# the MFMA pipes were busy.  GRBM_GUI_ACTIVE comes back summed over the
# chip's 8 XCDs (its per-dispatch value divided by the dispatch's duration is
# 8x the clock), so the GPU's busy cycles are that sum / 8, as rocprofv3's own
# MfmaUtil takes the largest instance.  Every matrix instruction in these
# kernels is v_mfma_f32_16x16x32_bf16: 16384 flops, 16 busy cycles of one SIMD
# at the bf16 dense rate (1024 flops per SIMD and clock, 4 SIMDs per CU).
MFMA_COUNTERS = ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
N_XCD, N_SIMD, FLOPS_PER_MFMA, PEAK_BF16 = 8, 1024, 16384, 2.5e15


def dispatch_durations(pmc_dir: str, kernel: str) -> list[float]:
    """Start-to-end seconds of every dispatch of `kernel` in a --pmc run."""
    per = {}
    for r in csv.DictReader(open(_one(os.path.join(pmc_dir, "*counter_collection.csv")))):
        if kernel in r["Kernel_Name"]:
            per[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    return [per[d] for d in sorted(per)]


def mfma_summary(pmc_dir: str, kernel: str, alg_flops: float | None = None) -> dict:
    """Medians over the dispatches of `kernel` of the MFMA_COUNTERS and what
    follows from them: MFMA-pipe utilisation (busy cycles over the SIMDs'
    cycles, rocprofv3's MfmaUtil), vector instructions per MFMA, and the
    executed and algorithmic flop rates over the counted cycles at the
    measured clock, as fractions of the 2.5 PFLOP/s bf16 peak."""
    med = statistics.median
    v = {c: med(counter_per_dispatch(pmc_dir, c, kernel)) for c in MFMA_COUNTERS}
    dur = med(dispatch_durations(pmc_dir, kernel))
    cycles = v["GRBM_GUI_ACTIVE"] / N_XCD
    out = dict(v)
    out.update(dispatch_s=dur, gpu_cycles=cycles, clock_ghz=cycles / dur / 1e9,
               mfma_util=v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * N_SIMD),
               busy_cycles_per_mfma=v["SQ_VALU_MFMA_BUSY_CYCLES"] / max(v["SQ_INSTS_MFMA"], 1.0),
               valu_per_mfma=v["SQ_INSTS_VALU"] / max(v["SQ_INSTS_MFMA"], 1.0),
               executed_flops=v["SQ_INSTS_MFMA"] * FLOPS_PER_MFMA)
    out["executed_frac"] = out["executed_flops"] / dur / PEAK_BF16
    if alg_flops:
        out["alg_flops"] = alg_flops
        out["alg_frac"] = alg_flops / dur / PEAK_BF16
    return out


def mfma_markdown(kernel: str, workload: str, command: str, m: dict) -> list[str]:
    md = [f"# Matrix-core counters: {kernel} on {workload}", "",
          "One `--pmc` pass (medians over the dispatches of the kernel):", "", "```", command, "```", "",
          "| counter | value per launch |", "|---|---|"]
    md += [f"| {c} | {m[c]:.4g} |" for c in MFMA_COUNTERS]
    md += ["", "Derived (GRBM_GUI_ACTIVE is summed over 8 XCDs; every matrix instruction is "
           "v_mfma_f32_16x16x32_bf16, 16384 flops):", "",
           "| quantity | value |", "|---|---|",
           f"| GPU cycles (GRBM_GUI_ACTIVE / 8) | {m['gpu_cycles']:.4g} |",
           f"| dispatch duration under counters | {m['dispatch_s'] * 1e6:.1f} µs |",
           f"| clock (cycles / duration) | {m['clock_ghz']:.2f} GHz |",
           f"| busy cycles per MFMA | {m['busy_cycles_per_mfma']:.2f} |",
           f"| **MFMA utilisation** = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs) | "
           f"**{m['mfma_util']:.3f}** |",
           f"| vector instructions per MFMA (SQ_INSTS_VALU / SQ_INSTS_MFMA) | {m['valu_per_mfma']:.2f} |",
           f"| executed MFMA flops / duration / 2.5 PFLOP/s | {m['executed_frac']:.3f} |"]
    if "alg_frac" in m:
        md += [f"| algorithmic flops ({m['alg_flops'] / 1e9:.1f} GFLOP) / duration / 2.5 PFLOP/s | "
               f"{m['alg_frac']:.3f} |"]
    md += ["", "The utilisation and the executed-flop fraction agree when the busy cycles per MFMA are 16 "
           "and the clock is 2.4 GHz; the executed flops exceed the algorithmic ones by the padded key "
           "slots, the row-sum products and, where taken, the hi + lo operand products. The duration here "
           "is the counter pass's, longer than an unprofiled launch's.", ""]
    return md


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--stats", help="directory of the --kernel-trace --stats run (not needed with --mfma)")
    ap.add_argument("--fetch", help="directory of the --pmc run with the TCC_EA0_RDREQ_{32B,64B,128B} counters")
    ap.add_argument("--write")
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--kernel-sha", default=None)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--bench-json", help="file holding the JSON line bench.py printed in the stats run")
    ap.add_argument("--command-stats", required=True)
    ap.add_argument("--command-fetch", default="")
    ap.add_argument("--command-write", default="")
    ap.add_argument("--out-md", required=True)
    ap.add_argument("--out-json")
    ap.add_argument("--mfma", help="directory of a --pmc run of MFMA_COUNTERS: write only its summary")
    a = ap.parse_args(argv)

    if a.mfma:
        alg = None
        if a.bench_json:
            for line in open(a.bench_json):
                if line.strip().startswith("{") and '"metric"' in line:
                    alg = json.loads(line)["roofline"].get("alg_flops_per_launch")
        m = mfma_summary(a.mfma, a.kernel, alg)
        md = mfma_markdown(a.kernel, a.workload, a.command_stats, m)
        os.makedirs(os.path.dirname(os.path.abspath(a.out_md)), exist_ok=True)
        with open(a.out_md, "w") as f:
            f.write("\n".join(md))
        print("\n".join(md))
        return 0

    st = kernel_stats(a.stats, a.kernel)
    bench = None
    if a.bench_json:
        for line in open(a.bench_json):
            line = line.strip()
            if line.startswith("{") and '"metric"' in line:
                bench = json.loads(line)
    tr = traffic(a.fetch, a.write, a.kernel) if a.fetch and a.write else None

    md = [f"# {a.kernel} on {a.workload}", "",
          "rocprofv3 kernel trace, `--stats` summary:", "", "```", a.command_stats, "```", "",
          "| kernel | calls | avg µs | min µs | max µs | % of GPU time |", "|---|---|---|---|---|---|",
          f"| {st['name']} | {st['calls']} | {st['avg_ns'] / 1e3:.2f} | {st['min_ns'] / 1e3:.2f} | "
          f"{st['max_ns'] / 1e3:.2f} | {st['percentage']:.1f} |", ""]
    if bench is not None:
        r = bench.get("roofline", {})
        md += [f"bench.py in the same run: kernel average {r.get('kernel_ms', float('nan')) * 1e3:.2f} µs "
               f"(HIP events on the launch stream), {bench['value']:.4g} {bench['unit']}, "
               f"roofline {r.get('bound')} {r.get('achieved')} {r.get('unit')} of {r.get('peak')} "
               f"(frac {r.get('frac')}).", ""]
    if tr is not None:
        md += ["HBM traffic per launch (two `--pmc` runs, medians over dispatches):", "", "```",
               a.command_fetch, a.command_write, "```", "",
               "| direction | kernel raw | contiguous copy (1 GiB known) | scale | kernel bytes |",
               "|---|---|---|---|---|",
               f"| read (32·n32 + 64·n64 + 128·n128) | {tr['read_bytes_raw'] / 1e6:.1f} MB | "
               f"{tr['copy_read_bytes'] / 2**30:.4f} GiB | {tr['read_scale']:.4f} | {tr['read_bytes'] / 1e6:.1f} MB |",
               f"| write (WRITE_SIZE) | {tr['write_bytes_raw'] / 1e6:.1f} MB | "
               f"{tr['copy_write_bytes'] / 2**30:.4f} GiB | {tr['write_scale']:.4f} | {tr['write_bytes'] / 1e6:.1f} MB |", "",
               f"Line granularity check: the 64-byte-piece gather of {tr['gather64_useful_bytes'] / 2**20:.0f} MiB "
               f"reads {tr['gather64_read_bytes'] / 2**20:.0f} MiB.", "",
               f"Total {tr['hbm_bytes_per_launch'] / 1e6:.1f} MB per launch"
               + (f" against {bench['roofline']['alg_bytes_per_launch'] / 1e6:.1f} MB algorithmic."
                  if bench is not None and "alg_bytes_per_launch" in bench.get("roofline", {}) else "."), ""]
    os.makedirs(os.path.dirname(os.path.abspath(a.out_md)), exist_ok=True)
    with open(a.out_md, "w") as f:
        f.write("\n".join(md))
    if a.out_json and tr is not None:
        rec = {"workload": a.workload, "kernel": a.kernel, "kernel_sha": a.kernel_sha,
               "command_fetch": a.command_fetch, "command_write": a.command_write, **tr}
        with open(a.out_json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    print("\n".join(md))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
