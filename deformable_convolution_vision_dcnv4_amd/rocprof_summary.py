"""Summaries of rocprofv3 runs of bench.py, as small text and JSON files.

    python -m deformable_convolution_vision_dcnv4_amd.rocprof_summary \\
        --workload fiit_stage1 --dtype f16 --stats DIR --fetch DIR --write DIR \\
        --command "..." --out PREFIX

--stats:  a `rocprofv3 --kernel-trace --stats --output-format csv` directory;
          the per-kernel table (calls, mean/min/max duration) is kept.
--fetch:  a `rocprofv3 --pmc FETCH_SIZE --output-format csv` directory;
--write:  a `rocprofv3 --pmc WRITE_SIZE --output-format csv` directory.
          Both counters are in KiB per dispatch.  Other counters found in the
          same runs are summarised too: TCC_HIT_sum / TCC_MISS_sum (L2 hit
          rate), SQ_INSTS_VALU, SQ_INSTS_VALU_FMA_F32, SQ_INSTS_LDS (wave
          instructions, reported per (pixel, group) unit as lane operations:
          x 64 / units), SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (share of
          LDS-busy cycles lost to bank conflicts).  Each is scaled by the
          factor that makes it read the known size of the plain device-to-
          device copies bench.py makes of its inputs (the rotating copies:
          each copies x, offset and mask once, so it reads and writes exactly
          their bytes).  The scaled bytes per launch of the operator's kernel
          are its measured HBM traffic.
Writes PREFIX_kernel_trace.txt and, with the counters, PREFIX_hbm_counters.json
and PREFIX_hbm_counters.txt, each with the command that produced the data.
"""
import argparse
import csv
import glob
import json
import os
import statistics
import sys

from . import build
from .workloads import SENSITIVITY, WORKLOADS, module_bytes

COPY_KERNEL = "__amd_rocclr_copyBuffer"
OP_KERNEL_PREFIXES = ("void dcnv4::", "dcnv4::")


def _one(pattern):
    found = sorted(glob.glob(pattern, recursive=True))
    if not found:
        raise SystemExit(f"no file matches {pattern}")
    return found[0]


def kernel_stats(d):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))))
    out = []
    for r in rows:
        out.append({"name": r["Name"], "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3, "percent": float(r["Percentage"])})
    return out


def counter_rows(d, counter):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows if r["Counter_Name"] == counter]


def is_op(name):
    return name.startswith(OP_KERNEL_PREFIXES) and ("k_window" in name or "k_direct" in name)


def scaled_counter(d, counter, copy_bytes_each):
    """(KiB per op dispatch, factor, op dispatches, copy dispatches) for one counter."""
    rows = counter_rows(d, counter)
    copies = [v for n, v in rows if n.startswith(COPY_KERNEL)]
    ops = [v for n, v in rows if is_op(n)]
    if not copies or not ops:
        raise SystemExit(f"{counter}: {len(copies)} copy and {len(ops)} operator dispatches")
    # copies come in (x, offset, mask) triples, in that order
    if len(copies) % 3:
        raise SystemExit(f"{counter}: {len(copies)} copy dispatches, not a multiple of 3")
    known = sum(copy_bytes_each[i % 3] for i in range(len(copies)))
    factor = known / (sum(copies) * 1024.0)
    return statistics.mean(ops), factor, len(ops), len(copies)


def op_mean(dirs, counter):
    """Mean over the operator's dispatches of `counter` in the first of
    `dirs` that holds it; None if none does."""
    for d in dirs:
        if not d:
            continue
        try:
            rows = counter_rows(d, counter)
        except SystemExit:
            continue
        ops = [v for n, v in rows if is_op(n)]
        if ops:
            return statistics.mean(ops)
    return None


def extra_counters(dirs, units):
    """L2 hit rate and per-unit instruction counts from whatever of these
    counters the runs collected."""
    out = {}
    hit, miss = op_mean(dirs, "TCC_HIT_sum"), op_mean(dirs, "TCC_MISS_sum")
    if hit is not None and miss is not None and hit + miss > 0:
        out["l2_hit"] = round(hit / (hit + miss), 4)
        out["l2_hits"] = round(hit)
        out["l2_misses"] = round(miss)
    for name, key in (("SQ_INSTS_VALU", "valu_lane_ops_per_unit"), ("SQ_INSTS_VALU_FMA_F32", "fma_f32_lane_ops_per_unit"),
                      ("SQ_INSTS_LDS", "lds_lane_ops_per_unit")):
        v = op_mean(dirs, name)
        if v is not None:
            out[key] = round(v * 64 / units, 1)
            out[name] = round(v)
    bc, act = op_mean(dirs, "SQ_LDS_BANK_CONFLICT"), op_mean(dirs, "SQ_LDS_IDX_ACTIVE")
    if bc is not None and act:
        out["lds_bank_conflict_share"] = round(bc / act, 3)
        out["SQ_LDS_BANK_CONFLICT"] = round(bc)
        out["SQ_LDS_IDX_ACTIVE"] = round(act)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--dtype", required=True)
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--op", default="forward", choices=("forward", "backward", "softmax", "module"))
    ap.add_argument("--command", required=True, help="the command line of the kernel-trace run")
    ap.add_argument("--counter-command", default=None,
                    help="the command line of the counter runs (COUNTER = FETCH_SIZE, then WRITE_SIZE)")
    ap.add_argument("--out", required=True, help="output path prefix")
    a = ap.parse_args(argv)
    wl = WORKLOADS[a.workload] if a.workload in WORKLOADS else SENSITIVITY[a.workload]
    s = {"f32": 4, "f16": 2, "bf16": 2}[a.dtype]
    Ho, Wo = wl.out_hw()
    x_b = wl.N * wl.H * wl.W * wl.C * s
    off_b = wl.N * Ho * Wo * wl.G * 2 * wl.P * s
    m_b = wl.N * Ho * Wo * wl.G * wl.P * s
    if a.op in ("forward", "softmax"):
        alg = wl.algorithmic_bytes(a.dtype)
        what = f"x {x_b} + offset {off_b} + mask {m_b} + out {x_b}"
    elif a.op == "backward":
        alg = wl.backward_bytes(a.dtype)
        what = (f"x {x_b} + offset {off_b} + mask {m_b} + grad_out {x_b} read; binary32 gradients "
                f"{x_b * 4 // s} + {off_b * 4 // s} + {m_b * 4 // s} written")
    else:
        alg = module_bytes(wl, a.dtype)
        what = f"x_in {x_b} read + out {x_b} written + weights {alg - 2 * x_b}"

    def head(cmd):
        return [f"workload: {wl.describe(a.dtype)} ({a.op})",
                f"algorithmic bytes per launch: {alg} ({what})",
                f"kernel source hash: {build.source_hash()} (forward kernels: {build.source_hash('forward')})",
                f"command: {cmd}", ""]

    if a.stats:
        st = kernel_stats(a.stats)
        lines = head(a.command) + [f"{'calls':>6} {'avg us':>10} {'min us':>10} {'max us':>10} {'% time':>7}  kernel"]
        for r in st:
            lines.append(f"{r['calls']:6d} {r['avg_us']:10.3f} {r['min_us']:10.3f} {r['max_us']:10.3f} "
                         f"{r['percent']:7.2f}  {r['name'][:110]}")
        if a.op in ("forward", "softmax"):
            ops = [r for r in st if is_op(r["name"])]
        elif a.op == "backward":
            ops = [r for r in st if "k_backward" in r["name"] or "k_zero_f32" in r["name"]]
        else:
            ops = [r for r in st if r["name"].startswith(OP_KERNEL_PREFIXES)]
        for r in ops:
            lines.append("")
            lines.append(f"operator kernel: {r['name']}")
            lines.append(f"  mean duration {r['avg_us']:.3f} us")
        if ops:
            # one launch of the operation = one call of its least-called kernel
            launches = min(r["calls"] for r in ops)
            per_launch = sum(r["avg_us"] * r["calls"] for r in ops) / launches
            lines.append("")
            lines.append(f"per launch (all kernels of one {a.op}): {per_launch:.3f} us -> "
                         f"{alg / (per_launch * 1e-6) / 1e9:.1f} GB/s algorithmic = "
                         f"{alg / (per_launch * 1e-6) / 8e12 * 100:.1f}% of 8 TB/s")
        with open(a.out + "_kernel_trace.txt", "w") as fh:
            fh.write("\n".join(lines) + "\n")

    if a.fetch and a.write:
        each = (x_b, off_b, m_b)
        f_kib, f_fac, f_n, f_c = scaled_counter(a.fetch, "FETCH_SIZE", each)
        w_kib, w_fac, w_n, w_c = scaled_counter(a.write, "WRITE_SIZE", each)
        fetch_b = f_kib * 1024.0 * f_fac
        write_b = w_kib * 1024.0 * w_fac
        ccmd = a.counter_command or a.command
        rec = {"workload": a.workload, "dtype": a.dtype,
               "kernel_source_hash": build.source_hash("forward" if a.op == "forward" else "all"),
               "command": ccmd,
               "fetch_kib_per_dispatch": round(f_kib, 3), "fetch_factor": round(f_fac, 4),
               "write_kib_per_dispatch": round(w_kib, 3), "write_factor": round(w_fac, 4),
               "operator_dispatches": [f_n, w_n], "copy_dispatches": [f_c, w_c],
               "hbm_read_bytes_per_launch": round(fetch_b), "hbm_write_bytes_per_launch": round(write_b),
               "hbm_bytes_per_launch": round(fetch_b + write_b),
               "algorithmic_read_bytes": x_b + off_b + m_b, "algorithmic_write_bytes": x_b,
               "algorithmic_bytes_per_launch": alg}
        extra = extra_counters([a.fetch, a.write], wl.units()) if a.op == "forward" else {}
        rec.update(extra)
        with open(a.out + "_hbm_counters.json", "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        lines = head(ccmd) + [
            f"FETCH_SIZE: {f_kib:.1f} KiB per operator dispatch (mean of {f_n}); copy calibration "
            f"factor {f_fac:.4f} ({f_c} copies of known size) -> {fetch_b / 1e6:.2f} MB read "
            f"(algorithmic {(x_b + off_b + m_b) / 1e6:.2f} MB)",
            f"WRITE_SIZE: {w_kib:.1f} KiB per operator dispatch (mean of {w_n}); copy calibration "
            f"factor {w_fac:.4f} -> {write_b / 1e6:.2f} MB written (algorithmic {x_b / 1e6:.2f} MB)",
            f"HBM traffic per launch: {(fetch_b + write_b) / 1e6:.2f} MB = "
            f"{(fetch_b + write_b) / alg:.3f} x algorithmic"]
        if "l2_hit" in extra:
            lines.append(f"L2 (TCC) hit rate: {extra['l2_hit']:.3f} ({extra['l2_hits']} hits, "
                         f"{extra['l2_misses']} misses per dispatch)")
        if "valu_lane_ops_per_unit" in extra:
            lines.append(f"VALU: {extra['valu_lane_ops_per_unit']:.0f} lane operations per (pixel, group) unit "
                         f"(SQ_INSTS_VALU {extra['SQ_INSTS_VALU']} wave instructions per dispatch); "
                         f"FP32 FMA {extra.get('fma_f32_lane_ops_per_unit', float('nan')):.0f} per unit")
        if "lds_lane_ops_per_unit" in extra:
            lines.append(f"LDS: {extra['lds_lane_ops_per_unit']:.0f} lane operations per unit; bank conflicts "
                         f"{extra.get('lds_bank_conflict_share', float('nan')):.3f} of LDS-busy cycles")
        with open(a.out + "_hbm_counters.txt", "w") as fh:
            fh.write("\n".join(lines) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
