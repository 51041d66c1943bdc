"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

  python -m attention_g4attn_amd.profsum stats <kernel_stats.csv> --cmd "<command>" --out <file>
  python -m attention_g4attn_amd.profsum traffic --fetch <counter_collection.csv>
      --write <counter_collection.csv> --kernel <name prefix> --copy-bytes N
      --cmd-fetch "<command>" --cmd-write "<command>" --out <file> [--grid N] [--sources ...]
  python -m attention_g4attn_amd.profsum mfma <counter_collection.csv> --kernel <name prefix>
      --cmd "<command>" --out <file> [--grid N] [--sources ...]
  python -m attention_g4attn_amd.profsum raw <counter_collection.csv> --kernel <name prefix>
      --cmd "<command>" --out <file> [--grid N] [--sources ...]

`traffic` scales FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernel by
what the same counters read for the plain device copy of --copy-bytes bytes in
the same run (rocclr's copyBuffer kernel), and records the sha256 of the kernel
sources so a reader can tell whether the figure still describes the code.

`mfma` turns SQ_VALU_MFMA_BUSY_CYCLES (matrix-core busy cycles summed over
the 1024 SIMDs) and SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 matrix work in units of
512 FLOPs) of one kernel into its matrix-core busy fraction over the
dispatch's duration at the 2.4 GHz peak clock, and its executed FLOPs.
"""
import argparse
import csv
import hashlib
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ["attention_g4attn_amd/csrc/prefill.hpp", "attention_g4attn_amd/csrc/common.hpp",
                  "attention_g4attn_amd/csrc/prefill_kv512.hip"]
DECODE_SOURCES = ["attention_g4attn_amd/csrc/decode_bf16.hip", "attention_g4attn_amd/csrc/decode_common.hpp",
                  "attention_g4attn_amd/csrc/common.hpp"]


def source_hash(files=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    lines = [f"# rocprofv3 kernel statistics", f"command: {args.cmd}", "",
             f"{'calls':>6} {'avg_ms':>12} {'total_ms':>12} {'pct':>6}  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e6:>12.4f} "
                     f"{float(r['TotalDurationNs']) / 1e6:>12.3f} {float(r['Percentage']):>6.2f}  "
                     f"{r['Name'][:150]}")
    open(args.out, "w").write("\n".join(lines) + "\n")


def counter(path, name_prefix, counter_name, grid=None):
    """Per-dispatch values of one counter for kernels whose name starts with
    name_prefix (and, given grid, launched with that many work-items)."""
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter_name or not r["Kernel_Name"].startswith(name_prefix):
            continue
        if grid is not None and int(r["Grid_Size"]) != grid:
            continue
        key = r["Dispatch_Id"]
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return list(per.values())


def traffic(args):
    f_k = counter(args.fetch, args.kernel, "FETCH_SIZE", args.grid)
    w_k = counter(args.write, args.kernel, "WRITE_SIZE", args.grid)
    f_c = counter(args.fetch, "__amd_rocclr_copyBuffer", "FETCH_SIZE")
    w_c = counter(args.write, "__amd_rocclr_copyBuffer", "WRITE_SIZE")
    if not (f_k and w_k and f_c and w_c):
        raise SystemExit("kernel or copy dispatches missing from the counter files")
    # the calibration copy is the largest copyBuffer dispatch of the run
    f_scale = args.copy_bytes / (max(f_c) * 1024.0)
    w_scale = args.copy_bytes / (max(w_c) * 1024.0)
    fb = statistics.mean(f_k) * 1024.0 * f_scale
    wb = statistics.mean(w_k) * 1024.0 * w_scale
    lines = [
        "# HBM traffic of one launch, from rocprofv3 counters",
        f"kernel: {args.kernel}",
        f"grid_size: {args.grid if args.grid is not None else 'any'}",
        f"command_fetch: {args.cmd_fetch}",
        f"command_write: {args.cmd_write}",
        f"dispatches: {len(f_k)} (fetch run), {len(w_k)} (write run)",
        f"fetch_size_kib_per_dispatch: {statistics.mean(f_k):.1f}",
        f"write_size_kib_per_dispatch: {statistics.mean(w_k):.1f}",
        f"copy_calibration_bytes: {args.copy_bytes}",
        f"copy_fetch_size_kib: {max(f_c):.1f}",
        f"copy_write_size_kib: {max(w_c):.1f}",
        f"fetch_scale: {f_scale:.5f}",
        f"write_scale: {w_scale:.5f}",
        f"hbm_read_bytes_per_launch: {fb:.6e}",
        f"hbm_write_bytes_per_launch: {wb:.6e}",
        f"hbm_bytes_per_launch: {fb + wb:.6e}",
        f"source_sha256: {source_hash(args.sources)}",
        "sources: " + ", ".join(args.sources),
    ]
    open(args.out, "w").write("\n".join(lines) + "\n")


SIMDS = 1024          # 256 CUs x 4 SIMDs
PEAK_CLOCK_HZ = 2.4e9


def mfma(args):
    busy, mops, dur = [], [], []
    per = {}
    for r in csv.DictReader(open(args.csv)):
        if not r["Kernel_Name"].startswith(args.kernel):
            continue
        if args.grid is not None and int(r["Grid_Size"]) != args.grid:
            continue
        d = per.setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    for d in per.values():
        busy.append(d["SQ_VALU_MFMA_BUSY_CYCLES"])
        mops.append(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"])
        dur.append(d["_ns"] * 1e-9)
    if not per:
        raise SystemExit("kernel dispatches missing from the counter file")
    b, m, t = statistics.mean(busy), statistics.mean(mops), statistics.mean(dur)
    lines = [
        "# Matrix-core activity of one launch, from rocprofv3 counters",
        f"kernel: {args.kernel}",
        f"grid_size: {args.grid if args.grid is not None else 'any'}",
        f"command: {args.cmd}",
        f"dispatches: {len(per)}",
        f"sq_valu_mfma_busy_cycles_per_dispatch: {b:.6e}",
        f"sq_insts_valu_mfma_mops_bf16_per_dispatch: {m:.6e}",
        f"dispatch_seconds: {t:.6f}",
        f"mfma_flops_per_dispatch: {m * 512:.6e}",
        f"mfma_busy_fraction_at_2.4GHz: {b / SIMDS / (t * PEAK_CLOCK_HZ):.4f}",
        f"mfma_tflops: {m * 512 / t / 1e12:.1f}",
        f"source_sha256: {source_hash(args.sources)}",
        "sources: " + ", ".join(args.sources),
    ]
    open(args.out, "w").write("\n".join(lines) + "\n")


def raw(args):
    """Mean per dispatch of every counter (base or derived) the run collected."""
    per = {}
    for r in csv.DictReader(open(args.csv)):
        if not r["Kernel_Name"].startswith(args.kernel):
            continue
        if args.grid is not None and int(r["Grid_Size"]) != args.grid:
            continue
        d = per.setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not per:
        raise SystemExit("kernel dispatches missing from the counter file")
    names = sorted({k for d in per.values() for k in d if k != "_ns"})
    lines = [
        "# Counters of one launch (mean over dispatches), from rocprofv3",
        f"kernel: {args.kernel}",
        f"grid_size: {args.grid if args.grid is not None else 'any'}",
        f"command: {args.cmd}",
        f"dispatches: {len(per)}",
        f"dispatch_seconds: {statistics.mean(d['_ns'] for d in per.values()) * 1e-9:.6f}",
    ]
    lines += [f"{n}: {statistics.mean(d[n] for d in per.values() if n in d):.6g}" for n in names]
    lines += [f"source_sha256: {source_hash(args.sources)}", "sources: " + ", ".join(args.sources)]
    open(args.out, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--sources", nargs="+", default=KERNEL_SOURCES,
                   help="files whose sha256 identifies the kernel version")
    t.add_argument("--grid", type=int, default=None, help="only launches of this grid size")
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("--kernel", required=True)
    m.add_argument("--cmd", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--sources", nargs="+", default=KERNEL_SOURCES,
                   help="files whose sha256 identifies the kernel version")
    m.add_argument("--grid", type=int, default=None, help="only launches of this grid size")
    r = sub.add_parser("raw")
    r.add_argument("csv")
    r.add_argument("--kernel", required=True)
    r.add_argument("--cmd", required=True)
    r.add_argument("--out", required=True)
    r.add_argument("--sources", nargs="+", default=KERNEL_SOURCES,
                   help="files whose sha256 identifies the kernel version")
    r.add_argument("--grid", type=int, default=None, help="only launches of this grid size")
    a = ap.parse_args()
    {"stats": stats, "traffic": traffic, "mfma": mfma, "raw": raw}[a.what](a)


if __name__ == "__main__":
    main()
