"""Summarise rocprofv3 output of bench.py by kernel and launch grid.

    python -m hybrid_linear_temporal_amd.profile_summary <dir>/<name>_kernel_trace.csv
    python -m hybrid_linear_temporal_amd.profile_summary --counters [--copy-bytes N] <counter_collection.csv> ...

The first form prints a markdown table of kernel, grid (workgroups), launches
and mean / min / max duration in microseconds. The second merges the counter
CSVs of several `rocprofv3 --pmc` runs of the same command (one counter set
per run) and prints, per kernel and grid, the mean per dispatch of every
counter and the figures derived from them:
  clock     GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration (the counter sums the
            eight XCDs' busy cycles);
  MFMA      SQ_VALU_MFMA_BUSY_CYCLES per GRBM_GUI_ACTIVE cycle, as a fraction
            of the same ratio in the library's dense MFMA loop
            (mfma_loop_kernel, hlta_ceiling_mfma_bf16) of the same run;
  LDS conf  SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE;
  wait      SQ_WAIT_ANY / SQ_WAVE_CYCLES (share of wave cycles spent waiting);
  fetch, write  FETCH_SIZE and WRITE_SIZE (KiB) scaled to bytes by what they
            read for the library's streaming copy (copy_stream_kernel,
            hlta_ceiling_copy) of --copy-bytes bytes in the same run.
"""
from __future__ import annotations

import argparse
import collections
import csv
import sys

N_XCD = 8


def short_name(name: str) -> str | None:
    """Readable kernel name of a library kernel, None for other kernels."""
    if "hlta" not in name:
        return None
    short = name
    for pre in ("hlta::(anonymous namespace)::", "void "):
        short = short.replace(pre, "")
    short = short.split("(")[0]
    for mangled, plain in (("16attn_mfma_kernelIDF16bLb1", "attn_mfma_kernel<bf16, ring>"),
                           ("16attn_mfma_kernelIfLb1", "attn_mfma_kernel<float, ring>"),
                           ("16attn_mfma_kernelIDF16bLb0ELb1", "attn_mfma_kernel<bf16, lse>"),
                           ("16attn_mfma_kernelIfLb0ELb1", "attn_mfma_kernel<float, lse>"),
                           ("16attn_mfma_kernelIDF16b", "attn_mfma_kernel<bf16>"),
                           ("16attn_mfma_kernelIf", "attn_mfma_kernel<float>"),
                           ("14gdn_seg_kernelILb0E", "gdn_seg_kernel<maps>"),
                           ("14gdn_seg_kernelILb1EDF16b", "gdn_seg_kernel<outputs, bf16>"),
                           ("14gdn_seg_kernelILb1Ef", "gdn_seg_kernel<outputs, float>"),
                           ("10mix_kernelIDF16b", "mix_kernel<bf16>"),
                           ("10mix_kernelIf", "mix_kernel<float>"),
                           ("15attn_fp8_kernelIDF16b", "attn_fp8_kernel<bf16>"),
                           ("15attn_fp8_kernelIf", "attn_fp8_kernel<float>"),
                           ("15quantize_kernelIDF16b", "quantize_kernel<bf16>"),
                           ("15quantize_kernelIf", "quantize_kernel<float>"),
                           ("13absmax_kernelIDF16b", "absmax_kernel<bf16>"),
                           ("13absmax_kernelIf", "absmax_kernel<float>"),
                           ("14rope_qk_kernelIDF16b", "rope_qk_kernel<bf16>"),
                           ("14rope_qk_kernelIf", "rope_qk_kernel<float>"),
                           ("16rope_ring_kernelIDF16b", "rope_ring_kernel<bf16>"),
                           ("16rope_ring_kernelIf", "rope_ring_kernel<float>"),
                           ("16attn_bwd_dq_mfmaE", "attn_bwd_dq_mfma"),
                           ("18attn_bwd_dkdv_mfmaILb0", "attn_bwd_dkdv_mfma<dK>"),
                           ("18attn_bwd_dkdv_mfmaILb1", "attn_bwd_dkdv_mfma<dV>"),
                           ("17attn_bwd_lse_mfmaE", "attn_bwd_lse_mfma"),
                           ("13attn_bwd_dsumE", "attn_bwd_dsum"),
                           ("14attn_bwd_statsI", "attn_bwd_stats (fp32)"),
                           ("11attn_bwd_dqI", "attn_bwd_dq (fp32)"),
                           ("13attn_bwd_dkdvI", "attn_bwd_dkdv (fp32)"),
                           ("16gdn_bwd_mat_prepI", "gdn_bwd_mat_prep"),
                           ("13gdn_bwd_chainI", "gdn_bwd_chain"),
                           ("16gdn_bwd_mat_gradI", "gdn_bwd_mat_grad"),
                           ("12dmix_partialI", "dmix_partial"),
                           ("10dmix_finalE", "dmix_final")):
        if mangled in short:
            short = plain
            break
    if short.startswith("attn_mfma_kernel<bool"):
        # rocprofv3 demangles the stream-mode (ring) instantiation this way
        short = "attn_mfma_kernel<ring>"
    return short


def summarise(path: str) -> str:
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        short = short_name(r["Kernel_Name"])
        if short is None:
            continue
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        grid = (int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])) // max(wg, 1)
        agg[(short, grid)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| kernel | workgroups | launches | mean us | min us | max us |", "|---|---|---|---|---|---|"]
    for (k, grid), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {k} | {grid} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} |")
    return "\n".join(out)


def _grid(r: dict) -> int:
    return int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1)


def summarise_counters(paths: list[str], copy_bytes: int) -> str:
    vals = collections.defaultdict(lambda: collections.defaultdict(list))   # (kernel, grid) -> counter -> values
    durs = collections.defaultdict(list)                                   # (kernel, grid) -> ns per dispatch
    for path in paths:
        seen = set()
        for r in csv.DictReader(open(path)):
            short = short_name(r["Kernel_Name"])
            if short is None:
                continue
            key = (short, _grid(r))
            vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if (path, r["Dispatch_Id"]) not in seen:
                seen.add((path, r["Dispatch_Id"]))
                durs[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    mean = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}

    def ref(kernel: str) -> dict | None:
        hits = [m for (k, _), m in mean.items() if k == kernel]
        return hits[0] if hits else None

    loop, copy = ref("mfma_loop_kernel"), ref("copy_stream_kernel")
    loop_ratio = (loop["SQ_VALU_MFMA_BUSY_CYCLES"] / loop["GRBM_GUI_ACTIVE"]
                  if loop and "SQ_VALU_MFMA_BUSY_CYCLES" in loop and loop.get("GRBM_GUI_ACTIVE") else None)
    fetch_scale = copy_bytes / (copy["FETCH_SIZE"] * 1024) if copy and copy.get("FETCH_SIZE") else None
    write_scale = copy_bytes / (copy["WRITE_SIZE"] * 1024) if copy and copy.get("WRITE_SIZE") else None

    def pct(x):
        return "" if x is None else f"{100 * x:.1f} %"

    counters = sorted({c for m in mean.values() for c in m})
    head = ["kernel", "workgroups", "dispatches", "mean us", "clock GHz", "MFMA busy vs dense loop", "LDS conf",
            "wait", "fetch GB", "write GB"]
    out = ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    order = sorted(mean, key=lambda k: -sum(durs[k]))
    for k in order:
        m, ns = mean[k], sum(durs[k]) / len(durs[k])
        gui = m.get("GRBM_GUI_ACTIVE")
        clock = f"{gui / N_XCD / ns:.2f}" if gui and ns > 0 else ""
        mfma = (m["SQ_VALU_MFMA_BUSY_CYCLES"] / gui / loop_ratio
                if loop_ratio and gui and "SQ_VALU_MFMA_BUSY_CYCLES" in m else None)
        conf = (m["SQ_LDS_BANK_CONFLICT"] / m["SQ_LDS_IDX_ACTIVE"]
                if m.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in m else None)
        wait = m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"] if m.get("SQ_WAVE_CYCLES") and "SQ_WAIT_ANY" in m else None
        fetch = f"{m['FETCH_SIZE'] * 1024 * fetch_scale / 1e9:.3f}" if fetch_scale and "FETCH_SIZE" in m else ""
        write = f"{m['WRITE_SIZE'] * 1024 * write_scale / 1e9:.3f}" if write_scale and "WRITE_SIZE" in m else ""
        out.append(f"| {k[0]} | {k[1]} | {len(durs[k])} | {ns / 1e3:.1f} | {clock} | {pct(mfma)} | {pct(conf)} | "
                   f"{pct(wait)} | {fetch} | {write} |")
    out.append("")
    out.append("Raw counters (mean per dispatch):")
    out.append("")
    out.append("| kernel | workgroups | " + " | ".join(counters) + " |")
    out.append("|" + "---|" * (len(counters) + 2))
    for k in order:
        out.append(f"| {k[0]} | {k[1]} | " + " | ".join(f"{mean[k][c]:.4g}" if c in mean[k] else ""
                                                      for c in counters) + " |")
    if fetch_scale or write_scale:
        out.append("")
        out.append(f"Scale factors from copy_stream_kernel ({copy_bytes} bytes read and written): "
                   f"FETCH_SIZE x {fetch_scale or float('nan'):.3f}, WRITE_SIZE x {write_scale or float('nan'):.3f}")
    return "\n".join(out)


def traffic_record(paths: list[str], kernel: str, copy_bytes: int) -> dict:
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per dispatch of one kernel (all
    its grids), from counter CSVs that also hold the streaming copy."""
    fetch, write, cf, cw = [], [], [], []
    for path in paths:
        for r in csv.DictReader(open(path)):
            short = short_name(r["Kernel_Name"])
            c, v = r["Counter_Name"], float(r["Counter_Value"])
            if short == kernel:
                (fetch if c == "FETCH_SIZE" else write if c == "WRITE_SIZE" else []).append(v)
            elif short == "copy_stream_kernel":
                (cf if c == "FETCH_SIZE" else cw if c == "WRITE_SIZE" else []).append(v)
    if not (fetch and write and cf and cw):
        raise SystemExit(f"need FETCH_SIZE and WRITE_SIZE of {kernel} and of copy_stream_kernel")
    fs, ws = copy_bytes / (sum(cf) / len(cf) * 1024), copy_bytes / (sum(cw) / len(cw) * 1024)
    total = (sum(fetch) / len(fetch) * fs + sum(write) / len(write) * ws) * 1024
    return {"bytes_per_launch": int(round(total)), "fetch_scale": fs, "write_scale": ws,
            "dispatches": len(fetch)}


def main(argv=None):
    ap = argparse.ArgumentParser(description="summarise rocprofv3 CSVs of bench.py")
    ap.add_argument("paths", nargs="+")
    ap.add_argument("--counters", action="store_true", help="the paths are --pmc counter_collection CSVs")
    ap.add_argument("--copy-bytes", type=int, default=2 << 30,
                    help="bytes the streaming copy moved per dispatch (bench.py's measured ceilings: 2 GiB)")
    ap.add_argument("--traffic-out", help="with --counters: write the HBM-bytes record of --kernel here")
    ap.add_argument("--kernel", help="kernel name as summarised, e.g. 'attn_mfma_kernel<bf16>'")
    ap.add_argument("--workload", default="p480_T31_bf16")
    ap.add_argument("--digest", help="source digest the record is valid for (bench.source_digest)")
    args = ap.parse_args(argv)
    if args.counters and args.traffic_out:
        t = traffic_record(args.paths, args.kernel, args.copy_bytes)
        with open(args.traffic_out, "w") as f:
            f.write(f"# HBM bytes per launch of {args.kernel} on {args.workload} (FETCH_SIZE + WRITE_SIZE, scaled by\n"
                    f"# the streaming copy's readings in the same runs; mean of {t['dispatches']} dispatches); valid\n"
                    f"# only for the kernel source with this digest\n"
                    f"source_digest={args.digest}\nbytes_per_launch={t['bytes_per_launch']}\n"
                    f"fetch_scale={t['fetch_scale']:.4f}\nwrite_scale={t['write_scale']:.4f}\n")
        print(open(args.traffic_out).read())
    elif args.counters:
        print(summarise_counters(args.paths, args.copy_bytes))
    else:
        print(summarise(args.paths[0]))


if __name__ == "__main__":
    sys.exit(main())
