"""Summarise a rocprofv3 kernel trace (CSV) of bench.py by kernel and launch grid.

    python -m hybrid_linear_temporal_amd.profile_summary <dir>/<name>_kernel_trace.csv

Prints a markdown table: kernel, grid (workgroups), launches, mean / min / max
duration in microseconds.
"""
from __future__ import annotations

import collections
import csv
import sys


def summarise(path: str) -> str:
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        if "hlta" not in name:
            continue
        short = name
        for pre in ("hlta::(anonymous namespace)::", "void "):
            short = short.replace(pre, "")
        short = short.split("(")[0]
        for mangled, plain in (("16attn_mfma_kernelIDF16bLb1", "attn_mfma_kernel<bf16, ring>"),
                               ("16attn_mfma_kernelIfLb1", "attn_mfma_kernel<float, ring>"),
                               ("16attn_mfma_kernelIDF16b", "attn_mfma_kernel<bf16>"),
                               ("16attn_mfma_kernelIf", "attn_mfma_kernel<float>"),
                               ("14gdn_chain_mfmaIDF16b", "gdn_chain_mfma<bf16>"),
                               ("14gdn_chain_mfmaIf", "gdn_chain_mfma<float>"),
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
                               ("12gdn_bwd_prepI", "gdn_bwd_prep"),
                               ("13gdn_bwd_chainI", "gdn_bwd_chain"),
                               ("14gdn_bwd_tokensI", "gdn_bwd_tokens"),
                               ("12dmix_partialI", "dmix_partial"),
                               ("10dmix_finalE", "dmix_final")):
            if mangled in short:
                short = plain
                break
        if short.startswith("attn_mfma_kernel<bool"):
            # rocprofv3 demangles the stream-mode (ring) instantiation this way
            short = "attn_mfma_kernel<ring>"
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        grid = (int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])) // max(wg, 1)
        agg[(short, grid)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| kernel | workgroups | launches | mean us | min us | max us |", "|---|---|---|---|---|---|"]
    for (k, grid), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {k} | {grid} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} |")
    return "\n".join(out)


if __name__ == "__main__":
    print(summarise(sys.argv[1]))
