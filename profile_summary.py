"""Turn rocprofv3 output of the benchmark into the short text summaries kept
under profiles/.

  python profile_summary.py trace <kernel_stats.csv> <command> [note] > profiles/X.md
  python profile_summary.py traffic <stream FETCH csv> <copy WRITE csv>
         <bench FETCH csv> <bench WRITE csv> <json path or -> <commands...>
  python profile_summary.py traffic-chunk <the same arguments>

The traffic mode scales each kernel's FETCH_SIZE by what that counter reads
for the 2 GiB tile-streaming read of `bench.py --stream-calibration` (the
attention's own load pattern: 16-byte nontemporal loads of 64-row tiles) and
WRITE_SIZE by what it reads for the plain 64 MiB copy of
`bench.py --copy-calibration`, prints a markdown table, and writes the
attention kernel's bytes per launch to the JSON path (bench.py reads
profiles/attn_qwen_c8_traffic.json while it matches the attention kernel
source); "-" writes no JSON.  The traffic-chunk mode writes instead the
bytes of one chunk_attn_compact call (its attention and merge-and-commit
launches), which bench.py --chunk 64 reads from
profiles/chunk_qwen_c8_chunk64_traffic.json while it matches chunk.hip.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_SRC = os.path.join(ROOT, "compressed_decode_attention_amd", "csrc", "attn.hip")
CHUNK_SRC = os.path.join(ROOT, "compressed_decode_attention_amd", "csrc", "chunk.hip")
COPY_KIB = 64 * 1024
STREAM_KIB = 2 * 1024 * 1024


def short(name: str) -> str:
    ours = "cda::" in name
    name = name.replace("cda::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0] if ours else name[:60]


def trace(stats_csv: str, command: str, note: str = "") -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    print(f"# rocprofv3 kernel trace summary\n\nCommand (from the repository root):\n\n"
          f"```\n{command}\n```\n")
    if note:
        print(note + "\n")
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows[:12]:
        print(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
              f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | "
              f"{float(r['Percentage']):.1f}% |")


def _mean(path: str, pats: tuple) -> dict:
    v = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if any(q in r["Kernel_Name"] for q in pats):
            v[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(x) / len(x) for k, x in v.items()}


# the device-to-device copy of `bench.py --copy-calibration` (the runtime's
# blit kernel, or torch's elementwise copy, depending on the build)
COPY_KERNELS = ("copyBuffer", "direct_copy")
STREAM_KERNELS = ("stream_tiles_kernel",)


def traffic(cf: str, cw: str, bf: str, bw: str, json_path: str, commands: list[str],
            chunk: bool = False) -> None:
    fcal = STREAM_KIB / list(_mean(cf, STREAM_KERNELS).values())[0]
    wcal = COPY_KIB / list(_mean(cw, COPY_KERNELS).values())[0]
    fetch, write = _mean(bf, ("cda::",)), _mean(bw, ("cda::",))
    print("# HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)\n")
    print("Commands (from the repository root), one counter per run:\n\n```")
    for c in commands:
        print(c)
    print("```\n")
    print(f"Calibration: the 2 GiB tile-streaming read reads as FETCH_SIZE x{1 / fcal:.4f} "
          f"of its true KiB and a plain 64 MiB copy as WRITE_SIZE x{1 / wcal:.4f}, so the "
          f"counters below are multiplied by {fcal:.4f} and {wcal:.4f}.\n")
    print("| kernel | fetched MB | written MB |")
    print("|---|---:|---:|")
    for k in fetch:
        print(f"| `{k}` | {fetch[k] * fcal * 1024 / 1e6:.3f} | {write.get(k, 0) * wcal * 1024 / 1e6:.3f} |")
    if json_path == "-":
        return
    if chunk:   # one chunk call: its attention launch and its merge-and-commit launch
        ks = [k for k in fetch if k.startswith("chunk_")]
        rec = {"chunk_src_sha256": hashlib.sha256(open(CHUNK_SRC, "rb").read()).hexdigest(),
               "kernels": ks,
               "fetch_bytes_per_call": sum(fetch[k] for k in ks) * fcal * 1024,
               "write_bytes_per_call": sum(write.get(k, 0) for k in ks) * wcal * 1024,
               "hbm_bytes_per_call": sum(fetch[k] * fcal + write.get(k, 0) * wcal for k in ks) * 1024,
               "fetch_scale": fcal, "write_scale": wcal}
        with open(json_path, "w") as f:
            json.dump(rec, f, indent=1)
        return
    # the decode attention kernel's bytes per launch, for bench.py
    attn = [k for k in fetch if k.startswith("attn_kernel")][0]
    rec = {"attn_src_sha256": hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest(),
           "kernel": attn,
           "fetch_bytes_per_launch": fetch[attn] * fcal * 1024,
           "write_bytes_per_launch": write[attn] * wcal * 1024,
           "hbm_bytes_per_launch": (fetch[attn] * fcal + write[attn] * wcal) * 1024,
           "fetch_scale": fcal, "write_scale": wcal}
    with open(json_path, "w") as f:
        json.dump(rec, f, indent=1)


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(*sys.argv[2:5])
    else:
        traffic(*sys.argv[2:7], sys.argv[7:], chunk=sys.argv[1] == "traffic-chunk")
