"""HBM traffic of one kernel from rocprofv3 counter runs, calibrated on a copy.

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are collected in two separate
rocprofv3 --pmc runs of the same command.  Their scale is checked on a plain
device copy of known size (this module's ``copy`` mode), so the reported bytes
are counter * (bytes the copy moves / what the counter reads for the copy).

  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/copy_fetch -o run -- \
      python3 -m equivariant_gnn_tensor_receiver_amd.profiling copy
  rocprofv3 --pmc WRITE_SIZE ... (same, copy_write)
  rocprofv3 --pmc FETCH_SIZE ... -d OUT/wl_fetch -- python3 bench.py --workload W --steps 2 --warmup 1 --no-cpu-baseline
  rocprofv3 --pmc WRITE_SIZE ... -d OUT/wl_write -- (same)
  python3 -m equivariant_gnn_tensor_receiver_amd.profiling summarize OUT W KERNEL_SUBSTRING NAME > traffic.json

A kernel trace (``rocprofv3 --kernel-trace --stats --output-format csv -d DIR``)
is turned into a short Markdown table with

  python3 -m equivariant_gnn_tensor_receiver_amd.profiling stats DIR TITLE "COMMAND" > kernels.md

The summary records the hash of the kernel's sources it was taken with;
bench.py ignores it once those sources change.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

COPY_BYTES = 1 << 30  # 1 GiB read and 1 GiB written per copy
COPY_REPS = 4
HERE = os.path.dirname(os.path.abspath(__file__))
SHARED_SOURCES = ("stream_impl.h", "device_common.h", "kernels.h", "cg_codegen.cpp", "plan.cpp")
KERNEL_SOURCES = {
    "stream": ("stream_gf.h", "stream_gf.hip"),
    "stream_bwdpos": ("stream_pos.h", "stream_pos.hip"),
    "stream_hess": ("stream_pos.h", "stream_pos.hip"),
    "gemm": ("gemm.hip",),
    "cw": ("channelwise.hip",),
}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the sources a kernel class is built from (its own and the shared ones)."""
    key = kernel if kernel in KERNEL_SOURCES else ("gemm" if kernel.startswith("gemm") else
                                                   "cw" if kernel.startswith("cw") else "stream")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[key] + SHARED_SOURCES:
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_probe():
    import torch

    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(COPY_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x {COPY_REPS}", flush=True)


def _per_dispatch(run_dir: str, counter: str, match) -> list[float]:
    """Counter value (summed over rows of one dispatch) per matching dispatch."""
    tot = defaultdict(float)
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter or not match(row["Kernel_Name"]):
                continue
            tot[row.get("Dispatch_Id") or row.get("Correlation_Id")] += float(row["Counter_Value"])
    return list(tot.values())


def summarize(out_dir: str, workload: str, kernel_substr: str, name: str) -> dict:
    res = {"workload": workload, "kernel": name, "kernel_match": kernel_substr,
           "source_hash": kernel_source_hash(name)}
    scale = {}
    for counter, tag in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        copy = _per_dispatch(os.path.join(out_dir, f"copy_{tag}"), counter,
                             lambda k: "copy" in k.lower() or "elementwise" in k.lower())
        big = [v for v in copy if v * 1024 > COPY_BYTES / 4]  # the 1 GiB copies, not setup kernels
        if not big:
            raise SystemExit(f"no copy dispatch found for {counter}")
        kib = sum(big) / len(big)
        scale[tag] = COPY_BYTES / (kib * 1024)
        vals = _per_dispatch(os.path.join(out_dir, f"{workload}_{tag}"), counter, lambda k: kernel_substr in k)
        if not vals:
            raise SystemExit(f"no dispatch of {kernel_substr!r} found for {counter}")
        res[f"{tag}_kib_per_dispatch"] = sum(vals) / len(vals)
        res[f"{tag}_dispatches"] = len(vals)
        res[f"copy_{tag}_kib"] = kib
        res[f"{tag}_scale"] = scale[tag]
    res["hbm_bytes_per_launch"] = int(res["fetch_kib_per_dispatch"] * 1024 * scale["fetch"]
                                      + res["write_kib_per_dispatch"] * 1024 * scale["write"])
    return res


def stats_table(run_dir: str, title: str, command: str) -> str:
    """Markdown table of a rocprofv3 --stats kernel summary (durations in microseconds)."""
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {run_dir}")
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# rocprofv3 kernel trace: {title}", "", "Command (from the repository root):", "", "```", command, "```",
           "", "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    out += ["", "Kernel template arguments: gf_kernel<LMAX, K, MODE, fp32 features split hi+lo, bundled units>",
            "with MODE 0 = receiver state (forward), 1 = tangent state, 2 = sender state, 3 = sender",
            "tangent state; pos_kernel<LMAX, K, fp32 features split hi+lo, 16-byte loads, bundled units,",
            "Hessian term>; gemm_lds_kernel<KIND, column tiles, indices per lane half, W split hi+lo, waves",
            "per block> and gemm_kernel<KIND, row tiles, column tiles, indices per lane half, W split hi+lo,",
            "vector loads> with KIND 0 = out, 1 = gS, 2 = g_x, 3 = gW."]
    return "\n".join(out) + "\n"


def main(argv):
    if len(argv) >= 1 and argv[0] == "copy":
        copy_probe()
    elif len(argv) == 5 and argv[0] == "summarize":
        print(json.dumps(summarize(*argv[1:]), indent=1))
    elif len(argv) == 4 and argv[0] == "stats":
        sys.stdout.write(stats_table(*argv[1:]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
