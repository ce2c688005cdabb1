"""Summaries of rocprofv3 output for the profiles/ directory.

Not used by the library itself; it turns the raw files a profiling run
leaves in its output directory into the short text summaries that are kept:

  python -m io_aware_softmax_02_amd.profile_summary trace  DB_GLOB TITLE COMMAND
      kernel-trace statistics (a --kernel-trace --stats database) as markdown
  python -m io_aware_softmax_02_amd.profile_summary counters CSV TITLE COMMAND
      per-dispatch averages of every counter in a --pmc CSV as markdown
  python -m io_aware_softmax_02_amd.profile_summary traffic FETCH_CSV WRITE_CSV OUT_JSON
      HBM bytes per launch from FETCH_SIZE / WRITE_SIZE passes, calibrated
      against a 512 MiB device copy made in the same process (bench.py makes
      one before its timed region); bench.py reads OUT_JSON
  python -m io_aware_softmax_02_amd.profile_summary traffic-table FETCH_CSV WRITE_CSV TITLE COMMAND
      calibrated HBM bytes per dispatch of every kernel in a run, as markdown
  python -m io_aware_softmax_02_amd.profile_summary fp32 LOG
      the JSON lines of `bench.py --fp32` as markdown
  python -m io_aware_softmax_02_amd.profile_summary contrast LOG
      the JSON lines of `bench.py --contrast` as markdown
  python -m io_aware_softmax_02_amd.profile_summary configs LOG
      the JSON lines of `bench.py --configs` as markdown
  python -m io_aware_softmax_02_amd.profile_summary cpu LOG
      the JSON lines of `bench.py --cpu-configs` as markdown
  python -m io_aware_softmax_02_amd.profile_summary sweep LOG
  python -m io_aware_softmax_02_amd.profile_summary splitkv LOG
      the JSON lines of `bench.py --sweep` / `bench.py --splitkv` as markdown
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import re
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 512 << 20
KERNELS = {"fwd_bf16_kernel": "fwd_bf16", "bwd_dkdv_kernel": "bwd_dkdv_bf16",
           "bwd_dq_kernel": "bwd_dq_bf16", "bwd_pre_kernel": "bwd_pre_bf16",
           "merge_kernel": "merge_bf16"}
# Sources whose digest a traffic record carries: a record is only reported
# while the kernels it measured are unchanged.
TRAFFIC_SOURCES = ["io_aware_softmax_02_amd/csrc/" + x for x in
                   ("attn_fwd_bf16.hip", "attn_bwd_bf16.hip", "lds_tile.h", "device_common.h",
                    "launch_chunks.h")] + \
                  ["io_aware_softmax_02_amd/build.py"]


def short(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    name = re.sub(r"^fa::", "", name)          # the library's own kernels
    return re.sub(r"\(.*", "", name)


def code_digest(path: str) -> str:
    """sha256 of a source file with its // and /* */ comments and all
    whitespace removed: a measurement stays valid across comment edits but
    not across code changes.  (Comment markers inside string literals would
    be stripped too; the kernel sources have none that matter.)"""
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode("utf-8")).hexdigest()


def source_digests() -> dict:
    return {p: code_digest(os.path.join(ROOT, p)) for p in TRAFFIC_SOURCES}


def trace(db_glob: str, title: str, cmd: str) -> str:
    con = sqlite3.connect(glob.glob(db_glob)[0])
    rows = con.execute("select name, total_calls, total_duration, average, percentage "
                       "from top_kernels").fetchall()
    res = {r[0]: r for r in con.execute(
        "select name, lds_size, vgpr_count, accum_vgpr_count, sgpr_count, grid_x, workgroup_x "
        "from kernels group by name").fetchall()}
    durs = collections.defaultdict(list)
    for n, dt in con.execute("select name, duration from kernels"):
        durs[n].append(dt / 1000.0)
    out = [f"# {title}\n", "Command (run from the repository root on one MI355X):\n",
           f"```\n{cmd}\n```\n",
           "| kernel | calls | total µs | average µs | median µs | % | grid (threads) | block | LDS B | arch VGPR | acc VGPR |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for n, calls, tot, avg, pct in rows:
        r = res.get(n)
        d = sorted(durs.get(n, [avg]))
        out.append(f"| `{short(n)}` | {calls} | {tot:.1f} | {avg:.1f} | {d[len(d) // 2]:.1f} | "
                   f"{pct:.1f} | {r[5]} | {r[6]} | {r[1]} | {r[2]} | {r[3]} |")
    return "\n".join(out) + "\n"


def per_dispatch(path: str) -> dict:
    """{kernel: {counter: mean over dispatches of the per-dispatch sum}}"""
    agg = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    for r in csv.DictReader(open(path)):
        agg[short(r["Kernel_Name"])][r["Counter_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return {k: {c: sum(d.values()) / len(d) for c, d in cs.items()} for k, cs in agg.items()}


def calibration(path: str, counter: str) -> float:
    """The counter's value on the calibration copy: the device-copy dispatches
    whose value is within 10% of the largest.  Other copies in the run (tensor
    clones of a few tens of MB, scalar read-backs) can use the same grid but
    move far fewer bytes."""
    rows = [r for r in csv.DictReader(open(path))
            if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter]
    per = collections.defaultdict(float)
    for r in rows:
        per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    top = max(per.values())
    big = [v for v in per.values() if v >= 0.9 * top]
    return sum(big) / len(big)


def counters(path: str, title: str, cmd: str) -> str:
    data = per_dispatch(path)
    names = sorted({c for cs in data.values() for c in cs})
    out = [f"# {title}\n", "Command (run from the repository root on one MI355X):\n",
           f"```\n{cmd}\n```\n",
           "Per-dispatch values, averaged over the profiled dispatches (summed over all XCDs, "
           "shader engines and SIMDs as rocprofv3 reports them).\n",
           "| kernel | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for k, cs in sorted(data.items()):
        out.append(f"| `{k}` | " + " | ".join(f"{cs.get(c, 0):,.0f}" for c in names) + " |")
    return "\n".join(out) + "\n"


def traffic(fetch_csv: str, write_csv: str, out_json: str) -> dict:
    f = {k: v["FETCH_SIZE"] for k, v in per_dispatch(fetch_csv).items() if "FETCH_SIZE" in v}
    w = {k: v["WRITE_SIZE"] for k, v in per_dispatch(write_csv).items() if "WRITE_SIZE" in v}
    cf, cw = calibration(fetch_csv, "FETCH_SIZE"), calibration(write_csv, "WRITE_SIZE")
    rf = COPY_BYTES / (cf * 1024.0)
    wf = COPY_BYTES / (cw * 1024.0)
    sha = source_digests()
    kern = {}
    for k in f:
        for pref, name in KERNELS.items():
            if k.startswith(pref) and "128" in k:
                kern[name] = {"rocprof_name": k, "fetch_size_kib": f[k], "write_size_kib": w.get(k),
                              "read_bytes": f[k] * 1024 * rf, "write_bytes": w.get(k, 0) * 1024 * wf,
                              "source_sha256": sha}
    rx = "|".join(list(KERNELS) + ["copyBuffer"])
    doc = {"what": "HBM traffic per launch at B=1 H=16 N=8192 d=128, from rocprofv3 FETCH_SIZE "
                   "and WRITE_SIZE (KiB per dispatch), each scaled by the same counter on a "
                   "512 MiB device copy run in the same bench process",
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_size_kib": cf,
                           "write_size_kib": cw, "read_factor": rf, "write_factor": wf},
           # the output directories are the ones the two CSVs were read from
           "commands": [f"export TMPDIR=/tmp; rocprofv3 --pmc {c} --kernel-include-regex '{rx}' "
                        f"-f csv -d {os.path.dirname(csv)} -o pmc -- python3 bench.py --steps 2 "
                        f"--warmup 1 --settle 0 --no-cpu-baseline"
                        for c, csv in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv))]
                       + [f"python -m io_aware_softmax_02_amd.profile_summary traffic "
                          f"{fetch_csv} {write_csv} {out_json}"],
           "kernels": kern}
    with open(out_json, "w") as fh:
        json.dump(doc, fh, indent=1)
    return doc


def traffic_table(fetch_csv: str, write_csv: str, title: str, cmd: str) -> str:
    fs, ws = per_dispatch(fetch_csv), per_dispatch(write_csv)
    f = {k: v["FETCH_SIZE"] for k, v in fs.items() if "FETCH_SIZE" in v}
    w = {k: v["WRITE_SIZE"] for k, v in ws.items() if "WRITE_SIZE" in v}
    rf = COPY_BYTES / (calibration(fetch_csv, "FETCH_SIZE") * 1024.0)
    wf = COPY_BYTES / (calibration(write_csv, "WRITE_SIZE") * 1024.0)
    calls = collections.Counter()
    for r in csv.DictReader(open(fetch_csv)):
        calls[short(r["Kernel_Name"])] += 1
    out = [f"# {title}\n", "Command (run from the repository root on one MI355X):\n",
           f"```\n{cmd}\n```\n",
           f"HBM bytes per dispatch: FETCH_SIZE x {rf:.3f} and WRITE_SIZE x {wf:.3f} (factors from "
           f"a {COPY_BYTES >> 20} MiB device copy in the same process), averaged over dispatches.\n",
           "| kernel | read MB | written MB |", "|---|---|---|"]
    for k in sorted(f, key=lambda x: -f[x]):
        if "copyBuffer" in k:
            continue
        name = k if len(k) <= 70 else k[:67] + "..."
        out.append(f"| `{name}` | {f[k] * 1024 * rf / 1e6:.1f} | {w.get(k, 0) * 1024 * wf / 1e6:.1f} |")
    return "\n".join(out) + "\n"


def _json_lines(path: str) -> list:
    return [json.loads(line) for line in open(path) if line.startswith("{")]


def fp32_md(path: str) -> str:
    out = ["# fp32 path (fa_fwd_f32, fa_bwd_f32)\n",
           "Command (repository root, one MI355X): `python bench.py --fp32 > LOG; "
           "python -m io_aware_softmax_02_amd.profile_summary fp32 LOG`\n",
           "Median of three runs of back-to-back launches, HIP events on the launch stream. "
           "d = 64 and 128 run on the fp32 matrix cores (v_mfma_f32_32x32x2_f32); the fp32 peak "
           "is 157.3 TF/s (published). Counted work: 4·B·H·N²·d forward, 14·B·H·N²·d fwd+bwd.\n",
           "| B | H | N | d | fwd ms | bwd ms | fwd TF/s | fwd share of fp32 peak | fwd+bwd TF/s |",
           "|---|---|---|---|---|---|---|---|---|"]
    for r in _json_lines(path):
        out.append(f"| {r['B']} | {r['H']} | {r['N']} | {r['d']} | {r['ms_fwd']:.4f} | {r['ms_bwd']:.4f} | "
                   f"{r['fwd_tflops']} | {r['fwd_frac_of_fp32_peak']:.1%} | {r['fwdbwd_tflops']} |")
    return "\n".join(out) + "\n"


def contrast_md(path: str) -> str:
    out = ["| shape | S = QKᵀ GEMM µs | softmax µs | O = PV GEMM µs | standard total µs | GEMM share of time | "
           "fa_fwd µs | speed-up | N×N bytes per tensor | extra memory, standard | extra memory, fa_fwd | "
           "max abs O difference |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in _json_lines(path):
        out.append(f"| B={r['B']} H={r['H']} N={r['N']} d={r['d']} | {r['ms_S_gemm'] * 1e3:.0f} | "
                   f"{r['ms_softmax'] * 1e3:.0f} | {r['ms_PV_gemm'] * 1e3:.0f} | "
                   f"{r['ms_standard_total'] * 1e3:.0f} | {r['gemm_time_fraction']:.0%} | "
                   f"{r['ms_fa_fwd'] * 1e3:.0f} | {r['ms_standard_total'] / r['ms_fa_fwd']:.1f}x | "
                   f"{r['nxn_bytes_per_tensor'] / 1e9:.2f} GB | {r['peak_extra_bytes_standard'] / 1e9:.2f} GB | "
                   f"{r['peak_extra_bytes_fa_fwd'] / 1e6:.1f} MB | {r['max_abs_diff_O_standard_vs_fa_fwd']} |")
    return "\n".join(out) + "\n"


def sweep_md(path: str) -> str:
    out = ["# Sequence-length sweep (bf16, B = 1, H = 16, d = 128)\n",
           "Command (repository root, one MI355X): `python bench.py --sweep > LOG; "
           "python -m io_aware_softmax_02_amd.profile_summary sweep LOG`\n",
           "Times are the median of several runs of back-to-back launches (HIP events on the "
           "launch stream). fwd+bwd TF/s counts 14·B·H·N²·d over fa_fwd + fa_bwd. `extra bytes` "
           "is the device memory the forward allocates beyond its inputs and outputs (torch "
           "peak-allocation counter); `fp32 S per head` is what one materialised score matrix "
           "would take.\n",
           "| N | fwd µs | fwd TF/s | bwd ms | fwd+bwd TF/s | extra bytes | inputs+outputs MB | fp32 S per head |",
           "|---|---|---|---|---|---|---|---|"]
    for r in _json_lines(path):
        b = r["fp32_scores_per_head_bytes"]
        size = f"{b / 2**30:.2f} GiB" if b >= 2**30 else f"{b / 2**20:.0f} MiB"
        out.append(f"| {r['N']} | {r['ms_fwd'] * 1e3:.0f} | {r['fwd_tflops']} | {r['ms_bwd']:.2f} | "
                   f"{r['fwdbwd_tflops']} | {r['fwd_peak_extra_bytes']} | "
                   f"{r['inputs_outputs_bytes_fwd'] / 1e6:.1f} | {size} |")
    return "\n".join(out) + "\n"


def configs_md(path: str) -> str:
    out = ["# Throughput on every named workload\n",
           "Command (repository root, one MI355X): `python bench.py --configs > LOG; "
           "python -m io_aware_softmax_02_amd.profile_summary configs LOG`\n",
           "Times are the median of five runs of back-to-back launches (HIP events on the launch "
           "stream). Counted work: forward 4·B·H·N²·d, backward 2.5× that. `% peak` is fwd+bwd "
           "against the published dense peak of the dtype (bf16 2500, fp32 157.3 TF/s).\n",
           "| workload | B, H, N, d | dtype | fwd µs | fwd TF/s | bwd µs | fwd+bwd TF/s | % peak |",
           "|---|---|---|---|---|---|---|---|"]
    for r in _json_lines(path):
        out.append(f"| `{r['workload']}` | {r['B']}, {r['H']}, {r['N']}, {r['d']} | {r['dtype']} | "
                   f"{r['ms_fwd'] * 1e3:.1f} | {r['fwd_tflops']} | {r['ms_bwd'] * 1e3:.1f} | "
                   f"{r['fwdbwd_tflops']} | {100 * r['fwdbwd_tflops'] / r['peak_tflops']:.1f} |")
    return "\n".join(out) + "\n"


def cpu_md(path: str) -> str:
    rows = list(_json_lines(path))
    cores = sorted({r["cores"] for r in rows})
    out = ["# The fp64 oracle on the host cores, every named workload\n",
           "Command (repository root, on the host CPUs of the MI355X machine; no GPU work): "
           "`python bench.py --cpu-configs > LOG; "
           "python -m io_aware_softmax_02_amd.profile_summary cpu LOG`\n",
           "The oracle as it stands (numpy float64, materialising S and P), timed on a bounded "
           "sample of each workload with "
           f"{', '.join(str(c) for c in cores)} BLAS threads. TF/s counts the same work as the "
           "GPU figures (forward 4·B·H·N²·d per head or per row share, backward 2.5× the "
           "forward). The last column scales the sample's time to the whole workload and is an "
           "**extrapolation**, not a measurement.\n",
           "| workload | B, H, N, d | sample | seconds | TF/s | whole workload, extrapolated s |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        ext = r.get("extrapolated_all_heads_seconds", r.get("extrapolated_full_forward_seconds"))
        out.append(f"| `{r['cpu_oracle']}` | {r['B']}, {r['H']}, {r['N']}, {r['d']} | "
                   f"{r['sample']} | {r['seconds']} | {r['tflops']:.4f} | {ext} |")
    return "\n".join(out) + "\n"


def splitkv_md(path: str) -> str:
    out = ["# Split-KV forward + merge against the plain forward (bf16, d = 128)\n",
           "Command (repository root, one MI355X): `python bench.py --splitkv > LOG; "
           "python -m io_aware_softmax_02_amd.profile_summary splitkv LOG`\n",
           "Median of five runs of 10 back-to-back launches, HIP events on the launch stream. "
           "`split` is `fa_fwd_split` (fp32 partial O and LSE per key range), `merge` is "
           "`fa_merge`; TF/s counts 4·B·H·N²·d over split + merge. The merge's bytes per "
           "launch are n_split·rows·(4d+4) read + rows·(2d+4) written; its bound is HBM "
           "(8 TB/s published).\n"]
    for r in _json_lines(path):
        out.append(f"\n## B={r['B']} H={r['H']} N={r['N']}: plain fa_fwd {r['plain_ms'] * 1e3:.1f} µs "
                   f"= {r['plain_tflops']} TF/s\n")
        out.append("| n_split | split µs | merge µs | total TF/s | merge GB/s | merge / HBM peak |")
        out.append("|---|---|---|---|---|---|")
        for x in r["splits"]:
            out.append(f"| {x['n_split']} | {x['split_ms'] * 1e3:.1f} | {x['merge_ms'] * 1e3:.1f} | "
                       f"{x['total_tflops']} | {x['merge_GBps']} | {x['merge_frac_of_hbm']} |")
    return "\n".join(out) + "\n"


ALLOC_CALLS = ("hipMalloc", "hipFree", "hipMallocAsync", "hipFreeAsync", "hipMallocManaged",
               "hipHostMalloc", "hipExtMallocWithFlags", "hipMemset", "hipMemsetAsync",
               "hipMemcpy", "hipMemcpyAsync")


def apicalls(trace_dir: str, title: str, cmd: str) -> str:
    """HIP API calls made on the thread of the roctx range `fa_steps`
    between its start and end (rocprofv3 CSV output: *_marker_api_trace.csv
    and *_hip_api_trace.csv in `trace_dir`)."""
    mk = [r for r in csv.DictReader(open(glob.glob(os.path.join(trace_dir, "*_marker_api_trace.csv"))[0]))
          if r["Function"] == "fa_steps"][0]
    t0, t1, tid = int(mk["Start_Timestamp"]), int(mk["End_Timestamp"]), mk["Thread_Id"]
    inside = collections.Counter()
    other_threads = 0
    for r in csv.DictReader(open(glob.glob(os.path.join(trace_dir, "*_hip_api_trace.csv"))[0])):
        if t0 <= int(r["Start_Timestamp"]) <= t1:
            if r["Thread_Id"] == tid:
                inside[r["Function"]] += 1
            else:
                other_threads += 1
    alloc = {k: v for k, v in inside.items() if k.startswith(ALLOC_CALLS)}
    out = [f"# {title}\n", "Command (run from the repository root on one MI355X):\n", f"```\n{cmd}\n```\n",
           f"HIP API calls made between the start and the end of the roctx range `fa_steps` "
           f"({(t1 - t0) / 1000:.1f} µs), on its thread:\n",
           "| HIP API function | calls |", "|---|---|"]
    for k, v in sorted(inside.items(), key=lambda kv: (-kv[1], kv[0])):
        out.append(f"| `{k}` | {v} |")
    out.append("")
    out.append(f"Allocation, free, memset or copy calls inside the range: "
               f"{sum(alloc.values()) if alloc else 0}" + (f" ({alloc})" if alloc else "") + ".")
    out.append(f"HIP calls on other threads inside the range: {other_threads}.")
    return "\n".join(out) + "\n"


def main(argv: list[str]) -> int:
    if len(argv) < 2:
        print(__doc__)
        return 2
    cmd = argv[1]
    if cmd == "trace":
        sys.stdout.write(trace(argv[2], argv[3], argv[4]))
    elif cmd == "counters":
        sys.stdout.write(counters(argv[2], argv[3], argv[4]))
    elif cmd == "traffic-table":
        sys.stdout.write(traffic_table(argv[2], argv[3], argv[4], argv[5]))
    elif cmd == "fp32":
        sys.stdout.write(fp32_md(argv[2]))
    elif cmd == "contrast":
        sys.stdout.write(contrast_md(argv[2]))
    elif cmd == "configs":
        sys.stdout.write(configs_md(argv[2]))
    elif cmd == "cpu":
        sys.stdout.write(cpu_md(argv[2]))
    elif cmd == "sweep":
        sys.stdout.write(sweep_md(argv[2]))
    elif cmd == "splitkv":
        sys.stdout.write(splitkv_md(argv[2]))
    elif cmd == "apicalls":
        sys.stdout.write(apicalls(argv[2], argv[3], argv[4]))
    elif cmd == "traffic":
        doc = traffic(argv[2], argv[3], argv[4])
        for k, v in doc["kernels"].items():
            print(k, round(v["read_bytes"] / 1e6, 1), "MB read", round(v["write_bytes"] / 1e6, 1), "MB written")
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
