"""Text summaries of rocprofv3 output for the profiles/ folder.

  python -m long_context_sparse_lsa_amd.profile_summary stats KERNEL_STATS_CSV STEPS
      Markdown table of the library's kernels (calls, mean and total time,
      time per step for a run of STEPS steps).

  python -m long_context_sparse_lsa_amd.profile_summary traffic WORKLOAD FETCH_CSV WRITE_CSV
      HBM bytes per launch of each library kernel from two counter runs
      (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; counter_collection.csv). The
      counters are scaled by what they read for the plain device copies that
      bench.py --copy-probe adds to the run (COPY_BYTES read and written
      each), so the table is in bytes of that copy's accounting. Prints the
      lines of profiles/hbm_traffic.txt for WORKLOAD, headed by the hash of
      the kernel sources they were taken on.

Only reads the CSV files it is given; nothing here touches the GPU.
"""
import collections
import csv
import hashlib
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
COPY_BYTES = 1 << 30
KERNELS = ("index_prefill_kernel", "index_decode_kernel", "index_score_kernel", "select_stage_a",
           "select_stage_b", "attn_prefill_kernel", "attn_decode_partial", "attn_decode_merge",
           "block_summary_kernel", "mtp_index_kernel", "attn_bwd_kernel", "bwd_count_kernel",
           "bwd_scan_blocks_kernel", "bwd_scan_totals_kernel", "bwd_scan_add_kernel", "bwd_fill_kernel",
           "bwd_reduce_kernel", "attn_bwd_finish_kernel", "fill_zero_kernel", "kl_warmup_kernel",
           "mfma_probe_kernel", "mfma_probe_data_kernel", "hi_step_kernel", "filter_threshold_kernel",
           "filter_select_kernel", "select_stage_m")


def sources_hash():
    """sha256 over the kernel sources (name and bytes of each csrc file)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


# kernel symbols reported under another timing name (the library times its
# 32-head-wave prefill attention kernel as "attn_prefill_kernel")
ALIASES = {"attn_prefill_shared": "attn_prefill_kernel"}


def base_name(full):
    for k in KERNELS:
        if k in full:
            return k
    for k, v in ALIASES.items():
        if k in full:
            return v
    return None


def stats(path, steps):
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg µs | total ms | ms per step |", "|---|---|---|---|---|"]
    agg = collections.OrderedDict()
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        k = base_name(r["Name"])
        if k is None:
            continue
        name = r["Name"].replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        agg[name] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6)
    for name, (calls, avg, tot) in agg.items():
        out.append(f"| `{name}` | {calls} | {avg:.1f} | {tot:.3f} | {tot / steps:.4f} |")
    return "\n".join(out)


def _per_dispatch(path, counter):
    """{kernel base name or 'copy': [value per dispatch]} of one counter."""
    per = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for key, v in per.items():
        n = names[key]
        k = base_name(n)
        if k is not None:
            out[k].append(v)
        elif "copyBuffer" in n and v * 1024 >= COPY_BYTES // 2:
            out["copy"].append(v)
    return out


def traffic(workload, fetch_csv, write_csv):
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    if not fetch.get("copy") or not write.get("copy"):
        raise SystemExit("no calibration copy found in the counter files (run bench.py with --copy-probe)")
    f_copy = sum(fetch["copy"]) / len(fetch["copy"]) * 1024  # counters are in KiB
    w_copy = sum(write["copy"]) / len(write["copy"]) * 1024
    f_scale, w_scale = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    lines = [f"# {workload}: copy calibration FETCH_SIZE x{f_scale:.4f}, WRITE_SIZE x{w_scale:.4f}"]
    for k in KERNELS:
        if k in fetch and k in write:
            fb = sum(fetch[k]) / len(fetch[k]) * 1024 * f_scale
            wb = sum(write[k]) / len(write[k]) * 1024 * w_scale
            lines.append(f"{workload} {k} fetch_bytes={fb:.0f} write_bytes={wb:.0f} launches={len(fetch[k])}")
    return "\n".join(lines)


def main(argv):
    if len(argv) == 3 and argv[0] == "stats":
        print(stats(argv[1], float(argv[2])))
    elif len(argv) == 4 and argv[0] == "traffic":
        print(f"sources: {sources_hash()}")
        print(traffic(argv[1], argv[2], argv[3]))
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
