"""Turn rocprofv3 CSV output into the short text summaries kept in this folder.

usage:
  python profiles/summarize.py stats <run_kernel_stats.csv> <title> <command>
  python profiles/summarize.py pmc <workload> <fetch_counter_collection.csv>
         <write_counter_collection.csv> <copy_fetch.csv> <copy_write.csv> <calls>
The pmc mode prints per-kernel FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
the copy-kernel scale factors (a plain 256 MiB device copy), and the scaled
HBM bytes per layer call as JSON.
"""
import collections
import csv
import json
import sys


def stats(path, title, command):
    rows = list(csv.DictReader(open(path)))
    print(f"# {title}\n\ncommand: `{command}`\n")
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        name = r["Name"].split("(")[0].replace("void ", "")
        if name.startswith("at::") or "elementwise" in name:
            continue
        print(f"| {name} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
              f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | {float(r['Percentage']):.1f}% |")


def per_kernel(path, counter):
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"].split("(")[0].replace("void ", "")].append(float(r["Counter_Value"]))
    return vals


def pmc(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    copy_bytes_kib = 256 * 1024
    cf = per_kernel(copy_fetch_csv, "FETCH_SIZE").get("__amd_rocclr_copyBuffer")
    cw = per_kernel(copy_write_csv, "WRITE_SIZE").get("__amd_rocclr_copyBuffer")
    f_scale = copy_bytes_kib / (sum(cf) / len(cf))
    w_scale = copy_bytes_kib / (sum(cw) / len(cw))
    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    out = {"workload": workload, "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "kernels": {}}
    total = 0.0
    for k in fetch:
        if not k.startswith("moe::"):
            continue
        f = sum(fetch[k]) / len(fetch[k])
        w = sum(write.get(k, [0.0])) / max(len(write.get(k, [1])), 1)
        b = (f * f_scale + w * w_scale) * 1024
        out["kernels"][k] = {"fetch_kib": round(f, 1), "write_kib": round(w, 1), "hbm_bytes": int(b)}
        total += b
    out["hbm_bytes_per_call"] = int(total)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4])
    else:
        pmc(*sys.argv[2:7])
