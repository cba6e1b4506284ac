"""Summaries of rocprofv3 output for the decode step: per-kernel-class durations and HBM traffic.

The step launches a fixed sequence: the embedding kernel, then per layer QKV GEMV, attention,
merge (present when the step was captured in a graph or the context spans several partitions),
O GEMV, gate-up GEMV, down GEMV, then the LM head GEMV and the argmax reduction (or a copy of the
hidden state).  Several classes share one kernel instantiation (the QKV and LM-head GEMVs, for
example), so dispatches are classified by their place in that sequence, not by name.

Usage (the CSV files are those rocprofv3 writes with --output-format csv):

  python -m decode_step_04_amd.profiling stats --trace run_kernel_trace.csv --n-layers 28 \
      --command "<the command that made the trace>" > summary.md

  python -m decode_step_04_amd.profiling overlap --kernels run_kernel_trace.csv \
      --copies run_memory_copy_trace.csv --title "<workload>" --command "<command>"
      (or --copy-kernel k_copy instead of --copies when a kernel makes the copies)

  python -m decode_step_04_amd.profiling traffic --n-layers 28 --workload <name> \
      --fetch fetch_counter_collection.csv --write write_counter_collection.csv \
      --calib-fetch cf_counter_collection.csv --calib-write cw_counter_collection.csv \
      --calib-bytes 1073741824 --out profiles/traffic.json

FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch and scaled by what the same counters read
for the library's copy kernel moving a known number of bytes each way (the calibration factor),
so the stored figure is in bytes per launch.
"""
import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

CLASSES_PER_LAYER = ("qkv", "attention", "merge", "o_proj", "gate_up", "down")
KERNEL_SOURCES = {  # kernel class -> source file whose change invalidates stored counters
    "qkv": "gemv.hip", "o_proj": "gemv.hip", "gate_up": "gemv.hip", "down": "gemv.hip",
    "lm_head": "gemv.hip", "attention": "attention.hip", "merge": "attention.hip",
    "embed": "misc.hip", "argmax": "misc.hip",
}
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def source_sha(kclass):
    with open(os.path.join(CSRC, KERNEL_SOURCES[kclass]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _dispatches(path):
    """Rows of a kernel-trace or counter-collection CSV, one dict per dispatch, in dispatch order.
    Counter rows (one per counter) are folded into dispatch['counters'][name]."""
    by_id = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            did = int(r["Dispatch_Id"])
            d = by_id.get(did)
            if d is None:
                d = by_id[did] = {"id": did, "name": r["Kernel_Name"], "counters": {}}
                if "Start_Timestamp" in r and r.get("End_Timestamp"):
                    d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                gx = r.get("Grid_Size_X") or r.get("Grid_Size")
                d["grid"] = gx
            if "Counter_Name" in r and r["Counter_Name"]:
                d["counters"][r["Counter_Name"]] = d["counters"].get(r["Counter_Name"], 0.0) + \
                    float(r["Counter_Value"])
    return [by_id[k] for k in sorted(by_id)]


def classify(disp, n_layers):
    """Yields (class, dispatch) for every dispatch inside a complete step sequence."""
    i = 0
    n = len(disp)
    while i < n:
        if not disp[i]["name"].startswith("qd::k_embed"):
            i += 1
            continue
        seq = [("embed", disp[i])]
        j = i + 1
        ok = True
        for _ in range(n_layers):
            for c in CLASSES_PER_LAYER:
                if j >= n:
                    ok = False
                    break
                name = disp[j]["name"]
                if c == "merge" and "k_attn_merge" not in name:
                    continue  # single-partition eager step: no merge launch
                if c == "attention" and "k_attn<" not in name:
                    ok = False
                if c in ("qkv", "o_proj", "gate_up", "down") and "k_gemv" not in name:
                    ok = False
                seq.append((c, disp[j]))
                j += 1
            if not ok:
                break
        if ok and j < n and "k_gemv" in disp[j]["name"]:
            seq.append(("lm_head", disp[j]))
            j += 1
            if j < n and "k_argmax" in disp[j]["name"]:
                seq.append(("argmax", disp[j]))
                j += 1
        if ok:
            yield from seq
            i = j
        else:
            i += 1


def class_table(disp, n_layers, key):
    out = {}
    for c, d in classify(disp, n_layers):
        v = key(d)
        if v is None:
            continue
        e = out.setdefault(c, {"name": d["name"], "values": []})
        e["values"].append(v)
    return out


def cmd_stats(a):
    disp = _dispatches(a.trace)
    tab = class_table(disp, a.n_layers, lambda d: d.get("ns"))
    print(f"# Kernel durations by class\n\nCommand: `{a.command}`\n")
    print("| class | kernel | launches | avg us | median us |")
    print("|---|---|---|---|---|")
    for c, e in sorted(tab.items(), key=lambda kv: -sum(kv[1]["values"])):
        v = e["values"]
        print(f"| {c} | `{e['name'][:60]}` | {len(v)} | {statistics.fmean(v) / 1e3:.3f} | "
              f"{statistics.median(v) / 1e3:.3f} |")


def _calib(path, counter, known_bytes):
    disp = _dispatches(path)
    vals = [d["counters"][counter] for d in disp
            if "k_copy" in d["name"] and counter in d["counters"]]
    if not vals:
        sys.exit(f"no k_copy dispatch with {counter} in {path}")
    kib = statistics.median(vals)
    return known_bytes / (kib * 1024.0), kib


def cmd_traffic(a):
    f_fac, f_kib = _calib(a.calib_fetch, "FETCH_SIZE", a.calib_bytes)
    w_fac, w_kib = _calib(a.calib_write, "WRITE_SIZE", a.calib_bytes)
    fetch = class_table(_dispatches(a.fetch), a.n_layers, lambda d: d["counters"].get("FETCH_SIZE"))
    write = class_table(_dispatches(a.write), a.n_layers, lambda d: d["counters"].get("WRITE_SIZE"))
    res = {}
    for c in fetch:
        if c not in write:
            continue
        fb = statistics.fmean(fetch[c]["values"]) * 1024.0 * f_fac
        wb = statistics.fmean(write[c]["values"]) * 1024.0 * w_fac
        res[c] = {"bytes_per_launch": int(round(fb + wb)), "fetch_bytes": int(round(fb)),
                  "write_bytes": int(round(wb)), "launches": len(fetch[c]["values"]),
                  "kernel": fetch[c]["name"], "source_sha": source_sha(c)}
    tab = {}
    if os.path.exists(a.out):
        with open(a.out) as f:
            tab = json.load(f)
    tab[a.workload] = res
    tab.setdefault("_calibration", {})[a.workload] = {
        "copy_bytes_each_way": a.calib_bytes, "fetch_kib": f_kib, "write_kib": w_kib,
        "fetch_factor": f_fac, "write_factor": w_fac}
    with open(a.out, "w") as f:
        json.dump(tab, f, indent=1, sort_keys=True)
    print(json.dumps(res, indent=1))


def _intervals(path, name=None, exclude=None):
    """(start, end) ns of the rows of a rocprofv3 trace CSV (kernel or memory-copy trace); for a
    kernel trace, only the kernels whose name contains `name`, or all but those containing
    `exclude`."""
    out = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if not (r.get("Start_Timestamp") and r.get("End_Timestamp")):
                continue
            kn = r.get("Kernel_Name", "")
            if name is not None and name not in kn:
                continue
            if exclude is not None and exclude in kn:
                continue
            out.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    return sorted(out)


def _union(iv):
    merged = []
    for a, b in sorted(iv):
        if merged and a <= merged[-1][1]:
            merged[-1][1] = max(merged[-1][1], b)
        else:
            merged.append([a, b])
    return merged


def _length(m):
    return sum(b - a for a, b in m)


def _intersect(x, y):
    i = j = 0
    tot = 0
    while i < len(x) and j < len(y):
        a, b = max(x[i][0], y[j][0]), min(x[i][1], y[j][1])
        if a < b:
            tot += b - a
        if x[i][1] < y[j][1]:
            i += 1
        else:
            j += 1
    return tot


def overlap(kernels, copies, skip=0.2):
    """Copy / compute overlap over the window from the first copy to the last one, the first
    `skip` fraction of that window dropped (warm-up): busy time of each engine (union of its
    intervals), their intersection, and the fractions of each hidden under the other."""
    c_all = _union(copies)
    if not c_all:
        return None
    t0, t1 = c_all[0][0], c_all[-1][1]
    t0 += int((t1 - t0) * skip)
    clip = lambda m: [[max(a, t0), min(b, t1)] for a, b in m if b > t0 and a < t1]  # noqa: E731
    k, c = clip(_union(kernels)), clip(c_all)
    both = _intersect(k, c)
    wall = t1 - t0
    return {"window_us": wall / 1e3, "kernel_busy_us": _length(k) / 1e3,
            "copy_busy_us": _length(c) / 1e3, "both_busy_us": both / 1e3,
            "copy_hidden_under_kernels": both / max(1, _length(c)),
            "kernels_hidden_under_copies": both / max(1, _length(k)),
            "either_busy_frac": (_length(k) + _length(c) - both) / max(1, wall),
            "copies": sum(1 for a, b in copies if b > t0 and a < t1),
            "kernels": sum(1 for a, b in kernels if b > t0 and a < t1)}


def cmd_overlap(a):
    if a.copy_kernel:  # copies made by a kernel: split the kernel trace by name
        res = overlap(_intervals(a.kernels, exclude=a.copy_kernel),
                      _intervals(a.kernels, name=a.copy_kernel), a.skip)
    else:
        res = overlap(_intervals(a.kernels), _intervals(a.copies), a.skip)
    print(f"# Copy / compute overlap: {a.title}\n\nCommand: `{a.command}`\n")
    if res is None:
        print("no memory copies in the trace")
        return
    print("| quantity | value |\n|---|---|")
    for k, v in res.items():
        print(f"| {k} | {v:.3f} |" if isinstance(v, float) else f"| {k} | {v} |")


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--trace", required=True)
    s.add_argument("--n-layers", type=int, required=True)
    s.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "calib_fetch", "calib_write", "workload", "out"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--n-layers", type=int, required=True)
    o = sub.add_parser("overlap")
    o.add_argument("--kernels", required=True)
    o.add_argument("--copies", default=None, help="memory-copy trace CSV")
    o.add_argument("--copy-kernel", default=None,
                   help="the copies are dispatches of this kernel in the kernel trace")
    o.add_argument("--title", default="")
    o.add_argument("--command", default="")
    o.add_argument("--skip", type=float, default=0.2)
    a = p.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "overlap": cmd_overlap}[a.cmd](a)


if __name__ == "__main__":
    main()
