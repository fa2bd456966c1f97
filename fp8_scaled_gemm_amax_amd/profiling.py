"""Summaries of rocprofv3 output for this library's kernels (measurement
tooling: nothing on the compute path imports it).

  python -m fp8_scaled_gemm_amax_amd.profiling stats DIR
      kernel table (calls, average / min / max duration, share of GPU time)
      from the *kernel_stats.csv that `rocprofv3 --kernel-trace --stats
      --output-format csv -d DIR` writes.

  python -m fp8_scaled_gemm_amax_amd.profiling trace DIR [--skip N | --skip-frac F]
      per-kernel average duration over the calls after each kernel's first N
      (or first fraction F: warmup / (warmup + steps) of a bench run, whatever
      the kernel's calls per step) from DIR's *kernel_trace.csv.

  python -m fp8_scaled_gemm_amax_amd.profiling counters DIR
      per-kernel average per dispatch of every counter in DIR's
      *counter_collection.csv (`rocprofv3 --pmc ...`).

  python -m fp8_scaled_gemm_amax_amd.profiling mfma DIR [--dispatch-mod M --dispatch-rem R]
      per-kernel matrix-core use from a `rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
      SQ_INSTS_VALU_MFMA_MOPS_F8 GRBM_GUI_ACTIVE` run: MFMA busy cycles over
      (active cycles per XCC x SIMDs), the average shader clock (active cycles
      per XCC over the dispatch's duration) and the FP8 rate the MOPS count
      gives. --dispatch-mod/--dispatch-rem keep a kernel's dispatches whose
      index (in launch order) is R modulo M, for kernels launched on two shapes.

  python -m fp8_scaled_gemm_amax_amd.profiling traffic --key KEY --kernel SUBSTR
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR
        --copy-kernel SUBSTR --copy-bytes N --sources FILE [FILE ...]
      HBM bytes per launch of the kernel whose name contains SUBSTR: its
      FETCH_SIZE and WRITE_SIZE (KiB per dispatch) each scaled by the factor
      that makes the same counter read N bytes for a plain copy kernel that
      reads N and writes N bytes. The record, with a digest of the kernel
      sources it was measured on, is merged into profiles/hbm_traffic.json
      under KEY; bench.py reports it only while the digest still matches.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_scaled_gemm_amax_amd", "csrc")


def source_digest(names):
    """First 16 hex digits of the SHA-256 over the named csrc files, in order."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(dirname, suffix):
    hits = sorted(glob.glob(os.path.join(dirname, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {dirname}")
    return hits[0]


def short_name(name):
    """Kernel name without the argument list and namespace noise."""
    for junk in ("void ", "fp8amax::", "(anonymous namespace)::"):
        name = name.replace(junk, "")
    return name.split("(")[0].strip()


def kernel_stats(dirname):
    rows = list(csv.DictReader(open(_one(dirname, "kernel_stats.csv"))))
    return [{"name": short_name(r["Name"]), "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
             "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
             "total_us": float(r["TotalDurationNs"]) / 1e3, "pct": float(r["Percentage"])} for r in rows]


def trace(dirname, skip, skip_frac=0.0):
    """{kernel name: (calls kept, average us, min us, max us)} over the calls
    after each kernel's first `skip` (or its first `skip_frac` of calls)."""
    per = collections.defaultdict(list)
    rows = sorted(csv.DictReader(open(_one(dirname, "kernel_trace.csv"))), key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        per[short_name(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = {}
    for k, d in per.items():
        s = int(round(skip_frac * len(d))) if skip_frac else skip
        d = d[s:] if len(d) > s else d
        out[k] = (len(d), sum(d) / len(d), min(d), max(d))
    return out


def _counter_rows(dirname, mod=None, rem=None):
    """Rows of DIR's *counter_collection.csv, optionally only each kernel's
    dispatches whose index in launch order is rem modulo mod."""
    rows = list(csv.DictReader(open(_one(dirname, "counter_collection.csv"))))
    if not mod:
        return rows
    order = collections.defaultdict(list)
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        k = short_name(r["Kernel_Name"])
        if r["Dispatch_Id"] not in order[k]:
            order[k].append(r["Dispatch_Id"])
    keep = {d for k, ids in order.items() for i, d in enumerate(ids) if i % mod == rem}
    return [r for r in rows if r["Dispatch_Id"] in keep]


def counters(dirname, mod=None, rem=None):
    """{kernel name: {counter: average value per dispatch}} (a counter's values
    over the instances of one dispatch are summed first)."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in _counter_rows(dirname, mod, rem):
        k = short_name(r["Kernel_Name"])
        per[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    return {k: {c: v / len(disp[k]) for c, v in d.items()} for k, d in per.items()}


def agent_info(dirname):
    """The GPU agent's row of DIR's *agent_info.csv."""
    for r in csv.DictReader(open(_one(dirname, "agent_info.csv"))):
        if r["Agent_Type"] == "GPU":
            return r
    raise SystemExit(f"no GPU agent in {dirname}")


def mfma(dirname, mod=None, rem=None):
    """{kernel: (dispatches, avg us, GHz, MFMA busy %, FP8 TFLOP/s)} for the
    kernels that issue FP8 MFMAs. GRBM_GUI_ACTIVE arrives summed over the XCCs
    (each counts the same active cycles), so it is divided by their number."""
    info = agent_info(dirname)
    xcc, simds = int(info["Num_Xcc"]), int(info["Simd_Count"])
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = collections.defaultdict(dict)
    for r in _counter_rows(dirname, mod, rem):
        k = short_name(r["Kernel_Name"])
        acc[k][r["Counter_Name"]] += float(r["Counter_Value"])
        dur[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    out = {}
    for k, c in acc.items():
        n = len(dur[k])
        t = sum(dur[k].values()) / n
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) / n
        if mops <= 0 or "GRBM_GUI_ACTIVE" not in c:
            continue
        cycles = c["GRBM_GUI_ACTIVE"] / n / xcc
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / n
        out[k] = (n, t * 1e6, cycles / t / 1e9, 100.0 * busy / (cycles * simds), mops * 512 / t / 1e12)
    return out


def _pick(table, substr):
    hits = [k for k in table if substr in k]
    if len(hits) != 1:
        raise SystemExit(f"kernel '{substr}' matches {hits or 'nothing'} in {sorted(table)}")
    return table[hits[0]], hits[0]


def cmd_stats(a):
    print(f"{'kernel':70s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s} {'% time':>7s}")
    for r in kernel_stats(a.dir):
        print(f"{r['name'][:70]:70s} {r['calls']:6d} {r['avg_us']:10.2f} {r['min_us']:10.2f} {r['max_us']:10.2f} "
              f"{r['pct']:7.2f}")


def cmd_trace(a):
    what = f"first {a.skip_frac:g} of" if a.skip_frac else f"first {a.skip}"
    print(f"{'kernel':70s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s}   ({what} calls of "
          f"each kernel skipped)")
    for k, (n, avg, lo, hi) in trace(a.dir, a.skip, a.skip_frac).items():
        print(f"{k[:70]:70s} {n:6d} {avg:10.2f} {lo:10.2f} {hi:10.2f}")


def cmd_counters(a):
    for k, d in counters(a.dir).items():
        print(k)
        for c, v in sorted(d.items()):
            print(f"    {c:32s} {v:16.1f}")


def cmd_mfma(a):
    print(f"{'kernel':60s} {'disp':>5s} {'avg us':>9s} {'GHz':>6s} {'MFMA busy %':>12s} {'FP8 TFLOP/s':>12s}")
    for k, (n, t, ghz, util, tf) in mfma(a.dir, a.dispatch_mod, a.dispatch_rem).items():
        print(f"{k[:60]:60s} {n:5d} {t:9.2f} {ghz:6.3f} {util:12.1f} {tf:12.1f}")


def cmd_traffic(a):
    # one call of the product may launch several kernels (a persistent product
    # and its half-tile tail): their per-dispatch bytes add up
    ftab = counters(a.fetch, a.dispatch_mod, a.dispatch_rem)
    wtab = counters(a.write, a.dispatch_mod, a.dispatch_rem)
    fetch_kib, write_kib, names = 0.0, 0.0, []
    for kern in a.kernel:
        f, kname = _pick(ftab, kern)
        w, _ = _pick(wtab, kern)
        fetch_kib += f["FETCH_SIZE"]
        write_kib += w["WRITE_SIZE"]
        names.append(kname)
    cfetch, cname = _pick(counters(a.copy_fetch), a.copy_kernel)
    cwrite, _ = _pick(counters(a.copy_write), a.copy_kernel)
    f_read = a.copy_bytes / (cfetch["FETCH_SIZE"] * 1024.0)
    f_write = a.copy_bytes / (cwrite["WRITE_SIZE"] * 1024.0)
    read = fetch_kib * 1024.0 * f_read
    written = write_kib * 1024.0 * f_write
    rec = {"kernel": " + ".join(names), "bytes_per_launch": round(read + written), "read_bytes": round(read),
           "write_bytes": round(written), "fetch_kib_raw": fetch_kib, "write_kib_raw": write_kib,
           "copy_kernel": cname, "copy_bytes": a.copy_bytes, "read_factor": round(f_read, 4),
           "write_factor": round(f_write, 4), "sources": a.sources, "source_digest": source_digest(a.sources)}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    table = json.load(open(path)) if os.path.exists(path) else {}
    table[a.key] = rec
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({a.key: rec}, indent=1))


def main(argv=None):
    p = argparse.ArgumentParser(prog="python -m fp8_scaled_gemm_amax_amd.profiling")
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.set_defaults(fn=cmd_stats)
    tr = sub.add_parser("trace")
    tr.add_argument("dir")
    tr.add_argument("--skip", type=int, default=0)
    tr.add_argument("--skip-frac", type=float, default=0.0)
    tr.set_defaults(fn=cmd_trace)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.set_defaults(fn=cmd_counters)
    mf = sub.add_parser("mfma")
    mf.add_argument("dir")
    t = sub.add_parser("traffic")
    for opt in ("--key", "--fetch", "--write", "--copy-fetch", "--copy-write", "--copy-kernel"):
        t.add_argument(opt, required=True)
    t.add_argument("--kernel", nargs="+", required=True, help="the kernels one call launches (bytes summed)")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--sources", nargs="+", required=True)
    for q in (mf, t):
        q.add_argument("--dispatch-mod", type=int, default=None)
        q.add_argument("--dispatch-rem", type=int, default=0)
    mf.set_defaults(fn=cmd_mfma)
    t.set_defaults(fn=cmd_traffic)
    a = p.parse_args(argv)
    a.fn(a)


if __name__ == "__main__":
    sys.exit(main())
