"""Text summaries of rocprofv3 output for the profiles/ folder.

    # per-kernel durations of a run (rocprofv3 --kernel-trace --stats --output-format csv)
    python -m sparse_attention_scores_amd.profile_summary trace STATS_CSV --cmd "..."

    # HBM bytes per dispatch from two counter runs (--pmc FETCH_SIZE, then
    # --pmc WRITE_SIZE, --output-format csv) of a command that also ran the
    # plain copy kernel of bench.py --copy-probe; the copy's own reading
    # calibrates both counters
    python -m sparse_attention_scores_amd.profile_summary traffic \\
        --fetch FETCH_CSV --write WRITE_CSV --copy-bytes N --cmd-fetch "..." --cmd-write "..."

    # matrix-core use per kernel: one counter run (--pmc SQ_INSTS_MFMA
    # SQ_VALU_MFMA_BUSY_CYCLES) and one kernel-trace run of the same command
    python -m sparse_attention_scores_amd.profile_summary mfma \
        --counters COUNTER_CSV --stats STATS_CSV --cmd-counters "..." --cmd-trace "..."

    # which of the library's kernels a run launched (e.g. the GPU test suite
    # under rocprofv3 --kernel-trace --stats), against every __global__
    # kernel defined in csrc
    python -m sparse_attention_scores_amd.profile_summary coverage STATS_CSV --cmd "..."

The traffic record carries a digest of the kernel sources; bench.py only
reports the recorded traffic while the sources still match it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# the calibration copy kernel that bench.py --copy-probe launches
COPY_KERNEL_PATTERN = "probe_copy_kernel"


def source_digest() -> str:
    """sha256 over the device sources (file names and contents, sorted)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if os.path.splitext(path)[1] in (".hip", ".hpp", ".cpp", ".h"):
            h.update(os.path.basename(path).encode())
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    """Kernel name without argument lists; templates kept."""
    n = re.sub(r"^void ", "", name.strip())
    depth, out = 0, []
    for ch in n:  # drop the parenthesised parameter list, keep template args
        if ch == "(":
            depth += 1
        if depth == 0:
            out.append(ch)
        if ch == ")":
            depth -= 1
    return "".join(out).strip()


def trace(stats_csv: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics: {cmd}",
             f"# {'kernel':<78s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"  {short_name(r['Name'])[:78]:<78s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")
    return "\n".join(lines) + "\n"


def _per_dispatch(counter_csv: str, counter: str):
    """Average counter value per dispatch, per kernel (values of one dispatch
    summed over their instances)."""
    tot = defaultdict(float)
    disp = defaultdict(set)
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] != counter:
            continue
        k = short_name(r["Kernel_Name"])
        tot[k] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    return {k: (tot[k] / len(disp[k]), len(disp[k])) for k in tot}


def traffic(fetch_csv: str, write_csv: str, copy_bytes: int, cmd_fetch: str, cmd_write: str) -> str:
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    copy_f = [v for k, (v, _) in fetch.items() if COPY_KERNEL_PATTERN in k]
    copy_w = [v for k, (v, _) in write.items() if COPY_KERNEL_PATTERN in k]
    if not copy_f or not copy_w:
        raise SystemExit("the copy kernel of bench.py --copy-probe is missing from the counter runs")
    ff = copy_bytes / (copy_f[0] * 1024.0)
    wf = copy_bytes / (copy_w[0] * 1024.0)
    lines = [
        "# HBM traffic per dispatch from rocprofv3 counters (KiB per dispatch, as read)",
        f"# FETCH_SIZE run: {cmd_fetch}",
        f"# WRITE_SIZE run: {cmd_write}",
        f"# calibration: the copy kernel moves {copy_bytes} bytes each way; "
        f"bytes = KiB * 1024 * factor",
        f"source_digest {source_digest()}",
        f"copy_bytes {copy_bytes}",
        f"copy_fetch_kib {copy_f[0]:.1f}",
        f"copy_write_kib {copy_w[0]:.1f}",
        f"fetch_factor {ff:.5f}",
        f"write_factor {wf:.5f}",
    ]
    for k in sorted(set(fetch) | set(write)):
        if COPY_KERNEL_PATTERN in k or "dsa::" not in k:
            continue
        f, nf = fetch.get(k, (float("nan"), 0))
        w, nw = write.get(k, (float("nan"), 0))
        lines.append(f"kernel {k.replace(' ', '')} fetch_kib {f:.1f} write_kib {w:.1f} "
                     f"dispatches {min(nf, nw)}")
    return "\n".join(lines) + "\n"


def read_traffic(path: str):
    """Parse a traffic record: (digest, fetch_factor, write_factor,
    {kernel: (fetch_kib, write_kib)})."""
    digest, ff, wf, kern = None, None, None, {}
    for line in open(path):
        p = line.split()
        if not p or p[0].startswith("#"):
            continue
        if p[0] == "source_digest":
            digest = p[1]
        elif p[0] == "fetch_factor":
            ff = float(p[1])
        elif p[0] == "write_factor":
            wf = float(p[1])
        elif p[0] == "kernel":
            kern[p[1]] = (float(p[3]), float(p[5]))
    return digest, ff, wf, kern


# MI355X: 256 CUs x 4 SIMDs, 2.4 GHz at the published dense peaks
N_SIMD, CLOCK_HZ = 1024, 2.4e9


def mfma(counter_csv: str, stats_csv: str, cmd_counters: str, cmd_trace: str) -> str:
    """Per kernel: MFMA instructions and matrix-core busy cycles per dispatch
    (SQ_VALU_MFMA_BUSY_CYCLES is summed over the SIMDs), the kernel's average
    duration from the trace run, and busy cycles / (duration x clock x SIMDs):
    the fraction of the chip's matrix-core time in use at the peak clock."""
    inst = _per_dispatch(counter_csv, "SQ_INSTS_MFMA")
    busy = _per_dispatch(counter_csv, "SQ_VALU_MFMA_BUSY_CYCLES")
    dur = {short_name(r["Name"]): float(r["AverageNs"]) * 1e-9
           for r in csv.DictReader(open(stats_csv))}
    lines = [f"# matrix-core use per kernel (MI355X: {N_SIMD} SIMDs, {CLOCK_HZ / 1e9:.1f} GHz)",
             f"# counters: {cmd_counters}",
             f"# trace:    {cmd_trace}",
             "# use = SQ_VALU_MFMA_BUSY_CYCLES per dispatch / (avg duration x clock x SIMDs)",
             f"# {'kernel':<60s} {'mfma_insts':>12s} {'busy_cycles':>14s} {'avg_us':>10s} {'use':>6s}"]
    for k in sorted(busy, key=lambda k: -busy[k][0]):
        if busy[k][0] <= 0 or k not in dur:
            continue
        use = busy[k][0] / (dur[k] * CLOCK_HZ * N_SIMD)
        lines.append(f"  {k[:60]:<60s} {inst.get(k, (0, 0))[0]:12.0f} {busy[k][0]:14.0f} "
                     f"{dur[k] * 1e6:10.2f} {use:6.3f}")
    return "\n".join(lines) + "\n"


def coverage(stats_csv: str, cmd: str) -> str:
    """The library kernels (dsa::) a run launched, with their calls, and the
    __global__ kernels defined in csrc that it never launched."""
    ran = {}
    for r in csv.DictReader(open(stats_csv)):
        n = short_name(r["Name"])
        if "dsa::" in n:
            ran[n] = ran.get(n, 0) + int(r["Calls"])
    defined = {}
    pat = re.compile(r"__global__\s+(?:__launch_bounds__\([^)]*\)\s+)?void\s+(\w+)\s*\(")
    for path in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        for m_ in pat.finditer(open(path).read()):
            defined[m_.group(1)] = os.path.basename(path)
    base = {re.search(r"dsa::(\w+)", n).group(1) for n in ran}
    missing = sorted(k for k in defined if k not in base)
    lines = [f"# kernels launched by: {cmd}",
             f"# {len(base & set(defined))} of {len(defined)} __global__ kernels in csrc ran "
             f"({len(ran)} template instantiations); never launched: "
             f"{', '.join(missing) if missing else 'none'}",
             f"# {'kernel':<78s} {'calls':>6s}"]
    for n in sorted(ran):
        lines.append(f"  {n[:78]:<78s} {ran[n]:6d}")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("--cmd", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--cmd-fetch", required=True)
    c.add_argument("--cmd-write", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--counters", required=True)
    m.add_argument("--stats", required=True)
    m.add_argument("--cmd-counters", required=True)
    m.add_argument("--cmd-trace", required=True)
    v = sub.add_parser("coverage")
    v.add_argument("stats_csv")
    v.add_argument("--cmd", required=True)
    a = ap.parse_args(argv)
    if a.what == "coverage":
        sys.stdout.write(coverage(a.stats_csv, a.cmd))
    elif a.what == "trace":
        sys.stdout.write(trace(a.stats_csv, a.cmd))
    elif a.what == "mfma":
        sys.stdout.write(mfma(a.counters, a.stats, a.cmd_counters, a.cmd_trace))
    else:
        sys.stdout.write(traffic(a.fetch, a.write, a.copy_bytes, a.cmd_fetch, a.cmd_write))


if __name__ == "__main__":
    main()
