"""Short text summaries of rocprofv3 results (rocpd SQLite databases).

    # per-kernel duration statistics of a --kernel-trace --stats run
    python -m decode_megakernel_persistent_amd.profsum stats RUN.db --cmd "<command>" > out.txt

    # HBM traffic of one kernel from two --pmc runs (FETCH_SIZE, WRITE_SIZE),
    # each scaled by what the same counter reads for a plain copy of known size
    python -m decode_megakernel_persistent_amd.profsum traffic --fetch F.db --write W.db \\
        --kernel mk_worker --copy-mib 1024 --algorithmic-bytes N --cmd-fetch "..." --cmd-write "..." > out.txt

Summaries are ``key = value`` lines plus a table, readable by ``read_kv``.
FETCH_SIZE and WRITE_SIZE are reported by rocprofv3 in KiB per dispatch.
"""

from __future__ import annotations

import argparse
import sqlite3
import statistics
import sys
from typing import Dict, List, Tuple


def read_kv(path: str) -> Dict[str, str]:
    out = {}
    with open(path) as f:
        for line in f:
            if " = " in line and not line.startswith(("|", "#")):
                k, v = line.split(" = ", 1)
                out[k.strip()] = v.strip()
    return out


def _kernels(db: str) -> List[Tuple[str, float]]:
    c = sqlite3.connect(db)
    rows = c.execute("select name, duration from kernels").fetchall()
    c.close()
    return [(n, float(d)) for n, d in rows]


def _short(name: str) -> str:
    n = name.split("(")[0] if not name.startswith("void at::") else name[:90]
    return n.replace("void ", "")


def stats(db: str, cmd: str) -> str:
    by: Dict[str, List[float]] = {}
    for n, d in _kernels(db):
        by.setdefault(_short(n), []).append(d / 1000.0)  # ns -> us
    total = sum(sum(v) for v in by.values())
    lines = [f"# rocprofv3 kernel trace summary", f"command = {cmd}", ""]
    lines.append("| kernel | calls | avg us | median us | min us | max us | total us | share |")
    lines.append("|---|---|---|---|---|---|---|---|")
    for n, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {n} | {len(v)} | {statistics.fmean(v):.2f} | {statistics.median(v):.2f} | {min(v):.2f} | "
                     f"{max(v):.2f} | {sum(v):.1f} | {100.0 * sum(v) / total:.1f}% |")
    for n, v in by.items():
        if n.startswith("mk::mk_worker"):
            lines.insert(2, f"mk_worker_avg_us = {statistics.fmean(v):.2f}")
            lines.insert(3, f"mk_worker_calls = {len(v)}")
    return "\n".join(lines) + "\n"


def _counter(db: str, counter: str) -> List[Tuple[str, int, float]]:
    c = sqlite3.connect(db)
    rows = c.execute("select kernel_name, dispatch_id, sum(value) from counters_collection where counter_name = ? "
                     "group by dispatch_id", (counter,)).fetchall()
    c.close()
    return [(n, int(d), float(v)) for n, d, v in rows]


def _split(rows, kernel: str, copy_bytes: int, reps: int = 3):
    mine = [v for n, _, v in rows if kernel in n]
    # the calibration copies: the last `reps` copy dispatches of the run (the
    # profile run issues them after the timed steps)
    copies = [v for n, d, v in sorted(rows, key=lambda r: r[1]) if "copy" in n.lower()][-reps:]
    return mine, copies


def traffic(fetch_db: str, write_db: str, kernel: str, copy_mib: int, algorithmic: float, cmd_f: str,
            cmd_w: str) -> str:
    from . import source_hash
    copy_bytes = copy_mib << 20
    f_rows, w_rows = _counter(fetch_db, "FETCH_SIZE"), _counter(write_db, "WRITE_SIZE")
    f_mine, f_copy = _split(f_rows, kernel, copy_bytes)
    w_mine, w_copy = _split(w_rows, kernel, copy_bytes)
    if not f_mine or not w_mine or not f_copy or not w_copy:
        raise SystemExit(f"missing dispatches: kernel {len(f_mine)}/{len(w_mine)}, copies {len(f_copy)}/{len(w_copy)}")
    f_scale = copy_bytes / (statistics.median(f_copy) * 1024.0)
    w_scale = copy_bytes / (statistics.median(w_copy) * 1024.0)
    fetch_b = statistics.fmean(f_mine) * 1024.0 * f_scale
    write_b = statistics.fmean(w_mine) * 1024.0 * w_scale
    tot = fetch_b + write_b
    lines = ["# HBM traffic per launch from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE in KiB per dispatch)",
             f"command_fetch = {cmd_f}", f"command_write = {cmd_w}", f"kernel = {kernel}",
             f"source_hash = {source_hash()}",
             f"calibration = plain copy of {copy_mib} MiB: FETCH_SIZE reads {statistics.median(f_copy):.0f} KiB "
             f"(scale {f_scale:.4f}), WRITE_SIZE reads {statistics.median(w_copy):.0f} KiB (scale {w_scale:.4f})",
             f"dispatches = {len(f_mine)} (fetch run), {len(w_mine)} (write run)",
             f"fetch_kib_per_launch_raw = {statistics.fmean(f_mine):.0f}",
             f"write_kib_per_launch_raw = {statistics.fmean(w_mine):.0f}",
             f"fetch_bytes_per_launch = {fetch_b:.0f}", f"write_bytes_per_launch = {write_b:.0f}",
             f"traffic_bytes_per_launch = {tot:.0f}"]
    if algorithmic > 0:
        lines.append(f"algorithmic_bytes_per_launch = {algorithmic:.0f}")
        lines.append(f"traffic_over_algorithmic = {tot / algorithmic:.4f}")
    last_f = {d for n, d, v in sorted(f_rows, key=lambda r: r[1]) if "copy" in n.lower()}
    last_w = {d for n, d, v in sorted(w_rows, key=lambda r: r[1]) if "copy" in n.lower()}
    cal = set(sorted(last_f)[-3:]) | set(sorted(last_w)[-3:])

    def keep(n, d):
        return kernel in n or d in cal
    lines += ["", "| dispatch | kernel | FETCH_SIZE KiB |", "|---|---|---|"]
    for n, d, v in f_rows:
        if keep(n, d):
            lines.append(f"| {d} | {_short(n)[:60]} | {v:.0f} |")
    lines += ["", "| dispatch | kernel | WRITE_SIZE KiB |", "|---|---|---|"]
    for n, d, v in w_rows:
        if keep(n, d):
            lines.append(f"| {d} | {_short(n)[:60]} | {v:.0f} |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="action", required=True)
    a = sub.add_parser("stats")
    a.add_argument("db")
    a.add_argument("--cmd", default="")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", default="mk_worker")
    b.add_argument("--copy-mib", type=int, required=True)
    b.add_argument("--algorithmic-bytes", type=float, default=0.0)
    b.add_argument("--cmd-fetch", default="")
    b.add_argument("--cmd-write", default="")
    args = ap.parse_args(argv)
    if args.action == "stats":
        sys.stdout.write(stats(args.db, args.cmd))
    else:
        sys.stdout.write(traffic(args.fetch, args.write, args.kernel, args.copy_mib, args.algorithmic_bytes,
                                 args.cmd_fetch, args.cmd_write))


if __name__ == "__main__":
    main()
