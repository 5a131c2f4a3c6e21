"""Summaries of rocprofv3 CSV output as short markdown (for profiles/).

    python -m layer_streamed_optimizer_amd.rocprof_summary stats  --csv X_kernel_stats.csv --command "..." \
            [--trace X_kernel_trace.csv]
    python -m layer_streamed_optimizer_amd.rocprof_summary pmc    --fetch F.csv --write W.csv --params N \
            --copy-bytes B --command-fetch "..." --command-write "..."
    python -m layer_streamed_optimizer_amd.rocprof_summary stream --trace X_kernel_trace.csv --layers L \
            --copies C --step-bytes B --command "..."

pmc: FETCH_SIZE and WRITE_SIZE are KiB per dispatch.  Each is scaled by
what the same counter reads for the plain copy kernel of known size (it
reads and writes copy-bytes), so the figure is bytes that reached HBM.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# the update kernel's sources and the public header they include (its tile
# size and enum values are part of the kernel's code), relative to here
KERNEL_SOURCES = ("csrc/lso_adam.hip", "csrc/lso_internal.h", "csrc/lso_bf16.h", "../include/lso.h")


_COMMENTS = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def code_of(text: str) -> str:
    """Source text without comments, whitespace collapsed: what the
    compiler sees of it."""
    return " ".join(_COMMENTS.sub(" ", text).split())


def kernel_hash(read=None) -> str:
    """Hash of the update kernel's code (its sources without comments, and
    the build flags): a profile taken with another hash measured another
    kernel.  read(name) returns a source's text (default: the file here)."""
    from . import build
    if read is None:
        def read(name):
            with open(os.path.join(HERE, name), encoding="utf-8") as f:
                return f.read()
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(code_of(read(name)).encode())
    h.update(" ".join(_portable(f, build.ROOT) for f in build.FLAGS).encode())
    return h.hexdigest()[:16]


def _portable(flag: str, root: str) -> str:
    """A build flag without the tree's own location: an include path inside
    the tree counts relative to its root, so a copy of the tree elsewhere
    has the same hash."""
    if flag.startswith("-I"):
        rel = os.path.relpath(flag[2:], root)
        if rel != ".." and not rel.startswith(".." + os.sep):
            return "-I" + rel.replace(os.sep, "/")
    return flag


def short(name: str, n: int = 70) -> str:
    return name if len(name) <= n else name[: n - 3] + "..."


def stats(args) -> str:
    rows = list(csv.DictReader(open(args.csv)))
    out = [f"# rocprofv3 kernel statistics: {args.title}", "",
           f"Command: `{args.command}`", "",
           "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share |",
           "|---|---|---|---|---|---|"]
    for r in rows[: args.top]:
        out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.1f}% |")
    if args.trace:
        # one kernel can serve several workloads in one run (the resident
        # update and the streamed pieces): split its dispatches by grid size
        by = {}
        for r in csv.DictReader(open(args.trace)):
            if args.kernel not in r["Kernel_Name"]:
                continue
            grid = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            key = (r["Kernel_Name"], grid)
            by.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        out += ["", f"Dispatches of `{args.kernel}` by grid (workgroups), from the kernel trace:", "",
                "| Kernel | Workgroups | Calls | Average (us) | Median (us) | Min (us) | Max (us) |",
                "|---|---|---|---|---|---|---|"]
        for (name, grid), d in sorted(by.items(), key=lambda kv: -len(kv[1]) * statistics.mean(kv[1])):
            out.append(f"| `{short(name)}` | {grid:,} | {len(d)} | {statistics.mean(d):.1f} | "
                       f"{statistics.median(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    out.append("")
    out.append(f"kernel_source_sha256: {kernel_hash()}")
    return "\n".join(out) + "\n"


def _per_kernel(path: str) -> dict:
    acc = {}
    for r in csv.DictReader(open(path)):
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def pmc(args) -> str:
    fetch, write = _per_kernel(args.fetch), _per_kernel(args.write)

    def pick(d, key):
        names = [k for k in d if key in k]
        if not names:
            sys.exit(f"no kernel matching {key!r}")
        vals = d[names[0]]
        return names[0], statistics.mean(vals), len(vals)

    kname, f_adam, n_adam = pick(fetch, args.kernel)
    _, w_adam, _ = pick(write, args.kernel)
    cname, f_copy, _ = pick(fetch, "copy_kernel")
    _, w_copy, _ = pick(write, "copy_kernel")
    copy_kib = args.copy_bytes / 1024.0
    sf, sw = copy_kib / f_copy, copy_kib / w_copy
    read_b = f_adam * sf * 1024.0
    write_b = w_adam * sw * 1024.0
    algo_r, algo_w = float(args.read_bytes) * args.params, 14.0 * args.params
    out = [f"# rocprofv3 HBM counters: {args.title}", "",
           f"FETCH_SIZE command: `{args.command_fetch}`", "",
           f"WRITE_SIZE command: `{args.command_write}`", "",
           "Counters are KiB per dispatch, averaged over dispatches.  Scale = bytes the",
           f"copy kernel moves each way ({args.copy_bytes:,} B) / what the counter reads for it.", "",
           "| Kernel | Dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) |",
           "|---|---|---|---|",
           f"| `{short(kname)}` | {n_adam} | {f_adam:,.1f} | {w_adam:,.1f} |",
           f"| `{short(cname)}` (copy, {args.copy_bytes:,} B each way) | - | {f_copy:,.1f} | {w_copy:,.1f} |",
           "",
           f"Scale factors: FETCH {sf:.4f}, WRITE {sw:.4f}", "",
           "| Per launch | Read (B) | Write (B) | Total (B) |",
           "|---|---|---|---|",
           f"| Measured (scaled) | {read_b:,.0f} | {write_b:,.0f} | {read_b + write_b:,.0f} |",
           f"| Algorithmic ({args.read_bytes} + 14 B x {args.params:,}) | {algo_r:,.0f} | {algo_w:,.0f} | "
           f"{algo_r + algo_w:,.0f} |",
           f"| Measured / algorithmic | {read_b / algo_r:.4f} | {write_b / algo_w:.4f} | "
           f"{(read_b + write_b) / (algo_r + algo_w):.4f} |",
           "",
           f"hbm_bytes_per_launch: {read_b + write_b:.6e}",
           f"kernel_source_sha256: {kernel_hash()}"]
    return "\n".join(out) + "\n"


def stream(args) -> str:
    rows = [r for r in csv.DictReader(open(args.trace))]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    copies = [r for r in rows if "block_copy" in r["Kernel_Name"]]
    upd = [r for r in rows if "fused_adam" in r["Kernel_Name"]]
    grads = [r for r in rows if "fill_normal_bf16" in r["Kernel_Name"]]
    by_q = {}
    for r in copies:
        by_q.setdefault(f"copy kernel, queue {r['Queue_Id']}", []).append(r)
    if args.memcpy:
        # DMA-engine copies of at least a piece (the bench's set-up copies are
        # chunked by the runtime into much smaller ones) that start at most
        # 10 ms after the last update has ended: the step's last D2H starts
        # right then, and the link probe the bench runs after the steps can
        # only start once that D2H (about 20 ms) is over
        cut = int(upd[-1]["End_Timestamp"]) + 10_000_000 if upd else None
        for r in csv.DictReader(open(args.memcpy)):
            if cut is not None and int(r["Start_Timestamp"]) > cut:
                continue
            if (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) > 1_000_000:
                by_q.setdefault(f"DMA {r['Direction'].replace('MEMORY_COPY_', '').lower()}", []).append(r)
        for v in by_q.values():
            v.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = [f"# rocprofv3 trace of the layer stream: {args.title}", "", f"Command: `{args.command}`", ""]
    # the last step: the last `copies` copies of each direction (one per
    # piece; a layer that does not move in pieces is one piece)
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
    out += ["| Stage | Engine | Count (last step) | Mean (ms) | Min (ms) | Max (ms) | GB/s at mean |",
            "|---|---|---|---|---|---|---|"]
    per_copy = args.step_bytes / args.copies
    for q, rs in sorted(by_q.items()):
        last = rs[-args.copies:]
        d = [dur(r) for r in last]
        out.append(f"| piece copy | {q} | {len(last)} | {statistics.mean(d):.1f} | {min(d):.1f} | "
                   f"{max(d):.1f} | {per_copy / (statistics.mean(d) * 1e-3) / 1e9:.1f} |")
    for name, rs, cnt in (("gradient producer", grads, args.layers), ("fused update", upd, args.copies)):
        last = rs[-cnt:]
        if last:
            d = [dur(r) for r in last]
            out.append(f"| {name} | {last[0]['Queue_Id']} | {len(last)} | {statistics.mean(d):.1f} | "
                       f"{min(d):.1f} | {max(d):.1f} | - |")
    # hidden compute: time the update/producer run with no copy in flight
    last_copies = [r for rs in by_q.values() for r in rs[-args.copies:]]
    t_lo = min(int(r["Start_Timestamp"]) for r in last_copies)
    t_hi = max(int(r["End_Timestamp"]) for r in last_copies)
    busy = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in last_copies)
    exposed = 0
    for r in upd[-args.copies:] + grads[-args.layers:]:
        s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        # length of [s, e) covered by the union of the copy intervals
        covered, cur = 0, s
        for a, b in busy:
            a, b = max(a, cur), min(b, e)
            if b > a:
                covered += b - a
                cur = b
        exposed += (e - s) - covered
    out += ["", f"Last step, first copy start to last copy end: {(t_hi - t_lo) / 1e6:.1f} ms; "
                f"update + producer time with no copy running beside it: {exposed / 1e6:.2f} ms"]
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("--csv", required=True)
    a.add_argument("--command", required=True)
    a.add_argument("--title", default="")
    a.add_argument("--top", type=int, default=6)
    a.add_argument("--trace", default=None, help="X_kernel_trace.csv: split --kernel's dispatches by grid")
    a.add_argument("--kernel", default="fused_adam")
    b = sub.add_parser("pmc")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--params", type=int, required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--kernel", default="fused_adam")
    b.add_argument("--read-bytes", type=int, default=14,
                   help="algorithmic bytes read per parameter (16 with FP32 gradients)")
    b.add_argument("--command-fetch", required=True)
    b.add_argument("--command-write", required=True)
    b.add_argument("--title", default="")
    c = sub.add_parser("stream")
    c.add_argument("--trace", required=True)
    c.add_argument("--layers", type=int, required=True)
    c.add_argument("--copies", type=int, required=True, help="copies per direction per step")
    c.add_argument("--memcpy", default=None, help="X_memory_copy_trace.csv (DMA-engine copies)")
    c.add_argument("--step-bytes", type=int, required=True, help="bytes per direction per step")
    c.add_argument("--command", required=True)
    c.add_argument("--title", default="")
    args = ap.parse_args(argv)
    text = {"stats": stats, "pmc": pmc, "stream": stream}[args.cmd](args)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
