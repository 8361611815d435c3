"""Text summaries of rocprofv3 CSV output (``-f csv``).

Kernel statistics of a ``--kernel-trace --stats`` run::

    python -m shared_matrix_expert_amd.profsum stats OUT_DIR --cmd "<rocprofv3 command>"

HBM traffic of one kernel from two ``--pmc`` runs (FETCH_SIZE, then
WRITE_SIZE, both in KiB per dispatch), each scaled by what the same counter
reads for the library's plain copy kernel of known size (``copy_bytes``)::

    python -m shared_matrix_expert_amd.profsum traffic FETCH_DIR WRITE_DIR --kernel dec_act \\
        --calib-bytes 268435456 --cmd-fetch "..." --cmd-write "..."

Per-dispatch means of any counters of one ``--pmc`` run, for chosen kernels::

    python -m shared_matrix_expert_amd.profsum counters OUT_DIR --kernels "pf_gemm<0>,pf_gemm<1>" \
        --cmd "..."

The traffic summary records the digest of the library sources it was taken
with, so that a reader can tell whether it still describes the current kernels.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import sys
from collections import defaultdict

from .build import sources_digest


def _find(out_dir: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(out_dir, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {out_dir}")
    return hits[-1]


def _col(row: dict, *names):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(f"none of {names} in {list(row)}")


def _base(name: str) -> str:
    """Kernel name without return type, namespace, template arguments and parameters."""
    return _short(name).split("<")[0]


def _short(name: str) -> str:
    """Kernel name with its template arguments, without return type, namespaces
    and parameters: 'void em::dec_up<1, true>(em::DecodeArgs)' -> 'dec_up<1, true>'."""
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    base = name[:cut].strip()
    if base.startswith("void "):
        base = base[5:]
    head, sep, tmpl = base.partition("<")
    return head.split("::")[-1] + (sep + tmpl.replace("em::", "") if sep else "")


def stats(out_dir: str, cmd: str, title: str, match: str = "") -> str:
    """Markdown table of the kernels whose full name contains `match` (all if
    empty); the share column is relative to the listed kernels."""
    path = _find(out_dir, "kernel_stats.csv")
    rows = [r for r in csv.DictReader(open(path))
            if match in _col(r, "Name", "KernelName", "Kernel_Name")]
    total = sum(float(_col(r, "TotalDurationNs")) for r in rows) or 1.0
    sel = f" (kernels whose name contains `{match}`)" if match else ""
    lines = [f"# {title}", "", f"Command: `{cmd}`", "", f"Listed{sel}:", "",
             "| kernel | calls | total ms | avg us | min us | max us | share % |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = _short(_col(r, "Name", "KernelName", "Kernel_Name"))
        calls = int(float(_col(r, "Calls")))
        tot_ns = float(_col(r, "TotalDurationNs"))
        avg = float(_col(r, "AverageNs")) / 1e3
        mn = float(_col(r, "MinNs")) / 1e3
        mx = float(_col(r, "MaxNs")) / 1e3
        lines.append(f"| {name} | {calls} | {tot_ns / 1e6:.3f} | {avg:.2f} | {mn:.2f} | {mx:.2f} | "
                     f"{100 * tot_ns / total:.1f} |")
    return "\n".join(lines) + "\n"


def _per_dispatch(out_dir: str, counter: str) -> dict:
    """{kernel name: [value per dispatch]} for one counter, keyed both by the
    name without template arguments (all instances) and with them (one)."""
    path = _find(out_dir, "counter_collection.csv")
    acc = defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if _col(r, "Counter_Name").split("[")[0] != counter:
            continue
        did = _col(r, "Dispatch_Id", "Dispatch_ID")
        acc[did] += float(_col(r, "Counter_Value"))
        names[did] = (_base(_col(r, "Kernel_Name")), _short(_col(r, "Kernel_Name")))
    out = defaultdict(list)
    for did, v in acc.items():
        base, short = names[did]
        out[base].append(v)
        if short != base:
            out[short].append(v)
    return out


def traffic(fetch_dir: str, write_dir: str, kernel: str, calib_bytes: int, cmd_fetch: str,
            cmd_write: str, workload: str) -> str:
    f = _per_dispatch(fetch_dir, "FETCH_SIZE")
    w = _per_dispatch(write_dir, "WRITE_SIZE")
    for tab, what in ((f, "FETCH_SIZE"), (w, "WRITE_SIZE")):
        for k in (kernel, "copy_bytes"):
            if not tab.get(k):
                raise SystemExit(f"no {what} dispatches of {k}")
    mean = lambda v: sum(v) / len(v)  # noqa: E731
    f_k, w_k = mean(f[kernel]), mean(w[kernel])
    f_c, w_c = mean(f["copy_bytes"]), mean(w["copy_bytes"])
    ff = calib_bytes / (f_c * 1024.0)
    fw = calib_bytes / (w_c * 1024.0)
    tb = f_k * 1024.0 * ff + w_k * 1024.0 * fw
    kv = [("kernel", kernel), ("workload", workload), ("fetch_cmd", cmd_fetch), ("write_cmd", cmd_write),
          ("dispatches_fetch", len(f[kernel])), ("dispatches_write", len(w[kernel])),
          ("fetch_kib_per_dispatch", f"{f_k:.1f}"), ("write_kib_per_dispatch", f"{w_k:.1f}"),
          ("calib_bytes", calib_bytes), ("calib_fetch_kib", f"{f_c:.1f}"), ("calib_write_kib", f"{w_c:.1f}"),
          ("fetch_factor", f"{ff:.4f}"), ("write_factor", f"{fw:.4f}"),
          ("traffic_bytes_per_dispatch", f"{tb:.0f}"), ("sources_sha256", sources_digest(kernel))]
    head = (f"# HBM traffic of {kernel} ({workload})\n"
            "# FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by bytes / counter of the plain\n"
            "# copy kernel copy_bytes over calib_bytes bytes in the same run.\n")
    return head + "".join(f"{k}: {v}\n" for k, v in kv)


def counters(out_dir: str, kernels: list, cmd: str, title: str) -> str:
    """Markdown table: per-dispatch mean of every counter in the run for each
    kernel (matched by name with or without template arguments), then the
    ratios that follow from them when the counters are present."""
    path = _find(out_dir, "counter_collection.csv")
    acc = defaultdict(float)
    names, ctrs = {}, []
    for r in csv.DictReader(open(path)):
        c = _col(r, "Counter_Name").split("[")[0]
        if c not in ctrs:
            ctrs.append(c)
        did = _col(r, "Dispatch_Id", "Dispatch_ID")
        acc[(did, c)] += float(_col(r, "Counter_Value"))
        names[did] = (_base(_col(r, "Kernel_Name")), _short(_col(r, "Kernel_Name")))
    lines = [f"# {title}", "", f"Command: `{cmd}`", "",
             "Per-dispatch means (each counter summed over its instances within a dispatch):", "",
             "| kernel | dispatches | " + " | ".join(ctrs) + " |",
             "|---|---:|" + "---:|" * len(ctrs)]
    derived = []
    for k in kernels:
        dids = [d for d, (b, s_) in names.items() if k in (b, s_)]
        if not dids:
            lines.append(f"| {k} | 0 |" + " |" * len(ctrs))
            continue
        m = {c: sum(acc[(d, c)] for d in dids) / len(dids) for c in ctrs}
        lines.append(f"| {k} | {len(dids)} | " + " | ".join(f"{m[c]:.4g}" for c in ctrs) + " |")
        row = []
        mops = {c[len("SQ_INSTS_VALU_MFMA_MOPS_"):]: v for c, v in m.items() if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_")}
        if any(mops.values()):
            parts = ", ".join(f"{t.lower()} {v * 512:.4g}" for t, v in mops.items() if v)
            row.append(("matrix-core flops (MOPS x 512)", f"{sum(mops.values()) * 512:.4g} ({parts})"))
        if m.get("SQ_INSTS_MFMA") and "SQ_INSTS_VALU" in m:
            row.append(("SQ_INSTS_VALU / SQ_INSTS_MFMA",
                        f"{m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.3f}"))
        if m.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in m:
            row.append(("LDS bank-conflict cycles per LDS instruction",
                        f"{m['SQ_LDS_BANK_CONFLICT'] / m['SQ_INSTS_LDS']:.3f}"))
        if m.get("SQ_BUSY_CU_CYCLES") and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            row.append(("MFMA busy cycles / CU busy cycles",
                        f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / m['SQ_BUSY_CU_CYCLES']:.3f}"))
        if row:
            derived.append((k, row))
    if derived:
        lines += ["", "Derived:", ""]
        for k, row in derived:
            lines += [f"- {k}: " + "; ".join(f"{a} = {b}" for a, b in row)]
    return "\n".join(lines) + "\n"


def read_traffic(path: str) -> dict:
    out = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        out[k.strip()] = v.strip()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("out_dir")
    a.add_argument("--cmd", required=True)
    a.add_argument("--title", default="rocprofv3 kernel statistics")
    a.add_argument("--match", default="", help="list only kernels whose name contains this")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("--kernel", required=True)
    b.add_argument("--calib-bytes", type=int, required=True)
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    b.add_argument("--workload", default="")
    c = sub.add_parser("counters")
    c.add_argument("out_dir")
    c.add_argument("--kernels", required=True, help="comma-separated kernel names")
    c.add_argument("--cmd", required=True)
    c.add_argument("--title", default="rocprofv3 counters")
    args = ap.parse_args(argv)
    if args.what == "stats":
        sys.stdout.write(stats(args.out_dir, args.cmd, args.title, args.match))
    elif args.what == "counters":
        sys.stdout.write(counters(args.out_dir, args.kernels.split(","), args.cmd, args.title))
    else:
        sys.stdout.write(traffic(args.fetch_dir, args.write_dir, args.kernel, args.calib_bytes,
                                 args.cmd_fetch, args.cmd_write, args.workload))


if __name__ == "__main__":
    main()
