"""Summaries of rocprofv3 output for the decode kernels (text for profiles/).

  python -m sparse_moe_decode_gemv_amd.profiling trace <run_results.db | kernel_trace.csv>
      per-kernel launch count and duration (mean / median / min), each
      gate/up launch classed as in-layer (after the router) or stand-alone;
      then per decode layer (router .. combine, launched back to back) the
      kernel count, the span from the first start to the last end, the idle
      time between the layer's kernels and the gap to the next layer.

  python -m sparse_moe_decode_gemv_amd.profiling counters <fetch.csv> <write.csv>
      HBM bytes per launch from two counter-collection runs (FETCH_SIZE, then
      WRITE_SIZE, in KiB per dispatch).  Both are scaled by what the same
      counter reads for the plain 1 GiB device copy that bench.py runs once
      (1 GiB read, 1 GiB written), and reported per kernel; the stand-alone
      gate/up line is what bench.py reports as the roofline traffic.

Reads only rocprofv3 output; runs nothing on the GPU.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import os
import re
import sqlite3
import statistics as st
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(HERE, "csrc", "moe_t1.hip")
BATCHED_SRC = os.path.join(HERE, "csrc", "moe_batched.hip")
CALIB_BYTES = 1 << 30

_NAMES = re.compile(r"(k1_router|k1_topk|k2_gateup|k3_slab|k3_down|kb_\w+|"
                    r"zero_fill_kernel|fill_\w+_kernel|copyBuffer\w*|\w+_kernel)")


def short(name: str) -> str:
    m = _NAMES.search(name)
    return m.group(1) if m else name[:40]


# Headers the kernel sources compile with (project headers only): a digest
# covers them too, so that a change there also retires a summary.
KERNEL_HEADERS = [os.path.join(HERE, "csrc", h) for h in ("moe_device.h", "moe_internal.h", "moe_topk.h")] + \
    [os.path.join(os.path.dirname(HERE), "include", "moe.h")]


def code_text(text: str) -> str:
    """The code of a C++ source: comments removed, runs of blank space
    collapsed (so that edits to prose do not change the digest)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(path: str = KERNEL_SRC) -> str:
    """First 16 hex digits of the SHA-256 of the code of ``path`` and of the
    project headers it compiles with, in that order."""
    h = hashlib.sha256()
    for f in [path] + KERNEL_HEADERS:
        with open(f, encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _classify(seq):
    """seq: [(name, grid, wg, value...)] in launch order -> key per launch.
    Gate/up launches are split by predecessor: after the router they are the
    layer's own, otherwise the stand-alone (expert_gateup) launches."""
    keys, prev = [], "-"
    for name in seq:
        k = name
        if name == "k2_gateup":
            k = "k2_gateup (in layer)" if prev == "k1_router" else "k2_gateup (stand-alone)"
        keys.append(k)
        prev = name
    return keys


def trace(path: str) -> str:
    if path.endswith(".db"):
        c = sqlite3.connect(path)
        rows = [(r[0], r[1], r[2]) for r in
                c.execute("select name, start, end from kernels order by start")]
    else:
        with open(path) as f:
            rows = sorted(((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
                           for r in csv.DictReader(f)), key=lambda r: r[1])
    names = [short(r[0]) for r in rows]
    keys = _classify(names)
    d = collections.defaultdict(list)
    for k, r in zip(keys, rows):
        d[k].append((r[2] - r[1]) / 1e3)
    out = [f"{'kernel':28s} {'launches':>8s} {'mean us':>9s} {'median':>9s} {'min':>9s}"]
    for k, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{k:28s} {len(v):8d} {st.mean(v):9.2f} {st.median(v):9.2f} {min(v):9.2f}")
    out += ["", layer_spans(names, rows)]
    return "\n".join(out)


_FIRST = ("k1_router", "kb_rmsnorm", "kb_router")
_LAST = ("k3_slab", "k3_down", "kb_combine")


def layer_spans(names, rows) -> str:
    """Decode layers as launched: a layer opens with the router (or the
    batched RMSNorm before it) and closes with the down/combine kernel, with
    only layer kernels in between.  Times in microseconds."""
    layers, cur = [], None
    for n, r in zip(names, rows):
        opens = n in _FIRST and not (n == "kb_router" and cur and cur[-1][0] == "kb_rmsnorm")
        if opens:
            cur = [(n, r[1], r[2])]
        elif cur is not None:
            if n.startswith(("k1_", "k2_", "k3_", "kb_")):
                cur.append((n, r[1], r[2]))
            else:
                cur = None
                continue
        if cur is not None and n in _LAST:
            layers.append(cur)
            cur = None
    if not layers:
        return "no complete decode layer in the trace"
    spans = [(l[-1][2] - l[0][1]) / 1e3 for l in layers]
    idle = [sum(max(0, b[1] - a[2]) for a, b in zip(l, l[1:])) / 1e3 for l in layers]
    nk = collections.Counter(len(l) for l in layers)
    between = [(b[0][1] - a[-1][2]) / 1e3 for a, b in zip(layers, layers[1:])
               if 0 <= b[0][1] - a[-1][2] < 50_000]
    seqs = collections.Counter(" > ".join(k[0] for k in l) for l in layers)
    out = [f"decode layers in the trace: {len(layers)}; kernels per layer: "
           + ", ".join(f"{k} ({v} layers)" for k, v in sorted(nk.items())),
           f"layer span (first start .. last end) us: mean {st.mean(spans):.2f} "
           f"median {st.median(spans):.2f} min {min(spans):.2f}",
           f"idle between a layer's kernels us: mean {st.mean(idle):.2f} "
           f"median {st.median(idle):.2f} max {max(idle):.2f}"]
    if between:
        out.append(f"gap to the next layer us: mean {st.mean(between):.2f} "
                   f"median {st.median(between):.2f}")
    for s_, c in seqs.most_common(3):
        out.append(f"  {c:5d} x {s_}")
    return "\n".join(out)


def _counter_means(path: str, counter: str):
    with open(path) as f:
        rows = list(csv.DictReader(f))
    disp = collections.OrderedDict()
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        disp.setdefault(d, [short(r["Kernel_Name"]), 0.0, int(r["Grid_Size"])])
        disp[d][1] += float(r["Counter_Value"])
    items = list(disp.values())
    keys = _classify([i[0] for i in items])
    agg = collections.defaultdict(list)
    for k, d, (name, v, grid) in zip(keys, disp.keys(), items):
        if name.startswith("copyBuffer"):
            # copies stay separate: another copy can share the calibration
            # copy's grid (the grid size is capped for large copies)
            k = f"{name} grid={grid} dispatch={d}"
        agg[k].append(v)
    return {k: st.mean(v) for k, v in agg.items()}, {k: len(v) for k, v in agg.items()}


def counters(fetch_csv: str, write_csv: str) -> str:
    fetch, n_f = _counter_means(fetch_csv, "FETCH_SIZE")
    write, _ = _counter_means(write_csv, "WRITE_SIZE")
    copies = [k for k in fetch if k.startswith("copyBuffer")]
    calib = max(copies, key=lambda k: fetch[k])  # the 1 GiB copy
    f_fetch = CALIB_BYTES / (fetch[calib] * 1024.0)
    f_write = CALIB_BYTES / (write[calib] * 1024.0)
    out = [f"calibration kernel: {calib} (1 GiB read + 1 GiB written)",
           f"fetch_scale: {f_fetch:.4f}",
           f"write_scale: {f_write:.4f}",
           f"{'kernel':28s} {'launches':>8s} {'FETCH KiB':>12s} {'WRITE KiB':>10s} {'HBM bytes/launch':>17s}"]
    traffic = None
    for k in sorted(fetch):
        if k.startswith("copyBuffer") or k not in write:
            continue
        b = int(round(fetch[k] * 1024 * f_fetch + write[k] * 1024 * f_write))
        out.append(f"{k:28s} {n_f[k]:8d} {fetch[k]:12.1f} {write[k]:10.1f} {b:17d}")
        if k in ("k2_gateup (in layer)", "kb_gateup"):  # the kernel bench.py's roofline names
            traffic = b
    out.append(f"kernel_source_sha256_16: {source_digest()}")
    out.append(f"batched_source_sha256_16: {source_digest(BATCHED_SRC)}")
    if traffic is not None:
        out.append(f"traffic_bytes_per_launch: {traffic}")
    return "\n".join(out)


def read_counter_summary(path: str):
    """(header values, HBM bytes per launch by kernel) of a summary written by
    ``counters``: the ``name: value`` lines and the table rows."""
    vals, table = {}, {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            cols = re.split(r"\s{2,}", line.strip())
            if len(cols) == 5 and cols[-1].isdigit():
                table[cols[0]] = int(cols[-1])
            elif ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    return vals, table


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace(argv[1]))
    elif len(argv) >= 3 and argv[0] == "counters":
        print(counters(argv[1], argv[2]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
