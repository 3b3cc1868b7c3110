"""Summarise a rocprofv3 kernel trace of the encoder (``--kernel-trace
--output-format csv``) per kernel and per site.

    python -m whisper_audio_encoder_amd.trace_summary <kernel_trace.csv> --workload c4 [--parts 2]

Per kernel: launches, rocprofv3's average duration and share of kernel time.
Per site (conv1, q|k|v, attention, ...), per application over the whole
batch: the site's share of the device's busy time, and the rate that share
gives on the site's algorithmic work.  The share splits every stretch of
time evenly among the kernels running in it, so the shares of all sites add
up to the time the device ran any kernel; a forward whose windows are split
over ``--parts`` streams runs kernels of different sites side by side, and
this is the time each of them accounts for.  With everything on one stream
the share is simply the sum of the site's kernel durations.
"""
from __future__ import annotations

import argparse
import csv
import re
import sys
from collections import defaultdict

from .configs import CONFIGS

# gemm_kernel<BM, BN, WM, WN, NW, EPI, TAG, PP>: EPI and TAG name the projection (PP, the main-loop
# schedule, is absent from traces of earlier builds)
GEMM_SITES = {(0, 0): "conv1", (0, 1): "fc1", (1, 0): "conv2", (2, 0): "oproj", (2, 1): "fc2", (3, 0): "qkv",
              (4, 0): "xkv"}
BLOCK_SITES = ("ln", "qkv", "attn", "oproj", "fc1", "fc2")


def site_of(name: str) -> str | None:
    m = re.search(r"gemm_kernel<\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+)(?:,\s*\d+)?>", name)
    if m:
        return GEMM_SITES.get((int(m.group(6)), int(m.group(7))))
    if "attn_kernel" in name:
        return "attn"
    if "ln_kernel" in name:
        return "lnf" if "true>" in name else "ln"
    if "ingest_kernel" in name:
        return "ingest"
    return None


def site_work(cfg, site):
    """(unit, amount) of one application of a site over the whole batch."""
    B, T, F, d, nm, H, Fd = cfg.batch, cfg.n_ctx, cfg.n_frames, cfg.d_model, cfg.n_mels, cfg.n_head, cfg.d_ff
    M = B * T
    return {
        "conv1": ("TFLOP/s", 2.0 * B * F * d * 3 * nm), "conv2": ("TFLOP/s", 2.0 * M * d * 3 * d),
        "qkv": ("TFLOP/s", 2.0 * M * 3 * d * d), "attn": ("TFLOP/s", 4.0 * B * H * T * T * 64),
        "oproj": ("TFLOP/s", 2.0 * M * d * d), "fc1": ("TFLOP/s", 2.0 * M * Fd * d), "fc2": ("TFLOP/s", 2.0 * M * d * Fd),
        "ln": ("GB/s", 6.0 * M * d), "lnf": ("GB/s", 8.0 * M * d),
        "ingest": ("GB/s", B * F * nm * 4.0 + B * (F + 2) * nm * 2.0),
    }[site]


def fair_share_ns(intervals):
    """intervals: (start, end, key).  Sweep the timeline and give each
    stretch to the kernels running in it in equal parts; returns {key: ns}
    and the busy time (the length of the union of all intervals)."""
    ev = []
    for i, (a, b, k) in enumerate(intervals):
        ev.append((a, 1, i))
        ev.append((b, -1, i))
    ev.sort(key=lambda e: (e[0], e[1]))
    share = defaultdict(float)
    active = set()
    busy = 0.0
    last = None
    for t, kind, i in ev:
        if last is not None and active and t > last:
            part = (t - last) / len(active)
            busy += t - last
            for j in active:
                share[intervals[j][2]] += part
        if kind == 1:
            active.add(i)
        else:
            active.discard(i)
        last = t
    return share, busy


def _rows(path: str, region: str):
    """The trace's kernel dispatches in start order; with region "first" or
    "second", those before or after the start of the second scratch fill
    (wenc_create clears a new handle's scratch, so in a bench.py trace the
    second fill starts the second handle, the one-stream roofline pass)."""
    with open(path) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
    if region == "all":
        return rows
    fills = [int(r["Start_Timestamp"]) for r in rows if "fillBuffer" in r["Kernel_Name"]]
    if len(fills) < 2:
        raise SystemExit("the trace holds fewer than two scratch fills: no second handle")
    cut = fills[1]
    return [r for r in rows if (int(r["Start_Timestamp"]) < cut) == (region == "first")]


def summarise(path: str, workload: str, parts: int, region: str = "all") -> str:
    cfg = CONFIGS[workload]
    per_kernel = defaultdict(list)
    per_site = defaultdict(list)
    intervals = []
    for row in _rows(path, region):
        name = row["Kernel_Name"]
        t0, t1 = int(row["Start_Timestamp"]), int(row["End_Timestamp"])
        per_kernel[name].append(t1 - t0)
        s = site_of(name)
        if s:
            per_site[s].append((t0, t1))
        intervals.append((t0, t1, s or "-"))
    share, busy = fair_share_ns(intervals)
    total = sum(sum(v) for v in per_kernel.values()) or 1
    forwards = len(per_site.get("lnf", [])) / parts if cfg.final_ln else len(per_site.get("ingest", [])) / parts
    out = [f"Per kernel ({path.split('/')[-1]}, {region} dispatches; {forwards:g} forwards of {workload} over "
           f"{parts} stream(s)):", "",
           "| kernel | site | calls | avg us | % of kernel time |", "|---|---|---|---|---|"]
    for name, d in sorted(per_kernel.items(), key=lambda kv: -sum(kv[1])):
        short = re.sub(r"\(.*", "", name.replace("void ", "").replace("wk::(anonymous namespace)::", ""))
        out.append(f"| `{short[:60]}` | {site_of(name) or '-'} | {len(d)} | {sum(d) / len(d) / 1e3:.1f} | "
                   f"{100.0 * sum(d) / total:.2f} |")
    out += ["", f"Per site, over the whole batch (share of the device's busy time, {busy / 1e6:.1f} ms in all, "
            f"{busy / 1e6 / max(forwards, 1):.3f} ms per forward):", "",
            "| site | applications | us per application | % of busy time | rate |", "|---|---|---|---|---|"]
    for s in ("conv1", "conv2", "ln", "qkv", "attn", "oproj", "fc1", "fc2", "lnf", "ingest"):
        if s not in per_site:
            continue
        apps = forwards * (cfg.n_layer * (2 if s == "ln" else 1) if s in BLOCK_SITES else 1)
        us = share[s] / apps / 1e3
        unit, work = site_work(cfg, s)
        rate = work / (us * 1e-6) / (1e12 if unit == "TFLOP/s" else 1e9)
        out.append(f"| {s} | {apps:g} | {us:.1f} | {100.0 * share[s] / busy:.2f} | {rate:.0f} {unit} |")
    return "\n".join(out)


def _kernel_label(name: str) -> str:
    """Site of a kernel, with the tile size where one site has two kernels."""
    site = site_of(name)
    m = re.search(r"gemm_kernel<\s*(\d+),\s*(\d+),", name)
    return f"{site} ({m.group(1)}x{m.group(2)})" if m and site else (site or "-")


def read_counters(path: str):
    """{dispatch id: (kernel name, duration ns, {counter: value})} of a
    rocprofv3 counter_collection.csv."""
    disp = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            d = disp.setdefault(row["Dispatch_Id"], [row["Kernel_Name"],
                                                      int(row["End_Timestamp"]) - int(row["Start_Timestamp"]), {}])
            d[2][row["Counter_Name"]] = d[2].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return disp


def utilisation(path: str, simds: int = 1024, xcds: int = 8) -> str:
    """MFMA busy share, VALU co-execution and effective clock per kernel from
    GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES, SQ_VALU_MFMA_COEXEC_CYCLES."""
    groups = defaultdict(list)
    for name, dur, c in read_counters(path).values():
        if site_of(name):
            groups[_kernel_label(name)].append((dur, c))
    out = ["| kernel (site) | dispatches | avg us | eff. clock GHz | MFMA busy | co-exec | peak at eff. clock TFLOP/s |",
           "|---|---|---|---|---|---|---|"]
    for label, rows in sorted(groups.items(), key=lambda kv: -sum(r[0] for r in kv[1])):
        dur = sum(r[0] for r in rows) / len(rows)
        cyc = sum(r[1].get("GRBM_GUI_ACTIVE", 0.0) for r in rows) / len(rows) / xcds
        busy = sum(r[1].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for r in rows) / len(rows)
        co = sum(r[1].get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) for r in rows) / len(rows)
        clk = cyc / dur if dur else 0.0
        out.append(f"| {label} | {len(rows)} | {dur / 1e3:.1f} | {clk:.2f} | {100.0 * busy / (simds * cyc):.1f}% | "
                   f"{100.0 * co / busy if busy else 0.0:.0f}% | {simds * 1024 * clk / 1e3:.0f} |")
    return "\n".join(out)


def stalls(path: str) -> str:
    """Per kernel of the encoder: instructions per wave (VALU, of which MFMA;
    LDS) from SQ_INSTS_*, and the share of the waves' resident cycles spent
    waiting for an instruction's dependencies (SQ_WAIT_INST_ANY /
    SQ_WAVE_CYCLES) or issuing VALU work (SQ_ACTIVE_INST_VALU /
    SQ_WAVE_CYCLES).  Counters as rocprofv3 sums them over the device."""
    groups = defaultdict(list)
    for name, dur, c in read_counters(path).values():
        if site_of(name):
            groups[_kernel_label(name)].append((dur, c))
    out = ["| kernel (site) | dispatches | avg us | waves | VALU insts per wave | MFMA per wave | LDS insts per wave | "
           "waiting on dependencies | VALU active |",
           "|---|---|---|---|---|---|---|---|---|"]
    for label, rows in sorted(groups.items(), key=lambda kv: -sum(r[0] for r in kv[1])):
        def tot(k):
            return sum(r[1].get(k, 0.0) for r in rows)
        waves = tot("SQ_WAVES")
        wc = tot("SQ_WAVE_CYCLES")
        per = (lambda k: tot(k) / waves) if waves else (lambda k: 0.0)
        out.append(f"| {label} | {len(rows)} | {sum(r[0] for r in rows) / len(rows) / 1e3:.1f} | {waves / len(rows):.0f} | "
                   f"{per('SQ_INSTS_VALU'):.0f} | {per('SQ_INSTS_MFMA'):.0f} | {per('SQ_INSTS_LDS'):.0f} | "
                   f"{100.0 * tot('SQ_WAIT_INST_ANY') / wc if wc else 0.0:.0f}% | "
                   f"{100.0 * tot('SQ_ACTIVE_INST_VALU') / wc if wc else 0.0:.0f}% |")
    return "\n".join(out)


EPI_NAMES = {0: "GELU fp16", 1: "GELU + positions fp32", 2: "residual fp32", 3: "q|k|v", 4: "cross K/V"}


def utilisation_by_grid(path: str, simds: int = 1024, xcds: int = 8) -> str:
    """GEMM dispatches grouped by epilogue, tile size and workgroup count
    (bench.py --gemm-tile-costs launches the same kernel over 1024 tiles and
    over 32 over a range of K).  GRBM_GUI_ACTIVE counts some cycles around
    each dispatch as well, so the clock is the slope of a least-squares line
    of cycles against duration over the longest third of a group's
    dispatches (its largest K), and the MFMA busy share is taken over the
    cycles of those dispatches at that clock."""
    with open(path) as fh:
        rows = list(csv.DictReader(fh))
    disp = {}
    for row in rows:
        d = disp.setdefault(row["Dispatch_Id"], [row["Kernel_Name"], int(row["Grid_Size"]) // int(row["Workgroup_Size"]),
                                                 int(row["End_Timestamp"]) - int(row["Start_Timestamp"]), {}])
        d[3][row["Counter_Name"]] = d[3].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    groups = defaultdict(list)
    for name, wgs, dur, c in disp.values():
        m = re.search(r"gemm_kernel<\s*(\d+),\s*(\d+),\s*\d+,\s*\d+,\s*\d+,\s*(\d+),", name)
        if m:
            groups[(EPI_NAMES.get(int(m.group(3)), m.group(3)), f"{m.group(1)}x{m.group(2)}", wgs)].append(
                (dur, c.get("GRBM_GUI_ACTIVE", 0.0) / xcds, c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)))
    out = ["| epilogue | tile | workgroups | dispatches fitted | their avg us | clock GHz (slope) | "
           "cycles outside the dispatch | MFMA busy at that clock |",
           "|---|---|---|---|---|---|---|---|"]
    for (epi, tile, wgs), rs in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1], -kv[0][2])):
        rs.sort()
        top = rs[len(rs) - max(2, len(rs) // 3):]
        n = len(top)
        mx = sum(r[0] for r in top) / n
        my = sum(r[1] for r in top) / n
        sxx = sum((r[0] - mx) ** 2 for r in top)
        f = sum((r[0] - mx) * (r[1] - my) for r in top) / sxx if sxx else 0.0  # cycles per ns = GHz
        extra = my - f * mx
        busy = sum(r[2] for r in top) / n / (simds * f * mx) if f else 0.0
        out.append(f"| {epi} | {tile} | {wgs} | {n} | {mx / 1e3:.1f} | {f:.2f} | {extra / 1e3:.1f} k | {100.0 * busy:.1f}% |")
    return "\n".join(out)


def traffic(fetch: str, write: str, copy_fetch: str, copy_write: str, copy_bytes: int, workload: str):
    """HBM bytes per application of each site from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by what the counter reads for a plain
    device copy of copy_bytes; returns (markdown, {site: (fetch, write)})."""
    def per_dispatch(path, counter):
        return [(n, c.get(counter, 0.0) * 1024.0) for n, _, c in read_counters(path).values()]

    def factor(path, counter, true_bytes):
        vals = [v for n, v in per_dispatch(path, counter) if "copyBuffer" in n or "elementwise" in n or "copy" in n]
        return true_bytes / max(vals) if vals and max(vals) > 0 else 1.0

    f_fetch = factor(copy_fetch, "FETCH_SIZE", copy_bytes)
    f_write = factor(copy_write, "WRITE_SIZE", copy_bytes)
    cfg = CONFIGS[workload]
    sites = defaultdict(lambda: [0.0, 0.0, 0])
    for idx, (path, counter, f) in enumerate(((fetch, "FETCH_SIZE", f_fetch), (write, "WRITE_SIZE", f_write))):
        for n, v in per_dispatch(path, counter):
            s = site_of(n)
            if s:
                sites[s][idx] += v * f
                if idx == 0:
                    sites[s][2] += 1
    forwards = sites["lnf"][2] if "lnf" in sites else 1
    out = [f"Calibration: a {copy_bytes} B device copy reads FETCH_SIZE x{f_fetch:.3f} and WRITE_SIZE "
           f"x{f_write:.3f} of its true bytes; below, counters times those factors, per application of the "
           f"site over the whole batch ({forwards} forwards).", "",
           "| site | fetch MB | write MB |", "|---|---|---|"]
    per_app = {}
    for s in ("conv1", "conv2", "ln", "qkv", "attn", "oproj", "fc1", "fc2", "lnf"):
        if s not in sites:
            continue
        apps = forwards * (cfg.n_layer * (2 if s == "ln" else 1) if s in BLOCK_SITES else 1)
        fb, wb = sites[s][0] / apps, sites[s][1] / apps
        per_app[s] = (fb, wb)
        out.append(f"| {s} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
    return "\n".join(out), per_app


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("trace", help="kernel_trace.csv, or counter_collection.csv with --util / --traffic")
    ap.add_argument("--workload", default="c4", choices=sorted(CONFIGS))
    ap.add_argument("--parts", type=int, default=2, help="streams a forward's windows are split over")
    ap.add_argument("--region", default="all", choices=["all", "first", "second"],
                    help="kernel trace of bench.py: its first handle (the timed forward) or its second (one stream)")
    ap.add_argument("--util", action="store_true", help="the file holds GRBM_GUI_ACTIVE and MFMA-busy counters")
    ap.add_argument("--stalls", action="store_true",
                    help="the file holds SQ_WAVES, SQ_WAVE_CYCLES, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_VALU and SQ_INSTS_*")
    ap.add_argument("--util-by-grid", action="store_true",
                    help="as --util, GEMM dispatches grouped by epilogue, tile size and workgroup count")
    ap.add_argument("--traffic", nargs=3, metavar=("WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="the file holds FETCH_SIZE; with the WRITE_SIZE run and the copy calibration runs")
    ap.add_argument("--copy-bytes", type=int, default=268435456)
    ap.add_argument("--json-site", default=None, help="with --traffic: print the JSON record bench.py reads for this site")
    a = ap.parse_args(argv)
    if a.stalls:
        print(stalls(a.trace))
    elif a.util_by_grid:
        print(utilisation_by_grid(a.trace))
    elif a.util:
        print(utilisation(a.trace))
    elif a.traffic:
        md, per_app = traffic(a.trace, *a.traffic, a.copy_bytes, a.workload)
        print(md)
        if a.json_site:
            import json
            import os
            sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
            import bench
            fb, wb = per_app[a.json_site]
            print(json.dumps({"site": a.json_site, "workload": a.workload,
                              "kernel_source_sha256": bench.kernel_source_hash(a.json_site),
                              "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                              "hbm_bytes_per_launch": fb + wb}, indent=1))
    else:
        print(summarise(a.trace, a.workload, a.parts, a.region))


if __name__ == "__main__":
    sys.exit(main())
