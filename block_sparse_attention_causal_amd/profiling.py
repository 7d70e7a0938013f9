"""Summaries of rocprofv3 output for the MoBA kernels (text tables for profiles/).

    python -m block_sparse_attention_causal_amd.profiling stats DIR
        per-kernel calls / average / total duration from a --kernel-trace --stats run
    python -m block_sparse_attention_causal_amd.profiling traffic FETCH_DIR WRITE_DIR \
            --copy-mib N --kernel attn_selected
        HBM bytes per launch of one kernel from two --pmc runs (FETCH_SIZE, then
        WRITE_SIZE), scaled by what the same counters read for a plain copy kernel
        (torch.neg over N MiB of fp32: N MiB read, N MiB written).
    python -m block_sparse_attention_causal_amd.profiling dram DIR --copy-mib N
        DRAM bytes read and written per launch of every kernel from one --pmc run of
        TCC_EA0_RDREQ_DRAM_32B_sum and TCC_EA0_WRREQ_WRITE_DRAM_32B_sum (requests in
        32-byte units, 64- and 128-byte requests counted 2 and 4 times), checked
        against the same copy.
    python -m block_sparse_attention_causal_amd.profiling counters DIR
        per-kernel mean of every counter of one --pmc run (one row per kernel)

The calibration copy is summed over all of its dispatches: torch splits an
elementwise kernel whose byte offsets overflow 32 bits (a 4 GiB copy) into
several launches.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import sys
from collections import defaultdict

# kernel key -> pattern on the (demangled or mangled) kernel name
KERNELS = {
    "attn_selected": r"k_attn<[^,]+, \d+, 1>|k_attnI\w+Li1EEEv|k_attn4<1[,>]|k_attn4ILi1E",
    "attn_self": r"k_attn<[^,]+, \d+, 0>|k_attnI\w+Li0EEEv|k_attn4<0[,>]|k_attn4ILi0E",
    "attn_dense": r"k_attn<[^,]+, \d+, 2>|k_attnI\w+Li2EEEv",
    "gate_fast": r"k_gate_fast",
    "gate_bound": r"k_gate_bound",
    "gate": r"k_gate\b|k_gateI",
    "pool": r"k_pool",
    "kbar_append": r"k_kbar_append",
    "decode_gate": r"k_dec_gate",
    "decode_part": r"k_dec_part",
    "decode_merge": r"k_dec_merge",
    "bwd_delta": r"k_bwd_delta",
    "bwd_dq_selected": r"k_bwd_dq_dma<1>|k_bwd_dq_dmaILi1E|k_bwd_dq<[^>]*, 1>|k_bwd_dqI\w+Li1EEEv",
    "bwd_dq_self": r"k_bwd_dq_dma<0>|k_bwd_dq_dmaILi0E|k_bwd_dq<[^>]*, 0>|k_bwd_dqI\w+Li0EEEv",
    "bwd_dkdv": r"k_bwd_dkdv",
    "route_count": r"k_route_count",
    "route_lists": r"k_route_lists",
    "route_offsets": r"k_route_offsets",
    "route_scatter": r"k_route_scatter",
    "setup": r"k_setup|k_block_info",
    "slab_copy": r"k_copy_rows",
    "copy_calibration": r"neg_kernel",
}


def kernel_key(name: str) -> str:
    for key, pat in KERNELS.items():
        if re.search(pat, name):
            return key
    return "other"


def _find(dirpath: str, suffix: str) -> list[str]:
    return sorted(glob.glob(os.path.join(dirpath, "**", "*" + suffix), recursive=True))


def _col(header, *cands):
    low = [h.lower() for h in header]
    for c in cands:
        if c.lower() in low:
            return low.index(c.lower())
    raise KeyError("none of %s in %s" % (cands, header))


def stats(dirpath: str) -> str:
    files = _find(dirpath, "kernel_stats.csv")
    if not files:
        raise FileNotFoundError("no *kernel_stats.csv under " + dirpath)
    rows = []
    for f in files:
        with open(f) as fh:
            r = csv.reader(fh)
            hdr = next(r)
            i_n, i_c = _col(hdr, "Name", "KernelName"), _col(hdr, "Calls")
            i_t, i_a = _col(hdr, "TotalDurationNs"), _col(hdr, "AverageNs")
            for row in r:
                rows.append((kernel_key(row[i_n]), row[i_n], int(row[i_c]), float(row[i_t]),
                             float(row[i_a])))
    rows.sort(key=lambda x: -x[3])
    out = ["| kernel | calls | avg ms | total ms | name |", "|---|---|---|---|---|"]
    for key, name, calls, tot, avg in rows:
        out.append("| %s | %d | %.4f | %.3f | %s |" % (key, calls, avg / 1e6, tot / 1e6,
                                                     name[:90]))
    return "\n".join(out)


def _counter_per_dispatch(dirpath: str, counter: str) -> dict:
    files = _find(dirpath, "counter_collection.csv")
    if not files:
        raise FileNotFoundError("no *counter_collection.csv under " + dirpath)
    per = defaultdict(lambda: defaultdict(float))   # key -> dispatch -> value
    for f in files:
        with open(f) as fh:
            r = csv.reader(fh)
            hdr = next(r)
            i_n = _col(hdr, "Kernel_Name", "Kernel-Name", "KernelName")
            i_d = _col(hdr, "Dispatch_Id", "Dispatch-Id", "DispatchId", "Correlation_Id")
            i_cn = _col(hdr, "Counter_Name", "Counter-Name")
            i_cv = _col(hdr, "Counter_Value", "Counter-Value")
            for row in r:
                if row[i_cn] != counter:
                    continue
                per[kernel_key(row[i_n])][row[i_d]] += float(row[i_cv])
    return {k: sorted(v.values()) for k, v in per.items()}


def _copy_total(per: dict) -> float:
    """Counter total over every dispatch of the calibration copy."""
    return sum(per.get("copy_calibration", [0.0]))


def traffic(fetch_dir: str, write_dir: str, copy_mib: int, kernel: str) -> str:
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    cal_bytes = copy_mib * 1024.0 * 1024.0
    f_copy = _copy_total(fetch) * 1024.0
    w_copy = _copy_total(write) * 1024.0
    f_scale = cal_bytes / f_copy if f_copy > 0 else float("nan")
    w_scale = cal_bytes / w_copy if w_copy > 0 else float("nan")
    fk = fetch.get(kernel, [])
    wk = write.get(kernel, [])
    f_mean = sum(fk) / len(fk) * 1024.0 if fk else float("nan")
    w_mean = sum(wk) / len(wk) * 1024.0 if wk else float("nan")
    lines = [
        "kernel: %s" % kernel,
        "launches_fetch: %d" % len(fk),
        "launches_write: %d" % len(wk),
        "fetch_bytes_raw_per_launch: %.6g" % f_mean,
        "write_bytes_raw_per_launch: %.6g" % w_mean,
        "copy_calibration_bytes: %.6g" % cal_bytes,
        "copy_fetch_raw: %.6g" % f_copy,
        "copy_write_raw: %.6g" % w_copy,
        "fetch_scale: %.6g" % f_scale,
        "write_scale: %.6g" % w_scale,
        "hbm_read_bytes_per_launch: %.6g" % (f_mean * f_scale),
        "hbm_write_bytes_per_launch: %.6g" % (w_mean * w_scale),
        "hbm_bytes_per_launch: %.6g" % (f_mean * f_scale + w_mean * w_scale),
    ]
    return "\n".join(lines)


DRAM_READ = "TCC_EA0_RDREQ_DRAM_32B_sum"
DRAM_WRITE = "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"


def dram(dirpath: str, copy_mib: int) -> str:
    rd = _counter_per_dispatch(dirpath, DRAM_READ)
    wr = _counter_per_dispatch(dirpath, DRAM_WRITE)
    cal_bytes = copy_mib * 1024.0 * 1024.0
    r_copy = _copy_total(rd) * 32.0
    w_copy = _copy_total(wr) * 32.0
    out = ["copy_calibration_bytes: %.6g" % cal_bytes,
           "copy_read_bytes: %.6g (ratio %.4f)" % (r_copy, r_copy / cal_bytes),
           "copy_write_bytes: %.6g (ratio %.4f)" % (w_copy, w_copy / cal_bytes),
           "",
           "| kernel | launches | GB read / launch | GB written / launch |",
           "|---|---|---|---|"]
    keys = sorted(set(rd) | set(wr), key=lambda k: -(sum(rd.get(k, [0])) + sum(wr.get(k, [0]))))
    for k in keys:
        if k == "copy_calibration":
            continue
        r, w = rd.get(k, []), wr.get(k, [])
        n = max(len(r), len(w))
        out.append("| %s | %d | %.4f | %.4f |" % (
            k, n, (sum(r) / len(r) * 32e-9) if r else float("nan"),
            (sum(w) / len(w) * 32e-9) if w else float("nan")))
    return "\n".join(out)


def counters(dirpath: str) -> str:
    files = _find(dirpath, "counter_collection.csv")
    if not files:
        raise FileNotFoundError("no *counter_collection.csv under " + dirpath)
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))  # key -> ctr -> disp
    for f in files:
        with open(f) as fh:
            r = csv.reader(fh)
            hdr = next(r)
            i_n = _col(hdr, "Kernel_Name", "Kernel-Name", "KernelName")
            i_d = _col(hdr, "Dispatch_Id", "Dispatch-Id", "DispatchId", "Correlation_Id")
            i_cn = _col(hdr, "Counter_Name", "Counter-Name")
            i_cv = _col(hdr, "Counter_Value", "Counter-Value")
            for row in r:
                per[kernel_key(row[i_n])][row[i_cn]][row[i_d]] += float(row[i_cv])
    names = sorted({c for k in per.values() for c in k})
    out = ["| kernel | " + " | ".join(names) + " |", "|---" * (len(names) + 1) + "|"]
    for key in sorted(per):
        vals = []
        for c in names:
            d = per[key].get(c, {})
            vals.append("%.4g" % (sum(d.values()) / len(d)) if d else "")
        out.append("| %s | %s |" % (key, " | ".join(vals)))
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--kernel", default="attn_selected")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    m = sub.add_parser("dram")
    m.add_argument("dir")
    m.add_argument("--copy-mib", type=int, required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats(a.dir))
    elif a.cmd == "dram":
        print(dram(a.dir, a.copy_mib))
    elif a.cmd == "counters":
        print(counters(a.dir))
    else:
        print(traffic(a.fetch_dir, a.write_dir, a.copy_mib, a.kernel))


if __name__ == "__main__":
    sys.exit(main())
