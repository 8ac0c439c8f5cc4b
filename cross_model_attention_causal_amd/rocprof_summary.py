"""Turn rocprofv3 output (CSV) into the short summaries kept with the repository.

    python -m cross_model_attention_causal_amd.rocprof_summary kernel-time DIR OUT.md --title T --cmd CMD
        kernel_stats.csv of a `rocprofv3 --kernel-trace --stats` run -> per-kernel table
    python -m cross_model_attention_causal_amd.rocprof_summary traffic FETCH WRITE CFETCH CWRITE OUT.md OUT.json \
        --workload W --cmd CMD --cal-cmd CMD
        counter_collection.csv of FETCH_SIZE and WRITE_SIZE runs of a workload and of the
        1 GiB copy calibration (bench.py --calibrate-copy) -> bytes per launch, scaled by
        what the counters read for the copy, and the JSON bench.py reads (with the SHA-256
        of each kernel's source and the shared headers, so a changed kernel drops it)
    python -m cross_model_attention_causal_amd.rocprof_summary counters OUT.md DIR [DIR ...] --kernel REGEX \
        --title T --cmd CMD
        counter_collection.csv of one or more --pmc runs -> per-launch averages per counter

Each DIR is a rocprofv3 output directory; the CSV files are found below it.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
HEADERS = ["common.hpp", "kernels.hpp", "score.hpp"]
# kernel -> source file (for the SHA that ties a traffic figure to the code it measured)
KERNEL_SOURCE = {
    "k_mapped_av_bsr": "mapped_av.hip", "k_mapped_av_idx": "mapped_av.hip", "k_mapped_av_dense": "mapped_av.hip",
    "k_tile_v": "mapped_av.hip", "k_block_stats": "compress.hip", "k_block_extract": "compress.hip",
    "k_bsr_scan": "compress.hip", "k_attn_maps_short": "attn_maps.hip", "k_attn_maps": "attn_maps.hip",
    "k_attn_rows": "attn_maps.hip", "k_gram_bf16": "cosine.hip", "k_cos_finalize": "cosine.hip",
    "k_head_map_fused": "cosine.hip",
}


def find_csv(d, name):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{name}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{name} under {d}")
    return hits[0]


def short_name(kernel):
    """`void cma::k_block_stats<128, 2>(cma::CompressArgs)` -> k_block_stats."""
    m = re.search(r"(k_[a-z0-9_]+)", kernel)
    return m.group(1) if m else kernel


def source_sha(name):
    src = KERNEL_SOURCE.get(name)
    if not src:
        return None, None
    h = hashlib.sha256()
    for f in [src] + HEADERS:
        h.update(open(os.path.join(SRC, f), "rb").read())
    return src, h.hexdigest()


def kernel_time(args):
    rows = list(csv.DictReader(open(find_csv(args.dir, "kernel_stats.csv"))))
    out = [f"# {args.title}", "", "Command:", "", "```", args.cmd, "```", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share of kernel time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r.get("Name") or r.get("KERNEL_NAME")
        out.append(f"| `{name[:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} % |")
    open(args.out, "w").write("\n".join(out) + "\n")


def counter_means(d, kernel_re=None):
    """{kernel: {counter: mean per dispatch}} from a counter_collection.csv."""
    rows = list(csv.DictReader(open(find_csv(d, "counter_collection.csv"))))
    acc = {}
    for r in rows:
        k = r.get("Kernel_Name") or r.get("Kernel-Name")
        if kernel_re and not re.search(kernel_re, k):
            continue
        c = r.get("Counter_Name") or r.get("Counter-Name")
        v = float(r.get("Counter_Value") or r.get("Counter-Value"))
        disp = r.get("Dispatch_Id") or r.get("Dispatch-Id")
        acc.setdefault(k, {}).setdefault(c, {}).setdefault(disp, 0.0)
        acc[k][c][disp] += v  # per-dimension rows of one dispatch add up
    return {k: {c: sum(d.values()) / len(d) for c, d in cs.items()} for k, cs in acc.items()}


def traffic(args):
    fetch, write = counter_means(args.fetch), counter_means(args.write)
    cf, cw = counter_means(args.cal_fetch), counter_means(args.cal_write)
    n = 1 << 30  # the calibration copy reads and writes 1 GiB per launch
    # the copy is the calibration run's largest kernel (the run also fills the source)
    cal_f = max(v["FETCH_SIZE"] for k, v in cf.items() if "FETCH_SIZE" in v and "copy" in k.lower())
    cal_w = max(v["WRITE_SIZE"] for k, v in cw.items() if "WRITE_SIZE" in v and "copy" in k.lower())
    ff, fw = n / 1024 / cal_f, n / 1024 / cal_w
    md = [f"# HBM traffic per launch, {args.workload} (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)", "",
          f"Each counter in its own run. Calibration: a plain device copy of 1 GiB reads {cal_f:.0f} KiB by "
          f"FETCH_SIZE and writes {cal_w:.0f} KiB by WRITE_SIZE per launch, so bytes = FETCH_SIZE x 1024 x {ff:.4f} "
          f"and WRITE_SIZE x 1024 x {fw:.4f}.", "", "Commands ({C} = FETCH_SIZE, then WRITE_SIZE):", "", "```",
          args.cmd, args.cal_cmd, "```", "",
          "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read (GB) | written (GB) | total (GB) |",
          "|---|---|---|---|---|---|"]
    js = {}
    for k in sorted(set(fetch) | set(write)):
        f = fetch.get(k, {}).get("FETCH_SIZE", 0.0)
        w = write.get(k, {}).get("WRITE_SIZE", 0.0)
        rb, wb = f * 1024 * ff, w * 1024 * fw
        md.append(f"| `{k[:60]}` | {f:.0f} | {w:.0f} | {rb / 1e9:.3f} | {wb / 1e9:.3f} | {(rb + wb) / 1e9:.3f} |")
        name = short_name(k)
        src, sha = source_sha(name)
        if src:
            js[name] = dict(source=src, headers=HEADERS, sha256=sha, bytes_per_launch=int(rb + wb),
                            read_bytes=int(rb), write_bytes=int(wb), fetch_kib=f, write_kib=w, fetch_factor=ff,
                            write_factor=fw, workload=args.workload)
    open(args.out_md, "w").write("\n".join(md) + "\n")
    json.dump(js, open(args.out_json, "w"), indent=1)


def counters(args):
    merged = {}
    for d in args.dirs:
        for k, cs in counter_means(d, args.kernel).items():
            merged.setdefault(k, {}).update(cs)
    md = [f"# {args.title}", "", "Commands (one counter group per run):", "", "```", args.cmd, "```", ""]
    md += ["Derived (per launch; GRBM_GUI_ACTIVE counts cycles on each of the 8 XCDs, the SQ_ counters add",
           "over the 256 CUs, and SQ_VALU_MFMA_BUSY_CYCLES over their 4 SIMDs each):", "",
           "* cycles = GRBM_GUI_ACTIVE / 8;",
           "* MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles);",
           "* CU busy = SQ_BUSY_CU_CYCLES / (256 x cycles);",
           "* VALU share = 4 x SQ_INSTS_VALU / (1024 SIMDs x cycles) (a wave64 vector instruction issues over 4 cycles",
           "  on a 16-lane SIMD; transcendental ones take longer, so this is a lower bound);",
           "* LDS conflict share = SQ_LDS_BANK_CONFLICT / (256 x cycles);",
           "* address unit busy = TA_BUSY_avr / cycles.", ""]
    for k, cs in merged.items():
        md += [f"Kernel `{k[:80]}`, per launch:", "", "| counter | value |", "|---|---|"]
        md += [f"| `{c}` | {v:.4g} |" for c, v in sorted(cs.items())]
        g = cs.get("GRBM_GUI_ACTIVE")
        if g:
            cyc = g / 8
            der = []
            if "SQ_VALU_MFMA_BUSY_CYCLES" in cs:
                der.append(("MFMA busy", cs["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cyc)))
            if "SQ_BUSY_CU_CYCLES" in cs:
                der.append(("CU busy", cs["SQ_BUSY_CU_CYCLES"] / (256 * cyc)))
            if "SQ_INSTS_VALU" in cs:
                der.append(("VALU share", 4 * cs["SQ_INSTS_VALU"] / (1024 * cyc)))
            if "SQ_LDS_BANK_CONFLICT" in cs:
                der.append(("LDS conflict share", cs["SQ_LDS_BANK_CONFLICT"] / (256 * cyc)))
            if "TA_BUSY_avr" in cs:
                der.append(("address unit busy", cs["TA_BUSY_avr"] / cyc))
            md += [f"| {name} | {val:.3f} |" for name, val in der]
        md.append("")
    open(args.out, "w").write("\n".join(md) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("kernel-time")
    a.add_argument("dir")
    a.add_argument("out")
    a.add_argument("--title", required=True)
    a.add_argument("--cmd", required=True)
    b = sub.add_parser("traffic")
    for x in ("fetch", "write", "cal_fetch", "cal_write", "out_md", "out_json"):
        b.add_argument(x)
    b.add_argument("--workload", required=True)
    b.add_argument("--cmd", required=True)
    b.add_argument("--cal-cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", default=None)
    c.add_argument("--title", required=True)
    c.add_argument("--cmd", required=True)
    args = ap.parse_args(argv)
    {"kernel-time": kernel_time, "traffic": traffic, "counters": counters}[args.what](args)


if __name__ == "__main__":
    sys.exit(main())
