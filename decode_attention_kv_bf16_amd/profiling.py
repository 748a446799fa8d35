"""Summaries of rocprofv3 output for this library's kernels.

    python -m decode_attention_kv_bf16_amd.profiling stats KERNEL_STATS_CSV --command CMD --out FILE.md
    python -m decode_attention_kv_bf16_amd.profiling traffic --fetch FETCH_DIR --write WRITE_DIR \
        --copy-bytes N --fetch-command CMD --write-command CMD --workload NAME --out-md FILE.md

    python -m decode_attention_kv_bf16_amd.profiling counters DIR [DIR ...] --command CMD \
        [--command CMD ...] --out FILE.md
    python -m decode_attention_kv_bf16_amd.profiling parity RECORD.json --command CMD --out FILE.md

`stats` turns a `--kernel-trace --stats --output-format csv` run into a
per-kernel table of launch durations. `traffic` turns two counter runs
(`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, both over a command that ends
with a device-to-device copy of N bytes) into HBM bytes per launch: each
counter's per-dispatch average (KiB) is scaled by the factor that makes the
same counter read N bytes for the copy kernel (the last copy dispatch of the
run). The result is merged into profiles/hbm_traffic.json, keyed by the
bench workload (`--key`, its --workload value) and then by kernel, with the
sha256 of the source files that hold the kernel, so that a reader can tell
whether the figures still describe the current code. `counters`
averages any `--pmc` counters per kernel and dispatch over one or more counter
runs and derives, where its inputs were collected, the matrix-core, vector-ALU
and LDS utilisation and the shader clock (see counter_table). `parity` turns
the record a GPU test run writes (DA_PARITY_RECORD=path) into a table of the
largest errors of every parity check.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
from collections import defaultdict

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
PROFILE_DIR = os.path.join(ROOT, "profiles")

# short kernel name -> (substring of the device symbol, substrings of which
# one must also occur, source file); the first entry that matches names a
# symbol. The attention kernel's last template argument is the paged flag
# (mangled "Lb1E", demangled ", true>": paged pool).
KERNELS = {
    # the GQA pass runs on the matrix cores (gqa_mfma_kernel) or, for fp32
    # and 16-wave shapes, on the vector ALUs (gqa_decode_kernel)
    "gqa_split_pass": ("_kernel", ("gqa_decode_kernel", "gqa_mfma_kernel"), ("gqa_decode.hip", "gqa_mfma.hip")),
    "gqa_combine": ("splitkv_combine_kernel", (), "combine.hip"),
    "mla_absorb": ("mla_absorb_kernel", (), ("mla_decode.hip", "mla_common.h")),
    # the E4M3 latent kernel first: its name also contains "mla_attend"
    "mla_attend_fp8_paged": ("mla_attend_fp8_kernel", ("Lb1E", ", true>"), ("mla_fp8.hip", "mla_common.h")),
    "mla_attend_fp8": ("mla_attend_fp8_kernel", (), ("mla_fp8.hip", "mla_common.h")),
    # 16 or 48 heads: mla_attend_kernel; multiples of 32: mla_attend32_kernel
    "mla_attend_paged": ("mla_attend", ("Lb1E", ", true>"), ("mla_decode.hip", "mla_common.h")),
    "mla_attend": ("mla_attend", ("mla_attend_kernel", "mla_attend32_kernel"), ("mla_decode.hip", "mla_common.h")),
    "mla_merge_project": ("mla_merge_project_kernel", (), ("mla_decode.hip", "mla_common.h")),
    "gqa_append_rope_fp8": ("gqa_append_rope_fp8_kernel", (), "append_rope.hip"),
    "gqa_append_rope": ("gqa_append_rope_kernel", (), "append_rope.hip"),
    "mla_append_rope": ("mla_append_rope_kernel", (), "append_rope.hip"),
    "probe_stream_read": ("stream_read_kernel", (), "hbm_probe.hip"),
    "probe_stream_copy": ("stream_copy_kernel", (), "hbm_probe.hip"),
}
# names under which a workload's launches of a kernel are recorded (GQA over
# paged pools runs the GQA kernel as one library call, gqa_decode_paged)
ALIASES = {"gqa_decode_paged": "gqa_split_pass", "gqa_decode_fp8": "gqa_split_pass",
           "gqa_window": "gqa_split_pass", "gqa_decode_fp8_paged": "gqa_split_pass"}


def source_sha256(short: str):
    short = ALIASES.get(short, short)
    if short not in KERNELS:
        return None
    files = KERNELS[short][2]
    h = hashlib.sha256()
    for name in (files if isinstance(files, tuple) else (files,)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(symbol: str):
    for short, (sub, any_of, _) in KERNELS.items():
        if sub in symbol and (not any_of or any(s in symbol for s in any_of)):
            return short
    return None


def _find(path: str, suffix: str) -> str:
    if os.path.isfile(path):
        return path
    for dirpath, _, files in os.walk(path):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(dirpath, f)
    raise FileNotFoundError(f"no *{suffix} under {path}")


def stats_table(stats_csv: str, rename=lambda s: s) -> str:
    rows = list(csv.DictReader(open(_find(stats_csv, "kernel_stats.csv"))))
    lines = ["| kernel | symbol | calls | avg us | min us | max us | share % |",
             "|---|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        sym = r["Name"]
        short = short_name(sym)
        lines.append(f"| {rename(short) if short else '-'} | `{sym[:90]}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    return "\n".join(lines)


def _renamer(pairs):
    """--rename KERNEL=NAME options as a function on short names."""
    m = dict(p.split("=", 1) for p in pairs)
    for new in m.values():
        if ALIASES.get(new, new) not in KERNELS:
            raise SystemExit(f"unknown kernel name {new}")
    return lambda s: m.get(s, s)


def tail_table(trace_dir: str, tail: int, rename=lambda s: s) -> str:
    """Per kernel, the average duration of its last `tail` dispatches in the
    kernel trace (the launches of the bench's last pass)."""
    rows = list(csv.DictReader(open(_find(trace_dir, "kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = defaultdict(list)
    for r in rows:
        s = short_name(r["Kernel_Name"])
        if s:
            per[rename(s)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"| kernel | dispatches | avg us, last {tail} | min us | max us |", "|---|---:|---:|---:|---:|"]
    for k, d in sorted(per.items()):
        last = d[-tail:]
        lines.append(f"| {k} | {len(d)} | {sum(last) / len(last):.2f} | {min(last):.2f} | {max(last):.2f} |")
    return "\n".join(lines)


def bench_roofline(log_path: str):
    """The roofline object of the bench JSON line in a profiled run's output."""
    for line in open(log_path):
        if line.startswith("{"):
            return json.loads(line).get("roofline")
    return None


def counter_averages(counter_dir: str, counter: str, rename=lambda s: s):
    """Per short kernel name: average counter value per dispatch, and the value
    for the last copy-kernel dispatch of the run (the calibration copy)."""
    rows = list(csv.DictReader(open(_find(counter_dir, "counter_collection.csv"))))
    per = defaultdict(list)
    copy_val = None
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        if "copyBuffer" in r["Kernel_Name"]:
            copy_val = v
            continue
        s = short_name(r["Kernel_Name"])
        if s:
            per[rename(s)].append(v)
    return {k: sum(v) / len(v) for k, v in per.items()}, {k: len(v) for k, v in per.items()}, copy_val


def _dispatches(counter_dir: str, rename=lambda s: s):
    """{dispatch id: (short kernel name, duration ns, {counter: value})} of one
    counter run; dispatches of kernels outside this library are dropped."""
    out = {}
    for r in csv.DictReader(open(_find(counter_dir, "counter_collection.csv"))):
        s = short_name(r["Kernel_Name"])
        if not s:
            continue
        d = out.setdefault(r["Dispatch_Id"], [rename(s), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), {}])
        d[2][r["Counter_Name"]] = float(r["Counter_Value"])
    return out


def counter_table(dirs, cus: int = 256, xccs: int = 8):
    """Per kernel: dispatches, mean duration under counters, the mean of every
    counter collected, and derived figures that follow rocprofv3's own
    derived-counter definitions (its --list-avail output). A counter with
    per-XCC instances is summed over the XCCs in the CSV, so GRBM_GUI_ACTIVE is
    divided by their number to give the elapsed GPU cycles of one XCC (what
    those definitions reduce with max):
      mfma_busy_pct  = 100 SQ_VALU_MFMA_BUSY_CYCLES / (gui * 4 * CUs)   (MfmaUtil)
      valu_busy_pct  = 100 SQ_ACTIVE_INST_VALU / CUs / gui              (VALUBusy)
      lds_busy_pct   = 100 SQ_LDS_IDX_ACTIVE / (gui * CUs)              (LdsUtil)
      lds_conflicts_per_access = SQ_LDS_BANK_CONFLICT /
                                 (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT) (LdsBankConflict)
      sclk_ghz       = gui / duration_ns
    Derived counters requested by name (MfmaUtil, ...) are averaged as they are."""
    per = defaultdict(lambda: {"n": 0, "dur": [], "vals": defaultdict(list)})
    for d in dirs:
        for _, (name, dur, vals) in _dispatches(d).items():
            rec = per[name]
            rec["dur"].append(dur)
            for k, v in vals.items():
                rec["vals"][k].append(v)
    rows = {}
    for name, rec in per.items():
        mean = {k: sum(v) / len(v) for k, v in rec["vals"].items()}
        dur = sum(rec["dur"]) / len(rec["dur"])
        row = {"dispatches": len(rec["dur"]), "duration_us": dur / 1e3, "counters": mean}
        gui = mean.get("GRBM_GUI_ACTIVE")
        if gui:
            gui /= xccs
            row["sclk_ghz"] = gui / dur
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                row["mfma_busy_pct"] = 100 * mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * 4 * cus)
            if "SQ_ACTIVE_INST_VALU" in mean:
                row["valu_busy_pct"] = 100 * mean["SQ_ACTIVE_INST_VALU"] / cus / gui
            if "SQ_LDS_IDX_ACTIVE" in mean:
                row["lds_busy_pct"] = 100 * mean["SQ_LDS_IDX_ACTIVE"] / (gui * cus)
        if "SQ_LDS_BANK_CONFLICT" in mean and "SQ_LDS_IDX_ACTIVE" in mean:
            den = mean["SQ_LDS_IDX_ACTIVE"] - mean["SQ_LDS_BANK_CONFLICT"]
            row["lds_conflicts_per_access"] = mean["SQ_LDS_BANK_CONFLICT"] / den if den > 0 else None
        rows[name] = row
    return rows


def parity_table(rec: dict, command: str) -> str:
    """Markdown table of a GPU test run's parity record: per check, the
    largest row-relative output error and |lse error| with the bars it was
    held to; a summary line for the MLA checks."""
    rows = sorted(rec["checks"].items())
    mla = [v for k, v in rows if "mla" in k.lower()]
    lines = ["# GPU parity: largest errors per check", "", "Command (from the repository root, on one MI355X):", "",
             "    " + command, "",
             f"pytest exit status {rec['exitstatus']}; {len(rows)} parity checks. Bar: row-relative output error "
             "<= 1e-2, |lse error| <= 1e-3 (some checks also hold a tighter per-row bound, shown as out_rtol).", ""]
    if mla:
        lines += [f"MLA checks: {len(mla)}; largest |lse error| {max(v['max_lse_abs_err'] for v in mla):.2e}; "
                  f"largest row-relative output error {max(v['max_row_rel_err'] for v in mla):.2e}.", ""]
    lines += ["| max row rel err | max lse err | out_rtol | lse_atol | test :: check |", "|---|---|---|---|---|"]
    for k, v in rows:
        lines.append(f"| {v['max_row_rel_err']:.2e} | {v['max_lse_abs_err']:.2e} | {v['out_rtol']:.1e} | "
                     f"{v['lse_atol']:.0e} | {k.replace('tests/', '').replace('|', '/')} |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="rocprofv3 kernel durations")
    s.add_argument("--out", required=True)
    s.add_argument("--rename", action="append", default=[], help="KERNEL=NAME")
    s.add_argument("--tail", type=int, default=0,
                   help="also average each kernel's last N dispatches (the bench's roofline pass)")
    s.add_argument("--bench-log", help="stdout of the profiled bench run (its JSON line)")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--fetch-command", required=True)
    t.add_argument("--write-command", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--key", required=True, help="the bench's --workload value the runs used")
    t.add_argument("--alg-bytes", default="{}", help="JSON {kernel: algorithmic bytes per launch}")
    t.add_argument("--out-md", required=True)
    t.add_argument("--rename", action="append", default=[], help="KERNEL=NAME")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--title", default="rocprofv3 counters per kernel")
    c.add_argument("--note", default="")
    c.add_argument("--out", required=True)
    pr = sub.add_parser("parity")
    pr.add_argument("record")
    pr.add_argument("--command", required=True)
    pr.add_argument("--out", required=True)
    a = ap.parse_args(argv)

    if a.cmd == "parity":
        text = parity_table(json.load(open(a.record)), a.command)
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
        return

    if a.cmd == "counters":
        rows = counter_table(a.dirs)
        derived = ("sclk_ghz", "mfma_busy_pct", "valu_busy_pct", "lds_busy_pct", "lds_conflicts_per_access")
        names = sorted({k for r in rows.values() for k in r["counters"]})
        lines = [f"# {a.title}", "", "Counter runs (from the repository root):", "", "```", *a.command, "```", ""]
        if a.note:
            lines += [a.note, ""]
        lines += ["Derived figures (rocprofv3's own definitions, GRBM_GUI_ACTIVE taken per XCC):", "",
                  "| kernel | dispatches | us under counters | " + " | ".join(derived) + " |",
                  "|---|---:|---:|" + "---:|" * len(derived)]
        fmt = lambda v: "-" if v is None else f"{v:.3g}"
        for k in sorted(rows):
            r = rows[k]
            lines.append(f"| {k} | {r['dispatches']} | {r['duration_us']:.2f} | "
                         + " | ".join(fmt(r.get(d)) for d in derived) + " |")
        lines += ["", "Counter means per dispatch (hardware counters summed over the device's instances; "
                  "rocprofv3's derived counters as it reports them):", "",
                  "| kernel | " + " | ".join(names) + " |", "|---|" + "---:|" * len(names)]
        for k in sorted(rows):
            lines.append(f"| {k} | " + " | ".join(fmt(rows[k]["counters"].get(n)) for n in names) + " |")
        with open(a.out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return

    if a.cmd == "stats":
        rn = _renamer(a.rename)
        text = (f"# {a.title}\n\nCommand (run from the repository root):\n\n```\n{a.command}\n```\n\n"
                f"All dispatches of the run (rocprofv3 --stats):\n\n{stats_table(a.csv, rn)}\n")
        if a.tail:
            text += (f"\nLast {a.tail} dispatches of each kernel (the bench's roofline pass, after "
                     f"warm-up, probe and timed passes):\n\n{tail_table(a.csv, a.tail, rn)}\n")
        if a.bench_log:
            rf = bench_roofline(a.bench_log)
            if rf:
                text += (f"\nThe bench line of this profiled run: dominant kernel `{rf['kernel']}`, "
                         f"{rf['avg_launch_us']} us per launch from HIP events around each launch "
                         f"of its roofline pass (events add a little to each launch).\n")
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
        return

    rn = _renamer(a.rename)
    fetch, nf, fcopy = counter_averages(a.fetch, "FETCH_SIZE", rn)
    write, nw, wcopy = counter_averages(a.write, "WRITE_SIZE", rn)
    if not fcopy or not wcopy:
        raise SystemExit("no calibration copy dispatch found in the counter runs")
    copy_kib = a.copy_bytes / 1024.0
    ff, wf = copy_kib / fcopy, copy_kib / wcopy
    alg = json.loads(a.alg_bytes)
    path = os.path.join(PROFILE_DIR, "hbm_traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    lines = [f"# HBM traffic per launch: {a.workload}", "",
             "Counter runs (from the repository root):", "", "```", a.fetch_command, a.write_command, "```", "",
             f"Calibration: a device-to-device copy of {a.copy_bytes} bytes at the end of each run reads "
             f"FETCH_SIZE = {fcopy:.1f} KiB and WRITE_SIZE = {wcopy:.1f} KiB, so the counters are scaled by "
             f"{ff:.3f} (fetch) and {wf:.3f} (write).", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / launch (scaled) | algorithmic bytes | ratio |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for k in sorted(set(fetch) & set(write)):
        b = fetch[k] * 1024 * ff + write[k] * 1024 * wf
        ab = alg.get(k)
        ratio = f"{b / ab:.3f}" if ab else "-"
        lines.append(f"| {k} | {nf[k]} | {fetch[k]:.1f} | {write[k]:.1f} | {b:.4g} | {ab if ab else '-'} | {ratio} |")
        rec.setdefault(a.key, {})[k] = dict(bytes_per_launch=b, fetch_kib=fetch[k], write_kib=write[k],
                                            fetch_factor=ff, write_factor=wf, workload=a.workload,
                                            source_sha256=source_sha256(k), algorithmic_bytes=ab)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
