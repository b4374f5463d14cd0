"""rocprofv3 evidence for bench.py: kernel trace + stats of the timed command,
HBM bytes per launch from FETCH_SIZE and WRITE_SIZE counter passes (one
counter per run), calibrated on a plain device copy of known size.

    python bench_profile.py --workload 2 [--steps 10] [--out rocprof_raw]
    python bench_profile.py --zero2 [--workload 3] [--fused-final]  (the ZeRO-2 streaming leg of bench.py)
    python bench_profile.py --queues --workload 4      (HBM request latency and credit stalls per kernel)

Needs an MI355X with rocprofv3. Writes:
  profiles/<kernel>_<workload tag>.md   the figures used and the commands that made them
  profiles/traffic.json                 HBM bytes per launch of the dominant kernel and per
                                        step (every launch of the step), keyed by workload and
                                        the hash of the kernel source (bench.py reports it only
                                        while that hash is current)
Raw rocprofv3 output stays under --out.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
TAGS = {0: "tiny_n262144_M4", 1: "gpt2_bucket_n15554976_M8", 2: "7p5B_shard_n117187500_M64",
        3: "llama7b_ragged_n809533440_M8", 4: "amp_shard_n2e9_M8"}


def src_hash() -> str:
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash  # one definition: bench.py checks the profile with it
    return kernel_source_hash()


def run(cmd, log):
    print("+", " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, cwd=ROOT, timeout=600)
    if r.returncode != 0:
        sys.exit(f"command failed ({r.returncode}): {' '.join(cmd)}; see {log}")


def one(pattern):
    hits = glob.glob(pattern)
    if len(hits) != 1:
        sys.exit(f"expected one file for {pattern}, found {hits}")
    return hits[0]


def counter_per_dispatch(path, kernel_pred):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if kernel_pred(r["Kernel_Name"])]
    if not vals:
        sys.exit(f"no matching dispatch in {path}")
    return sum(vals) / len(vals), len(vals)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--out", default="rocprof_raw", help="raw rocprofv3 output (relative; not committed)")
    ap.add_argument("--profiles-dir", default="profiles", help="where the summaries go (relative)")
    ap.add_argument("--summarize-only", action="store_true", help="re-read existing raw output, run nothing")
    ap.add_argument("--zero2", action="store_true", help="profile bench.py --zero2 (one micro-batch)")
    ap.add_argument("--queues", action="store_true",
                    help="HBM request queues instead: average read and write latency at the L2-fabric interface "
                         "and DRAM-credit stalls, per kernel of the bench command (two counter passes)")
    ap.add_argument("--fused-final", action="store_true",
                    help="with --zero2: the fused final pass (bench.py --zero2 --fused-final)")
    a = ap.parse_args()
    if a.queues:
        return main_queues(a)
    if a.zero2:
        return main_zero2(a)
    sys.path.insert(0, ROOT)
    from synth.workloads import workload
    w = workload(a.workload)
    out = os.path.join(a.out, f"w{a.workload}")  # relative to the repository root
    os.chdir(ROOT)
    os.makedirs(out, exist_ok=True)
    profiles = a.profiles_dir
    # clean steps only: a workload with inf injection also times skipped steps
    # by default, whose update launches exit early and would mix into the trace
    bench = ["python", "-u", "bench.py", "--workload", str(a.workload), "--cpu-sample", "0", "--steps",
             str(a.steps), "--warmup", "2", "--no-skipped-leg"]
    calib = ["python", "-u", "bench.py", "--calib-copy", "--steps", "3"]
    rp = "rocprofv3"
    cmds = {
        "trace": [rp, "--kernel-trace", "--stats", "--output-format", "csv", "-d", f"{out}/trace", "-o", "run",
                  "--"] + bench,
        "fetch": [rp, "--pmc", "FETCH_SIZE", "--output-format", "csv", "-d", f"{out}/fetch", "-o", "run", "--"] + bench,
        "write": [rp, "--pmc", "WRITE_SIZE", "--output-format", "csv", "-d", f"{out}/write", "-o", "run", "--"] + bench,
        "cfetch": [rp, "--pmc", "FETCH_SIZE", "--output-format", "csv", "-d", f"{out}/cfetch", "-o", "run", "--"] + calib,
        "cwrite": [rp, "--pmc", "WRITE_SIZE", "--output-format", "csv", "-d", f"{out}/cwrite", "-o", "run", "--"] + calib,
    }
    if not a.summarize_only:
        for k, c in cmds.items():
            run(c, f"{out}/{k}.log")

    stats = list(csv.DictReader(open(one(f"{out}/trace/run_kernel_stats.csv"))))
    ours = [r for r in stats if "fused_kernel" in r["Name"] or "finalize_kernel" in r["Name"]
            or "partials_kernel" in r["Name"]]
    dom = max((r for r in ours if "fused_kernel" in r["Name"]), key=lambda r: float(r["TotalDurationNs"]))
    dom_name = dom["Name"]
    is_dom = lambda name: name == dom_name
    copy_name = "__amd_rocclr_copyBuffer"
    fetch_kib, nf = counter_per_dispatch(one(f"{out}/fetch/run_counter_collection.csv"), is_dom)
    write_kib, nw = counter_per_dispatch(one(f"{out}/write/run_counter_collection.csv"), is_dom)
    cf_kib, _ = counter_per_dispatch(one(f"{out}/cfetch/run_counter_collection.csv"), lambda n: n == copy_name)
    cw_kib, _ = counter_per_dispatch(one(f"{out}/cwrite/run_counter_collection.csv"), lambda n: n == copy_name)
    copy_bytes = 4 << 30
    f_fetch = cf_kib * 1024 / copy_bytes
    f_write = cw_kib * 1024 / copy_bytes
    fetch_b = fetch_kib * 1024 / f_fetch
    write_b = write_kib * 1024 / f_write
    n = w.n_total
    # every fused launch of the timed command, per step (the dominant kernel
    # runs once per step): both passes of a two-pass step
    is_fused = lambda name: "fused_kernel" in name
    fetch_rows = list(csv.DictReader(open(one(f"{out}/fetch/run_counter_collection.csv"))))
    write_rows = list(csv.DictReader(open(one(f"{out}/write/run_counter_collection.csv"))))
    step_b = (sum(float(r["Counter_Value"]) for r in fetch_rows if is_fused(r["Kernel_Name"])) / nf * 1024 / f_fetch
              + sum(float(r["Counter_Value"]) for r in write_rows if is_fused(r["Kernel_Name"])) / nw * 1024 / f_write)
    alg_step = (2 * w.M + (34 if w.two_pass else 26)) * n
    # bytes of the dominant kernel by the traffic model: single pass 2M+26, or the
    # fold pass (2M+4) / update pass (30) of a two-pass step
    if not w.two_pass:
        alg = (2 * w.M + 26) * n
    elif "(zero::Mode)1" in dom_name:
        alg = (2 * w.M + 4) * n
    else:
        alg = 30 * n
    avg_us = float(dom["AverageNs"]) / 1e3
    achieved = alg / (avg_us * 1e-6) / 1e9
    kshort = dom_name.split("(zero::PlanHeader")[0].replace("void zero::(anonymous namespace)::", "")
    kfile = kshort.replace("<(zero::Mode)", "_mode").replace(", ", "_").replace(">", "").replace("<", "_")
    os.makedirs(profiles, exist_ok=True)
    md = os.path.join(profiles, f"{kfile}_{TAGS[a.workload]}.md")
    with open(md, "w") as f:
        f.write(f"# {kshort} on {w.name}\n\n")
        f.write("Commands (repository root, MI355X, ROCm 7.2):\n\n")
        for k, c in cmds.items():
            f.write(f"    {' '.join(c)}\n")
        f.write("\nKernel stats (rocprofv3 --kernel-trace --stats), kernels of the step:\n\n")
        f.write("| kernel | calls | average us | min us | max us |\n|---|---|---|---|---|\n")
        for r in ours:
            nm = r["Name"].replace("void zero::(anonymous namespace)::", "").replace("zero::(anonymous namespace)::", "")
            nm = re.split(r"\((?:zero::PlanHeader|zero::Partial)", nm)[0]
            f.write(f"| {nm} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | {float(r['MinNs'])/1e3:.2f} | "
                    f"{float(r['MaxNs'])/1e3:.2f} |\n")
        f.write(f"\nDominant kernel: `{kshort}`, average {avg_us:.2f} us over {dom['Calls']} launches.\n")
        f.write(f"Algorithmic bytes per launch: {alg:,.0f} ({alg / n:.0f} B x {n:,} parameters) -> "
                f"{achieved:.1f} GB/s = {achieved / 8000:.4f} of 8000 GB/s.\n\n")
        f.write("HBM counters per launch (average over dispatches), calibrated on a 4 GiB device copy:\n\n")
        f.write(f"- copy calibration: FETCH_SIZE {cf_kib:,.1f} KiB and WRITE_SIZE {cw_kib:,.1f} KiB for "
                f"{copy_bytes:,} B each -> factors {f_fetch:.4f} (read), {f_write:.4f} (write)\n")
        f.write(f"- FETCH_SIZE {fetch_kib:,.1f} KiB over {nf} dispatches -> {fetch_b:,.0f} B read\n")
        f.write(f"- WRITE_SIZE {write_kib:,.1f} KiB over {nw} dispatches -> {write_b:,.0f} B written\n")
        f.write(f"- traffic {fetch_b + write_b:,.0f} B per launch = {(fetch_b + write_b) / alg:.4f} x the "
                f"algorithmic bytes\n")
        f.write(f"- every fused launch of a step together: {step_b:,.0f} B per step = {step_b / alg_step:.4f} x "
                f"the step's algorithmic bytes ({alg_step / n:.0f} B x {n:,})\n")
        f.write(f"\nLibrary source hash (kernels and host planner, sha256[:16]): {src_hash()}\n")
    tf_path = os.path.join(profiles, "traffic.json")
    tf = json.load(open(tf_path)) if os.path.exists(tf_path) else {}
    tf[str(a.workload)] = {"kernel": kshort, "kernel_source_sha256_16": src_hash(),
                           "bytes_per_launch": round(fetch_b + write_b), "read_bytes": round(fetch_b),
                           "bytes_per_step": round(step_b), "algorithmic_bytes_per_step": alg_step,
                           "write_bytes": round(write_b), "algorithmic_bytes": alg,
                           "rocprof_avg_us": round(avg_us, 2), "fetch_factor": round(f_fetch, 5),
                           "write_factor": round(f_write, 5), "summary": os.path.join("profiles", os.path.basename(md))}
    json.dump(tf, open(tf_path, "w"), indent=1, sort_keys=True)
    print(open(md).read())


def main_zero2(a):
    """The ZeRO-2 leg: every bucket reduce (Mode::Acc launches, one per bucket
    and step) and the update (one Mode::PassB launch per step), aggregated per
    step; the dominant phase gets the counter-measured traffic."""
    sys.path.insert(0, ROOT)
    from synth.workloads import workload, zero2_buckets
    wi = 3 if a.workload == 2 else a.workload
    w = workload(wi)
    nb = len(zero2_buckets(w))
    out = os.path.join(a.out, f"w{wi}_zero2" + ("_fused" if a.fused_final else ""))
    os.chdir(ROOT)
    os.makedirs(out, exist_ok=True)
    warm = 2
    fused = a.fused_final
    bench = ["python", "-u", "bench.py", "--zero2", "--workload", str(wi), "--cpu-sample", "0", "--steps",
             str(a.steps), "--warmup", str(warm)] + (["--fused-final"] if fused else [])
    calib = ["python", "-u", "bench.py", "--calib-copy", "--steps", "3"]
    rp = "rocprofv3"
    cmds = {
        "trace": [rp, "--kernel-trace", "--stats", "--output-format", "csv", "-d", f"{out}/trace", "-o", "run",
                  "--"] + bench,
        "fetch": [rp, "--pmc", "FETCH_SIZE", "--output-format", "csv", "-d", f"{out}/fetch", "-o", "run", "--"] + bench,
        "write": [rp, "--pmc", "WRITE_SIZE", "--output-format", "csv", "-d", f"{out}/write", "-o", "run", "--"] + bench,
        "cfetch": [rp, "--pmc", "FETCH_SIZE", "--output-format", "csv", "-d", f"{out}/cfetch", "-o", "run", "--"] + calib,
        "cwrite": [rp, "--pmc", "WRITE_SIZE", "--output-format", "csv", "-d", f"{out}/cwrite", "-o", "run", "--"] + calib,
    }
    if not a.summarize_only:
        for k, c in cmds.items():
            run(c, f"{out}/{k}.log")
    steps = a.steps + warm
    stats = list(csv.DictReader(open(one(f"{out}/trace/run_kernel_stats.csv"))))
    if fused:
        groups = {"fused final passes": "(zero::Mode)4"}
    else:
        groups = {"bucket reduces": "(zero::Mode)3", "update": "(zero::Mode)2"}
    n = w.n_total
    alg = {"bucket reduces": (2 * w.M + 4) * n, "update": 30 * n, "fused final passes": (2 * w.M + 26) * n}
    # The bucket reduces run on two streams and overlap, so a phase's time
    # per step is its wall span in the kernel trace (first start to last end
    # of its dispatches within the step), not the sum of kernel durations.
    trace = sorted(csv.DictReader(open(one(f"{out}/trace/run_kernel_trace.csv"))),
                   key=lambda r: int(r["Start_Timestamp"]))
    spans = {g: [] for g in groups}
    cur = []
    for r in trace:
        nm = r["Kernel_Name"]
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        if fused:
            # a step: the final passes of every bucket, then the record (bucket_finalize_kernel)
            if "bucket_finalize_kernel" in nm:
                if cur:
                    spans["fused final passes"].append(max(e for _, e in cur) - min(b for b, _ in cur))
                cur = []
            elif "fused_kernel" in nm and groups["fused final passes"] in nm:
                cur.append((t0, t1))
            continue
        if "fused_kernel" not in nm:
            continue
        if groups["update"] in nm:
            if cur:
                spans["bucket reduces"].append(max(e for _, e in cur) - min(b for b, _ in cur))
            spans["update"].append(t1 - t0)
            cur = []
        elif groups["bucket reduces"] in nm:
            cur.append((t0, t1))
    per = {}
    for g, tag in groups.items():
        rows = [r for r in stats if "fused_kernel" in r["Name"] and tag in r["Name"]]
        sp = spans[g][warm:] if len(spans[g]) > warm else spans[g]
        per[g] = dict(rows=rows, ns=sum(sp) / max(len(sp), 1), calls=sum(int(r["Calls"]) for r in rows) / steps)
    dom = max(per, key=lambda g: per[g]["ns"])
    pred = lambda name, tag=groups[dom]: "fused_kernel" in name and tag in name
    copy_name = "__amd_rocclr_copyBuffer"

    def counter_total(path, kernel_pred):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if kernel_pred(r["Kernel_Name"])]
        if not vals:
            sys.exit(f"no matching dispatch in {path}")
        return sum(vals), len(vals)

    fetch_kib, nf = counter_total(one(f"{out}/fetch/run_counter_collection.csv"), pred)
    write_kib, nw = counter_total(one(f"{out}/write/run_counter_collection.csv"), pred)
    cf_kib, _ = counter_per_dispatch(one(f"{out}/cfetch/run_counter_collection.csv"), lambda nm: nm == copy_name)
    cw_kib, _ = counter_per_dispatch(one(f"{out}/cwrite/run_counter_collection.csv"), lambda nm: nm == copy_name)
    copy_bytes = 4 << 30
    f_fetch = cf_kib * 1024 / copy_bytes
    f_write = cw_kib * 1024 / copy_bytes
    fetch_b = fetch_kib * 1024 / f_fetch / steps
    write_b = write_kib * 1024 / f_write / steps
    os.makedirs(a.profiles_dir, exist_ok=True)
    md = os.path.join(a.profiles_dir, (f"zero2_fused_final_pass_{TAGS[wi]}.md" if fused else
                                       f"zero2_bucket_reduce_and_update_{TAGS[wi]}.md"))
    with open(md, "w") as f:
        if fused:
            f.write(f"# ZeRO-2 streaming step on {w.name}: {nb} fused final passes (one micro-batch, folded and "
                    f"applied in one pass) + the record per step\n\n")
        else:
            f.write(f"# ZeRO-2 streaming step on {w.name}: {nb} bucket reduces + one update per step\n\n")
        f.write("Commands (repository root, MI355X, ROCm 7.2):\n\n")
        for k, c in cmds.items():
            f.write(f"    {' '.join(c)}\n")
        f.write(f"\nKernel stats (rocprofv3 --kernel-trace --stats) over {steps} steps ({warm} warm-up):\n\n")
        f.write("| kernel | calls | average us | min us | max us | total us |\n|---|---|---|---|---|---|\n")
        for g in groups:
            for r in per[g]["rows"]:
                nm = r["Name"].replace("void zero::(anonymous namespace)::", "")
                nm = re.split(r"\((?:zero::PlanHeader|zero::Partial)", nm)[0]
                f.write(f"| {nm} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | {float(r['MinNs'])/1e3:.2f} | "
                        f"{float(r['MaxNs'])/1e3:.2f} | {float(r['TotalDurationNs'])/1e3:.1f} |\n")
        f.write("\nPer step (a phase's wall span in the kernel trace, after the warm-up steps):\n\n"
                "| phase | launches | wall us | algorithmic bytes | GB/s |\n|---|---|---|---|---|\n")
        for g in groups:
            f.write(f"| {g} | {per[g]['calls']:.0f} | {per[g]['ns'] / 1e3:.1f} | {alg[g]:,} | "
                    f"{alg[g] / per[g]['ns']:.1f} |\n")
        f.write(f"\nDominant phase: {dom} ({alg[dom] / n:.0f} B per parameter x {n:,} parameters).\n\n")
        f.write("HBM counters of the dominant phase per step, calibrated on a 4 GiB device copy:\n\n")
        f.write(f"- copy calibration: factors {f_fetch:.4f} (FETCH_SIZE), {f_write:.4f} (WRITE_SIZE)\n")
        f.write(f"- FETCH_SIZE over {nf} dispatches -> {fetch_b:,.0f} B read per step\n")
        f.write(f"- WRITE_SIZE over {nw} dispatches -> {write_b:,.0f} B written per step\n")
        f.write(f"- traffic {fetch_b + write_b:,.0f} B per step = {(fetch_b + write_b) / alg[dom]:.4f} x the "
                f"algorithmic bytes\n")
        f.write(f"\nLibrary source hash (kernels and host planner, sha256[:16]): {src_hash()}\n")
    tf_path = os.path.join(a.profiles_dir, "traffic.json")
    tf = json.load(open(tf_path)) if os.path.exists(tf_path) else {}
    tf[f"{wi}_zero2_K1" + ("_fused" if fused else "")] = {"kernel": dom, "kernel_source_sha256_16": src_hash(),
                            "bytes_per_launch": round(fetch_b + write_b), "read_bytes": round(fetch_b),
                            "write_bytes": round(write_b), "algorithmic_bytes": alg[dom],
                            "rocprof_us_per_step": round(per[dom]["ns"] / 1e3, 2), "fetch_factor": round(f_fetch, 5),
                            "write_factor": round(f_write, 5), "summary": os.path.join("profiles", os.path.basename(md))}
    json.dump(tf, open(tf_path, "w"), indent=1, sort_keys=True)
    print(open(md).read())


QUEUE_PASSES = [
    ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_LEVEL_sum"],
    ["TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum", "TCC_BUSY_sum", "GRBM_GUI_ACTIVE"],
]


def main_queues(a):
    """Why a kernel's bytes move at the rate they do: per fused kernel of the
    bench command, the read and write requests that leave the L2 for the
    fabric, their average latency there (requests in flight summed over
    cycles, over requests), and the share of the L2's busy cycles stalled for
    DRAM credits. Two counter passes (at most four TCC counters each)."""
    sys.path.insert(0, ROOT)
    from synth.workloads import workload
    w = workload(a.workload)
    out = os.path.join(a.out, f"w{a.workload}_queues")
    os.chdir(ROOT)
    os.makedirs(out, exist_ok=True)
    bench = ["python", "-u", "bench.py", "--workload", str(a.workload), "--cpu-sample", "0", "--steps",
             str(a.steps), "--warmup", "2", "--no-skipped-leg"]
    cmds = {f"pass{i}": ["rocprofv3", "--pmc", *p, "--output-format", "csv", "-d", f"{out}/pass{i}", "-o", "run",
                         "--"] + bench for i, p in enumerate(QUEUE_PASSES)}
    if not a.summarize_only:
        for k, c in cmds.items():
            run(c, f"{out}/{k}.log")
    per = {}
    for k in cmds:
        for r in csv.DictReader(open(one(f"{out}/{k}/run_counter_collection.csv"))):
            nm = r["Kernel_Name"]
            if "fused_kernel" not in nm:
                continue
            nm = nm.split("(zero::PlanHeader")[0].replace("void zero::(anonymous namespace)::", "")
            per.setdefault(nm, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    os.makedirs(a.profiles_dir, exist_ok=True)
    md = os.path.join(a.profiles_dir, f"hbm_queues_{TAGS[a.workload]}.md")
    with open(md, "w") as f:
        f.write(f"# HBM request queues of the step's kernels on {w.name}\n\n")
        f.write("Commands (repository root, MI355X, ROCm 7.2):\n\n")
        for c in cmds.values():
            f.write(f"    {' '.join(c)}\n")
        f.write("\nPer kernel, averaged over its dispatches. Requests are those the L2 sends to the fabric (reads in "
                "128 B, writes in 64 B); latency is requests in flight summed over cycles, divided by requests "
                "(TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ); a credit stall is a cycle the L2 could not send for "
                "want of DRAM credits, as a share of its busy cycles.\n\n")
        f.write("| kernel | read requests | write requests | read latency (cycles) | write latency (cycles) | "
                "read credit stalls | write credit stalls |\n|---|---|---|---|---|---|---|\n")
        for nm, c in per.items():
            m = {k: sum(v) / len(v) for k, v in c.items()}
            rd, wr, busy = m["TCC_EA0_RDREQ_sum"], m["TCC_EA0_WRREQ_sum"], m["TCC_BUSY_sum"]
            f.write(f"| {nm} | {rd:,.0f} | {wr:,.0f} | {m['TCC_EA0_RDREQ_LEVEL_sum'] / rd:,.0f} | "
                    f"{(m['TCC_EA0_WRREQ_LEVEL_sum'] / wr if wr else 0):,.0f} | "
                    f"{m['TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum'] / busy:.3f} | "
                    f"{m['TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum'] / busy:.3f} |\n")
        f.write(f"\nLibrary source hash (kernels and host planner, sha256[:16]): {src_hash()}\n")
    print(open(md).read())


if __name__ == "__main__":
    main()
