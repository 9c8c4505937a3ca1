"""Summaries of rocprofv3 runs of bench.py, written under profiles/.

Each summary names the command that produced its numbers (a rocprofv3 run of bench.py, run from
/tmp with the repository root in $R) and is regenerated from that run's CSV output:

  python bench_profiles.py trace    --workload W --dir OUT [--log BENCH_LOG] [--plain BENCH_JSON]
      kernel statistics of `rocprofv3 --kernel-trace --stats` -> profiles/W_kernel_trace.md
  python bench_profiles.py traffic  --workload W --fetch OUT1 --write OUT2 --log FETCH_LOG
      HBM bytes per launch from two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
      `bench.py --calibrate`, scaled by what the counters read for the 1 GiB copies that
      --calibrate makes -> profiles/W_pmc_traffic.md and profiles/W_score_traffic.json (the record
      bench.py reports as roofline.traffic while the kernel's sources are unchanged)
  python bench_profiles.py counters --out NAME DIR...
      utilisation counters of `--pmc` runs (three passes, counter sets below) per (workload,
      kernel) -> profiles/NAME.md
  python bench_profiles.py parity --record FILE
      the per-test parity records that tests/gpu_harness.py appends to $SKV_PARITY_RECORD during
      `pytest -m gpu` (units compared, certified near-ties, largest error as a fraction of the
      tolerance) -> profiles/parity_record.md

Counter arithmetic (MI355X: 256 CUs in 8 XCDs, 4 SIMDs per CU). GRBM_GUI_ACTIVE counts GPU-busy
cycles on each XCD and sums them, so the kernel's busy cycles are GRBM_GUI_ACTIVE / 8.
  VALUBusy     = SQ_ACTIVE_INST_VALU / (256 * busy)        (VALU instruction-issue cycles per CU)
  SALUBusy     = SQ_INST_CYCLES_SALU / (256 * busy)
  ScalarActive = SQ_ACTIVE_INST_SCA  / (256 * busy)        (scalar ALU + scalar memory issue)
  LDSActive    = SQ_ACTIVE_INST_LDS  / (256 * busy),  LDSBankConflict = SQ_LDS_BANK_CONFLICT / (256 * busy)
  MFMABusy     = SQ_VALU_MFMA_BUSY_CYCLES / (4 * 256 * busy)
  TABusy       = TA_TA_BUSY_sum / (256 * busy)             (texture addresser: the vector memory unit)
  TA data stall= TCP_TCP_TA_DATA_STALL_CYCLES_sum / (256 * busy)
  WaitAny      = SQ_WAIT_ANY / SQ_WAVE_CYCLES              (share of wave time waiting on any counter)
  L2 hit       = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CU, SIMD, XCD = 256, 4, 8

PASSES = {
    "A": "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INST_CYCLES_SALU SQ_WAIT_INST_ANY SQ_WAIT_ANY "
         "GRBM_GUI_ACTIVE",
    "B": "SQ_INSTS_VALU SQ_INSTS_SMEM SQ_INST_CYCLES_SMEM SQ_ACTIVE_INST_SCA SQ_INSTS_VALU_FMA_F64 SQ_INSTS_LDS "
         "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE",
    "C": "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_MFMA SQ_INSTS_VMEM_RD TA_TA_BUSY_sum "
         "TCP_TCP_TA_DATA_STALL_CYCLES_sum TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
}

# the source files a scoring kernel's HBM traffic depends on: its own file, the shared device
# helpers and launch declarations, the metadata layout it reads (written by meta.hip, sized by the
# binding), the host planner, the workload draw
TRAFFIC_SOURCES = ["sparse_kv_cache_build_amd/csrc/common.hpp", "sparse_kv_cache_build_amd/csrc/launch.hpp",
                   "sparse_kv_cache_build_amd/csrc/meta.hip", "sparse_kv_cache_build_amd/csrc/abi.cpp",
                   "sparse_kv_cache_build_amd/_binding.py", "workloads/__init__.py"]


def short(name: str) -> str:
    """Kernel name without 'void', the namespace and the argument list."""
    n = re.sub(r"^void ", "", name).replace("(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in n:   # cut at the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            break
        out.append(ch)
    return "".join(out).replace("skv::", "")


def base_name(name: str) -> str:
    return short(name).split("<")[0]


def bench_json(path: str):
    """The JSON line bench.py printed (stdout, possibly mixed with its log lines)."""
    if not path or not os.path.exists(path):
        return None
    for line in open(path):
        line = line.strip()
        if line.startswith('{"metric"'):
            return json.loads(line)
    return None


def bench_step_line(path: str):
    if not path or not os.path.exists(path):
        return None
    for line in open(path):
        if "us/step" in line and line.startswith("[bench]"):
            return line.strip()
    return None


def describe(workload: str) -> str:
    sys.path.insert(0, ROOT)
    import workloads as W
    c = W.CONFIGS[workload]
    ctx = f"L={c['L']}" if "L" in c else f"lengths {c['Lmin']}..{c['Lmax']}"
    sel = {"topk": f"top-{c.get('k')} pages", "budget": f"{c.get('pct')} % page budget",
           "thresh": f"Gaussian threshold (alpha {c.get('sel_alpha')}, Delta {c.get('delta')})",
           "token_topk": f"top-{c.get('k')} tokens per KV head"}[c["policy"]]
    key = {"box": "box page bound", "gauss": "Gaussian page scores", "proj": f"rank-{c.get('proj_rank')} projected keys",
           "pool": f"pooled keys (blocks of {c.get('pool_block')})",
           "lsh": f"soft-LSH ({c.get('lsh_tables')} tables x {c.get('lsh_bits')} bits)"}[c["score"]]
    attn = "softmax" if c["alphas"][0] == 1.0 else f"{c['alphas'][0]}-entmax"
    return (f"{workload} decode step (B={c['B']}, {c['Hq']} q / {c['Hkv']} KV heads, d={c['d']}, {ctx}, S={c['S']}, "
            f"{c['dtype']}, {key}, {sel}, {attn})")


def cmd_trace(a):
    rows = list(csv.DictReader(open(glob.glob(os.path.join(a.dir, "*kernel_stats.csv"))[0])))
    rows = [r for r in rows if "skv::" in r["Name"]]
    rows.sort(key=lambda r: -float(r["AverageNs"]) * (0 if base_name(r["Name"]).startswith("meta_") else 1))
    js = bench_json(a.log)
    step_kernels = [r for r in rows if not base_name(r["Name"]).startswith("meta_")]
    total = sum(float(r["AverageNs"]) for r in step_kernels) / 1e3
    out = [f"# Kernel trace: {describe(a.workload)}", "",
           "Command (MI355X, one GPU; repository root in $R):", "",
           f"    cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o bench -- "
           f"python3 $R/bench.py --workload {a.workload} --steps {a.steps} --warmup {a.warmup} --no-cpu", "",
           f"rocprofv3 kernel statistics of the library's kernels ({a.steps} timed + {a.warmup} warm-up + 1 "
           "initial step; meta_* kernels build the page metadata, outside the step):", "",
           "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    out += ["", f"Kernel time of one step (sum of the per-step kernels' averages): {total:.2f} us."]
    step = bench_step_line(a.log)
    if step:
        out.append(f"bench.py in the same run: {step[len('[bench] '):]}.")
    if js:
        rf = js["roofline"]
        dom = [r for r in rows if base_name(r["Name"]) == rf["kernel"]]
        if dom:
            out.append(f"HIP events the library records around each {rf['kernel']} launch: {rf['avg_us']} us "
                       f"against rocprofv3's {float(dom[0]['AverageNs']) / 1e3:.2f} us (under kernel tracing every "
                       "dispatch carries the profiler's completion handling, which the events see).")
    plain = bench_json(a.plain)
    if plain:
        rf = plain["roofline"]
        out.append(f"Without the profiler (`python3 $R/bench.py --workload {a.workload} --no-cpu`, "
                   f"{plain['steps']} steps, same box): {plain['ms_per_step'] * 1e3:.1f} us per step "
                   f"({plain['value']} steps/s, {plain['config']['pct_of_peak']} % of 8 TB/s); {rf['kernel']} "
                   f"{rf['avg_us']} us by the library's events, {rf['achieved']} GB/s = {rf['frac']} of peak.")
    path = os.path.join(PROFILES, f"{a.workload}_kernel_trace.md")
    open(path, "w").write("\n".join(out) + "\n")
    print("wrote", path)


def counter_rows(d: str):
    f = glob.glob(os.path.join(d, "*counter_collection.csv"))
    return list(csv.DictReader(open(f[0]))) if f else []


def copy_calibration(rows, counter):
    """Mean counter value (KiB) of the 1 GiB copies: the largest dispatches of the copy kernel."""
    vals = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter]
    vals.sort(reverse=True)
    top = vals[:3]
    if not top:
        raise SystemExit(f"no 1 GiB copy found for {counter} (run bench.py with --calibrate)")
    return sum(top) / len(top)


def per_launch(rows, counter):
    acc = collections.defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == counter and "skv::" in r["Kernel_Name"]:
            acc[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def sources_for(kernel: str):
    own = "sparse_kv_cache_build_amd/csrc/" + ("attn.hip" if kernel.startswith("attn_") else "score.hip")
    return [own] + TRAFFIC_SOURCES


def sha256_of(sources):
    h = hashlib.sha256()
    for rel in sources:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()


def cmd_traffic(a):
    fr, wr = counter_rows(a.fetch), counter_rows(a.write)
    one_gib_kib = float(1 << 20)
    ff = one_gib_kib / copy_calibration(fr, "FETCH_SIZE")
    wf = one_gib_kib / copy_calibration(wr, "WRITE_SIZE")
    fk, wk = per_launch(fr, "FETCH_SIZE"), per_launch(wr, "WRITE_SIZE")
    js = bench_json(a.log)
    if not js:
        raise SystemExit("the fetch run's log holds no bench.py JSON line")
    dom = js["roofline"]["kernel"]
    names = sorted(fk, key=lambda k: -fk[k])
    out = [f"# HBM traffic (PMC): {describe(a.workload)}", "",
           "Commands (two separate runs, one counter each; repository root in $R):", "",
           f"    cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out> -o fetch -- python3 $R/bench.py "
           f"--workload {a.workload} --steps 3 --warmup 1 --no-cpu --calibrate",
           f"    cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out> -o write -- python3 $R/bench.py "
           f"--workload {a.workload} --steps 3 --warmup 1 --no-cpu --calibrate", "",
           "`--calibrate` copies a 1 GiB buffer three times after the timed steps (torch copy, "
           "`__amd_rocclr_copyBuffer`): each copy reads and writes exactly 1,048,576 KiB.", "",
           "| counter | 1 GiB copy reads as (KiB, mean of 3) | scale factor |", "|---|---|---|",
           f"| FETCH_SIZE | {one_gib_kib / ff:.1f} | {ff:.4f} |", f"| WRITE_SIZE | {one_gib_kib / wf:.1f} | {wf:.4f} |", "",
           "Per launch (mean over the launches of the run), scaled:", "",
           "| kernel | FETCH KiB (raw) | fetched MB | WRITE KiB (raw) | written MB |", "|---|---|---|---|---|"]
    for k in names:
        w = wk.get(k, 0.0)
        out.append(f"| {k} | {fk[k]:.1f} | {fk[k] * ff * 1024 / 1e6:.1f} | {w:.1f} | {w * wf * 1024 / 1e6:.2f} |")
    dk = [k for k in names if k.split("<")[0] == dom]
    if not dk:
        raise SystemExit(f"dominant kernel {dom} not among the counted kernels")
    fb, wb = fk[dk[0]] * ff * 1024, wk.get(dk[0], 0.0) * wf * 1024
    alg = js["roofline"]["bytes_per_launch"]
    out += ["", f"{dk[0]}: {(fb + wb) / 1e6:.1f} MB of HBM traffic per launch against {alg / 1e6:.1f} MB algorithmic "
                f"(bench.py bytes_per_launch): ratio {(fb + wb) / alg:.4f}."]
    path = os.path.join(PROFILES, f"{a.workload}_pmc_traffic.md")
    open(path, "w").write("\n".join(out) + "\n")
    srcs = sources_for(dom)
    rec = {"kernel": dom, "workload": a.workload, "sources": srcs, "sources_sha256": sha256_of(srcs),
           "fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb, "fetch_factor": ff, "write_factor": wf,
           "algorithmic_bytes": alg}
    jpath = os.path.join(PROFILES, f"{a.workload}_score_traffic.json")
    json.dump(rec, open(jpath, "w"), indent=1)
    print("wrote", path, jpath)


def cmd_counters(a):
    res = collections.defaultdict(lambda: collections.defaultdict(dict))   # (wl, kernel) -> counter -> {dispatch: v}
    dur = collections.defaultdict(list)
    for d in a.dirs:
        m = re.match(r".*ctr_(.+)_([ABC])/?$", d.rstrip("/"))
        if not m:
            raise SystemExit(f"directory {d} is not named ctr_<workload>_<pass>")
        wl = m.group(1)
        for r in counter_rows(d):
            key = (wl, short(r["Kernel_Name"]))
            if a.by_grid:   # one row per launch configuration (workgroups of the grid)
                key = (wl, f"{key[1]}, {int(r['Grid_Size']) // int(r['Workgroup_Size'])} WG")
            res[key][r["Counter_Name"]][(d, r["Dispatch_Id"])] = float(r["Counter_Value"])
            if m.group(2) == "A" and r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                dur[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [f"# Utilisation counters of {a.title}", "",
           "Commands (three passes per workload, one counter set each, repository root in $R"
           + ("; `--sets 1` keeps one buffer set):" if "--sets 1" in a.bench_args else "):"), ""]
    for p, ctrs in PASSES.items():
        out.append(f"    cd /tmp && rocprofv3 --pmc {ctrs} --kernel-include-regex '<kernels>' --output-format csv "
                   f"-d <out> -o ctr -- python3 $R/bench.py {a.bench_args}   # pass {p}")
    out += ["", f"Kernels: `{a.regex}`.", "",
            "Per kernel and workload, means over its dispatches (busy = GRBM_GUI_ACTIVE / 8 cycles; "
            "formulas in bench_profiles.py):", "",
            "| workload | kernel | us (pass A) | VALUBusy % | SALUBusy % | ScalarActive % | LDSActive % | "
            "LDSBankConflict % | MFMABusy % | TABusy % | TA data stall % | WaitAny % | L2 hit % | VALU inst/wave | "
            "SMEM inst/wave | VMEM rd/wave | FMA_F64/wave | LDS inst/wave | MFMA/wave |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for (wl, k), ctr in sorted(res.items()):
        avg = {n: sum(v.values()) / len(v) for n, v in ctr.items()}
        busy = avg.get("GRBM_GUI_ACTIVE", 0.0) / XCD

        def pct(n, div=1):
            return f"{100 * avg[n] / (CU * div) / busy:.1f}" if busy and n in avg else "-"

        def per_wave(n):
            return f"{avg[n] / avg['SQ_WAVES']:.0f}" if n in avg and avg.get("SQ_WAVES") else "-"
        wait = f"{100 * avg['SQ_WAIT_ANY'] / avg['SQ_WAVE_CYCLES']:.1f}" if avg.get("SQ_WAVE_CYCLES") else "-"
        hit = (f"{100 * avg['TCC_HIT_sum'] / (avg['TCC_HIT_sum'] + avg['TCC_MISS_sum']):.1f}"
               if "TCC_HIT_sum" in avg and avg["TCC_HIT_sum"] + avg.get("TCC_MISS_sum", 0) else "-")
        us = f"{sum(dur[(wl, k)]) / len(dur[(wl, k)]):.1f}" if dur[(wl, k)] else "-"
        out.append(f"| {wl} | {k} | {us} | {pct('SQ_ACTIVE_INST_VALU')} | {pct('SQ_INST_CYCLES_SALU')} | "
                   f"{pct('SQ_ACTIVE_INST_SCA')} | {pct('SQ_ACTIVE_INST_LDS')} | {pct('SQ_LDS_BANK_CONFLICT')} | "
                   f"{pct('SQ_VALU_MFMA_BUSY_CYCLES', SIMD)} | {pct('TA_TA_BUSY_sum')} | "
                   f"{pct('TCP_TCP_TA_DATA_STALL_CYCLES_sum')} | {wait} | {hit} | {per_wave('SQ_INSTS_VALU')} | "
                   f"{per_wave('SQ_INSTS_SMEM')} | {per_wave('SQ_INSTS_VMEM_RD')} | {per_wave('SQ_INSTS_VALU_FMA_F64')} | "
                   f"{per_wave('SQ_INSTS_LDS')} | {per_wave('SQ_INSTS_MFMA')} |")
    if a.notes:
        out += ["", open(a.notes).read().rstrip()]
    path = os.path.join(PROFILES, f"{a.out}.md")
    open(path, "w").write("\n".join(out) + "\n")
    print("wrote", path)


def cmd_parity(a):
    recs = [json.loads(l) for l in open(a.record) if l.strip()]
    units = sum(r.get("units", 0) for r in recs)
    ties = sum(r.get("near_ties", 0) for r in recs)
    checked = sum(r.get("tie_units_checked", 0) for r in recs)
    worst = max((r.get("max_err_over_tol", 0.0) for r in recs), default=0.0)
    out = ["# GPU parity record", "",
           "Command (MI355X, one GPU, repository root; the harness appends one JSON line per compared case):", "",
           "    SKV_PARITY_RECORD=<file> python -u -m pytest tests -m gpu -v -x --timeout 300 --timeout-method thread", "",
           f"{len(recs)} records, {units} units (sequence, KV head) compared against the oracle; certified near-ties "
           f"(selection decisions within the threshold tolerance, whose outputs are then checked against the oracle "
           f"run on the GPU's own selection): {ties}, units re-checked that way: {checked}; largest output error "
           f"{worst:.4f} of the tolerance |gpu - ref| <= 1e-3 + 2e-3 |ref|.", "",
           "| test | workload | B | max len | units | near-ties | max err / tol | other |", "|---|---|---|---|---|---|---|---|"]
    std = {"workload", "B", "Hq", "Hkv", "d", "S", "max_len", "seqs", "units", "near_ties", "tie_units_checked",
           "max_err_over_tol", "ties", "test"}
    for r in recs:
        other = ", ".join(f"{k}={v}" for k, v in r.items() if k not in std)
        out.append(f"| {r.get('test', '').replace('tests/', '')} | {r.get('workload', '')} | {r.get('B', '')} | "
                   f"{r.get('max_len', '')} | {r.get('units', '')} | {r.get('near_ties', '')} | "
                   f"{r.get('max_err_over_tol', '')} | {other} |")
    path = os.path.join(PROFILES, "parity_record.md")
    open(path, "w").write("\n".join(out) + "\n")
    print("wrote", path)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--workload", required=True)
    t.add_argument("--dir", required=True)
    t.add_argument("--log")
    t.add_argument("--plain", help="output of a bench.py run without the profiler")
    t.add_argument("--steps", type=int, default=20)
    t.add_argument("--warmup", type=int, default=3)
    f = sub.add_parser("traffic")
    f.add_argument("--workload", required=True)
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--log", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--out", required=True)
    c.add_argument("--regex", default="")
    c.add_argument("--notes", help="a text file appended to the summary")
    c.add_argument("--by-grid", action="store_true", help="one row per grid size of each kernel")
    c.add_argument("--title", default="the hot kernels")
    c.add_argument("--bench-args", default="--workload <W> --steps 3 --warmup 1 --no-cpu --sets 1",
                   help="the bench.py arguments of the profiled runs, as the summary states them")
    c.add_argument("dirs", nargs="+")
    r = sub.add_parser("parity")
    r.add_argument("--record", required=True)
    a = ap.parse_args()
    {"trace": cmd_trace, "traffic": cmd_traffic, "counters": cmd_counters, "parity": cmd_parity}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
