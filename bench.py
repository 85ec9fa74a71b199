#!/usr/bin/env python3
"""Throughput of the CLHA calibration hot path on one MI355X (gfx950).

One step calibrates one CLWS pair (two layers that share their routed experts):
  reset the pair's accumulators -> collect layer a -> collect layer b (route,
  bucket, Gram sums read straight from x) -> aggregate H_comb -> GPTQ of the pair's expert
  jobs (damping, factor of the inverse, column loop, lazy block updates, loss).
Inputs are seeded synthetic arrays, every pair's resident in HBM before the
timed region; steps cycle over the pairs.  Prints one JSON line.

Default workload: full depth (24 layers as 12 CLWS pairs; 64 routed experts
top-6 with a Zipf(1.1) router load plus 2 shared experts; d = 2048; 262,144
tokens per layer; gate and up 1408x2048 bf16 per expert, stacked into 66 jobs
of 2816x2048 = 132 matrices per pair; 2-bit, group 128, equal weighting).  The
default 12 timed steps are one pass over all 24 layers.  --workload selects
another shape sheet of gen.WORKLOADS (2 mid MoE block, 4 CLHA-MP, 5 drift
stress, whose steps cycle over the drift values t of one pair).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ID] [--pairs N]
                  [--no-cpu-baseline]

--down-proj measures the experts' second matrices of the mid MoE block instead:
one step resets the down_proj accumulators, collects both layers' SwiGLU
inputs h = bf16(silu(x Wg^T) * (x Wu^T)) and their Gram sums (routing taken
from the main context's collection of the same batch, done once before
timing), aggregates, and runs GPTQ on the 66 down_proj matrices (2048x1408).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "expert matrices calibrated/sec (Hessian+CLHA-GPTQ); SYRK % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 matrix peak
PEAK_FP32_TFLOPS = 157.3           # MI355X fp32 matrix peak
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E bandwidth
SYRK_SRC = os.path.join(ROOT, "gptq_calibration_moe_amd", "csrc", "syrk.hip")
DOWN_SRC = os.path.join(ROOT, "gptq_calibration_moe_amd", "csrc", "down.hip")
DOWN_TRAFFIC = os.path.join(ROOT, "profiles", "down_gemm_mid_moe_block_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=12)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--pairs", type=int, default=0,
                    help="keep only the first N pairs (drift values) resident; 0 = all of the workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=3, help="workload id of gen.WORKLOADS (default 3, full depth)")
    ap.add_argument("--copy-probe", type=int, metavar="BYTES", help="only copy BYTES on the device and exit")
    ap.add_argument("--down-proj", action="store_true", help="measure the down_proj calibration step instead")
    ap.add_argument("--act-order", action="store_true", help="GPTQ with activation order")
    ap.add_argument("--static-groups", action="store_true", help="GPTQ with static groups")
    ap.add_argument("--profile-commands", metavar="DIR", help="print the profiling command lines and exit")
    ap.add_argument("--summarize-profiles", metavar="DIR", help="write profiles/ summaries from DIR and exit")
    ap.add_argument("--summarize-options-profile", nargs=2, metavar=("DIR", "BENCH_JSON"),
                    help="write the options step's trace summary and bench line under profiles/ and exit")
    ap.add_argument("--summarize-down-profile", nargs=2, metavar=("DIR", "BENCH_JSON"),
                    help="write the down_proj profile summaries from DIR and the bench output file, and exit")
    ap.add_argument("--down-counter-commands", metavar="DIR",
                    help="print the down_proj GEMM's counter command lines and exit")
    ap.add_argument("--summarize-down-traffic", metavar="DIR",
                    help="write the down_proj GEMM's traffic record from DIR and exit")
    ap.add_argument("--experiment", choices=("drift", "sharpness"),
                    help="run a section-4 experiment on the drift-stress shapes and write its table")
    ap.add_argument("--out", help="JSON file of the experiment table (default under profiles/)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def syrk_source_hash():
    return hashlib.sha256(open(SYRK_SRC, "rb").read()).hexdigest()[:16]


def down_source_hash():
    return hashlib.sha256(open(DOWN_SRC, "rb").read()).hexdigest()[:16]


def cpu_baseline(wl, inp, w_host, budget_s=10.0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    routing and bucketing of all tokens of both layers, then, routed expert by
    routed expert until about budget_s seconds have passed, the expert's Gram
    sums in both layers, aggregation, GPTQ of its gate|up job and its loss."""
    import numpy as np
    import gen
    import oracle
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        blas = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            threads = max(blas)
    except Exception:
        pass
    t0 = time.perf_counter()
    topk = [oracle.route(inp["logits"][l], wl.top_k) for l in range(2)]
    done = 0
    for e in range(wl.n_routed):
        S, n = [], []
        for l in range(2):
            s_l, c_l = oracle.layer_hessians(inp["x"][l], topk[l], wl.n_routed, wl.n_shared, slots=[e])
            S.append(s_l[e])
            n.append(c_l[e])
        H, _ = oracle.aggregate(S, n, wl.alpha)
        wv = gen.weights_value(wl, w_host[e]).astype(np.float64)
        g = oracle.gptq(wv, H, wl.bits, wl.group, wl.damp, wl.block)
        oracle.loss(wv, g["wq"], H)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    mats = done * len(wl.mats)
    return {"value": round(mats / dt, 4), "unit": "matrices/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"oracle (fp64 NumPy) on routed experts 0..{done - 1} of the {wl.name} workload: "
                       f"routing and bucketing of all {wl.n_tokens} tokens of both layers, then per expert "
                       f"its Gram sums in both layers, aggregation, GPTQ of its {wl.job_rows}x{wl.d} "
                       f"gate|up job and the loss = {mats} matrices in {dt:.2f} s")}


# Profiling runs behind the committed summaries, on two resident pairs (the
# kernels and their shapes are those of every pair).  The counter runs read
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) in passes of their own; the
# copy probe moves a known number of bytes so that each counter can be scaled
# to bytes.  Two more passes read the matrix-core counters (MFMA busy cycles,
# MFMA operations by type) and the LDS counters (bank conflicts against LDS
# activity), each within one pass's counter limits.  `--profile-commands DIR`
# prints these lines; `--summarize-profiles DIR` turns their CSV output into
# the text summaries.
COPY_BYTES = 1 << 30
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_I8 "
                 "SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_INSTS_VALU_MFMA_MOPS_F64 GRBM_GUI_ACTIVE")
LDS_COUNTERS = "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_BUSY_CYCLES SQ_WAVE_CYCLES GRBM_GUI_ACTIVE"
_BENCH = "-- python3 bench.py --workload {wid} --pairs 2 --no-cpu-baseline"
PROFILE_RUNS = [
    ("trace", "timeout -k 10 600 rocprofv3 --kernel-trace --stats --output-format csv -d {dir}/trace -o run "
              + _BENCH + " --steps 3 --warmup 1"),
    ("fetch", "timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {dir}/fetch -o run "
              + _BENCH + " --steps 1 --warmup 1"),
    ("write", "timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {dir}/write -o run "
              + _BENCH + " --steps 1 --warmup 1"),
    ("mfma", "timeout -s KILL 300 rocprofv3 --pmc " + MFMA_COUNTERS + " --output-format csv -d {dir}/mfma -o run "
             + _BENCH + " --steps 1 --warmup 1"),
    ("lds", "timeout -s KILL 300 rocprofv3 --pmc " + LDS_COUNTERS + " --output-format csv -d {dir}/lds -o run "
            + _BENCH + " --steps 1 --warmup 1"),
    ("copy_fetch", "timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {dir}/copy_fetch -o run "
                   f"-- python3 bench.py --copy-probe {COPY_BYTES}"),
    ("copy_write", "timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {dir}/copy_write -o run "
                   f"-- python3 bench.py --copy-probe {COPY_BYTES}"),
]


def copy_probe(nbytes):
    """One plain device-to-device copy of nbytes (the counter scale reference)."""
    import torch
    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes}), flush=True)


def _csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _short(name):
    name = name.replace("void ", "")
    return name.split("(")[0] if name.startswith("clha::") else name[:70]


def _trace_lines(trace_dir, title, cmd, notes, steps=4, timed=3, setup_free=False):
    """Kernel-time table of a traced bench run (1 warm-up + `timed` steps).  When
    the run routes each step's two layers (2 routing launches per step), only the
    launches from the first timed step's routing on are counted, which leaves
    out the set-up (buffer fills, input copies) and the warm-up step, whose first
    touch of fresh device memory is slow.  Otherwise each kernel's first
    launches (1/steps of them) are taken as the warm-up's and left out; with
    setup_free, kernels launched fewer than `steps` times ran only in the set-up
    and are left out too."""
    trace = _csv(_find(trace_dir, "kernel_trace.csv"))
    routes = sorted(int(r["Start_Timestamp"]) for r in trace if "route_kernel" in r["Kernel_Name"])
    window = routes[2 * (steps - timed)] if len(routes) == 2 * steps else None
    by_name = {}
    for r in trace:
        if window is not None and int(r["Start_Timestamp"]) < window:
            continue
        by_name.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    stats = []
    for name, ds in by_name.items():
        ds.sort()
        if window is not None:
            keep = [t for _, t in ds]
        else:
            if setup_free and len(ds) < steps:
                continue
            if setup_free:
                ds = ds[len(ds) % steps:]          # launches before the steps
            keep = [t for _, t in ds[len(ds) // steps:]] if len(ds) >= steps else [t for _, t in ds]
        if keep:
            stats.append({"Name": name, "Calls": len(keep), "TotalDurationNs": sum(keep),
                          "AverageNs": sum(keep) / len(keep)})
    stats.sort(key=lambda r: -r["TotalDurationNs"])
    lines = [title, "", "Command (repository root):", "", f"    {cmd}", "",
             f"{steps} steps traced (1 warm-up + {timed} timed); the set-up's and the warm-up step's launches "
             f"are left out and per-step figures are totals / {timed}.", *notes, "",
             "| kernel | calls/step | ms/step | avg us/launch | % |", "|---|---:|---:|---:|---:|"]
    total = sum(float(r["TotalDurationNs"]) for r in stats)
    for r in stats:
        t = float(r["TotalDurationNs"])
        lines.append(f"| {_short(r['Name'])} | {int(r['Calls']) / timed:g} | {t / 1e6 / timed:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {100 * t / total:.1f} |")
    lines += ["", f"Sum of kernel time per step: {total / 1e6 / timed:.3f} ms", ""]
    return lines


def down_traffic():
    """HBM bytes per down_gemm launch from the committed counter record, while
    down.hip is the source it was taken on (else None)."""
    if not os.path.exists(DOWN_TRAFFIC):
        return None
    rec = json.load(open(DOWN_TRAFFIC))
    return rec.get("hbm_bytes_per_launch") if rec.get("down_source_sha256_16") == down_source_hash() else None


DOWN_COUNTER_RUNS = (
    ("fetch", "timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {dir}/fetch -o run "
              "-- python3 bench.py --down-proj --steps 1 --warmup 1"),
    ("write", "timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {dir}/write -o run "
              "-- python3 bench.py --down-proj --steps 1 --warmup 1"),
    ("copy_fetch", "timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {dir}/copy_fetch -o run "
                   "-- python3 bench.py --copy-probe 1073741824"),
    ("copy_write", "timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {dir}/copy_write -o run "
                   "-- python3 bench.py --copy-probe 1073741824"),
)


def summarize_down_traffic(d):
    """down_gemm's HBM traffic per launch from the counter passes of DOWN_COUNTER_RUNS in
    DIR (copy-probe scaled, as for the Gram sums), written to DOWN_TRAFFIC."""
    def per_kernel(sub, counter, key):
        tot, cnt = 0.0, 0
        for r in _csv(_find(os.path.join(d, sub), "counter_collection.csv")):
            if r["Counter_Name"] == counter and key in r["Kernel_Name"]:
                tot += float(r["Counter_Value"])
                cnt += 1
        return tot, cnt
    def copy_kib(sub, counter):
        v, c = per_kernel(sub, counter, "copyBuffer")
        return v / c if c else None
    f_scale = COPY_BYTES / 1024 / copy_kib("copy_fetch", "FETCH_SIZE")
    w_scale = COPY_BYTES / 1024 / copy_kib("copy_write", "WRITE_SIZE")
    fv, fc = per_kernel("fetch", "FETCH_SIZE", "down_gemm_kernel")
    wv, wc = per_kernel("write", "WRITE_SIZE", "down_gemm_kernel")
    rec = {"workload": "mid_moe_block_down_proj", "kernel": "down_gemm_kernel",
           "down_source_sha256_16": down_source_hash(),
           "fetch_kib_per_launch": fv / fc, "write_kib_per_launch": wv / wc,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_bytes_per_launch": (fv / fc * f_scale + wv / wc * w_scale) * 1024,
           "commands": [c.format(dir=d) for _, c in DOWN_COUNTER_RUNS]}
    json.dump(rec, open(DOWN_TRAFFIC, "w"), indent=1)
    print(json.dumps(rec))


DOWN_TRACE = ("timeout -k 10 400 rocprofv3 --kernel-trace --stats --output-format csv -d {dir}/trace -o run "
              "-- python3 bench.py --down-proj --steps 3 --warmup 1")


def summarize_down_profile(d, bench_json):
    """Writes the down_proj step's kernel-trace summary and bench line under profiles/."""
    lines = _trace_lines(os.path.join(d, "trace"),
                         "# Kernel time per step, down_proj calibration of the mid MoE block "
                         "(MI355X, rocprofv3 kernel trace)", DOWN_TRACE.format(dir=d),
                         ["The routing of the block's main context (and its Gram sums) runs once before the",
                          "steps; those launches are left out.  The factorisation and GPTQ overlap on",
                          "concurrent streams; wall-clock stage times are `stages_ms_per_step` in the bench line."],
                         setup_free=True)
    open(os.path.join(ROOT, "profiles", "down_proj_mid_moe_block_kernel_trace.md"), "w").write("\n".join(lines))
    line = open(bench_json).read().strip().splitlines()[-1]
    json.loads(line)
    out = ["# Bench line, down_proj calibration of the mid MoE block (MI355X)", "",
           "Command (repository root):", "", "    timeout -k 10 400 python3 -u bench.py --down-proj", "",
           "Output:", "", "```json", line, "```", ""]
    open(os.path.join(ROOT, "profiles", "bench_down_proj_mid_moe_block.md"), "w").write("\n".join(out))


OPTIONS_TRACE = ("timeout -k 10 400 rocprofv3 --kernel-trace --stats --output-format csv -d {dir}/trace -o run "
                 "-- python3 bench.py --workload 2 --act-order --static-groups --steps 3 --warmup 1 "
                 "--no-cpu-baseline")


def summarize_options_profile(d, bench_json):
    """Writes the kernel-trace summary and bench line of the step with GPTQ's
    activation-order and static-group options under profiles/."""
    lines = _trace_lines(os.path.join(d, "trace"),
                         "# Kernel time per step, mid_moe_block workload with GPTQ activation order and "
                         "static groups (MI355X, rocprofv3 kernel trace)", OPTIONS_TRACE.format(dir=d),
                         ["The factorisation runs as four Hessian groups on concurrent streams, overlapped with the",
                          "GPTQ kernels, so per-kernel times overlap in wall time; wall-clock stage times are",
                          "`stages_ms_per_step` in the bench line."])
    open(os.path.join(ROOT, "profiles", "gptq_options_mid_moe_block_kernel_trace.md"), "w").write("\n".join(lines))
    line = open(bench_json).read().strip().splitlines()[-1]
    json.loads(line)
    out = ["# Bench line, mid MoE block with GPTQ activation order and static groups (MI355X)", "",
           "Command (repository root):", "",
           "    timeout -k 10 400 python3 -u bench.py --workload 2 --act-order --static-groups --no-cpu-baseline", "",
           "Output:", "", "```json", line, "```", ""]
    open(os.path.join(ROOT, "profiles", "bench_gptq_options_mid_moe_block.md"), "w").write("\n".join(out))


def summarize_profiles(d, wid):
    """Writes, for workload `wid`, the kernel-trace summary, the per-kernel HBM
    traffic (counter values scaled by the copy probe), the matrix-core and LDS
    counter summaries under profiles/, and the Gram-sum traffic record that
    bench.py reports while syrk.hip is unchanged."""
    import gen
    name = gen.WORKLOADS[wid].name
    cmd = {k: c.format(dir=d, wid=wid) for k, c in PROFILE_RUNS}
    lines = _trace_lines(os.path.join(d, "trace"),
                         f"# Kernel time per step, {name} workload (MI355X, rocprofv3 kernel trace)",
                         cmd["trace"],
                         ["One step is one CLWS pair.  The factorisation runs as four Hessian groups on",
                          "concurrent streams, overlapped with the GPTQ kernels, so per-kernel times overlap in",
                          "wall time; wall-clock stage times are `stages_ms_per_step` in the bench line."])
    open(os.path.join(ROOT, "profiles", f"clha_step_{name}_kernel_trace.md"), "w").write("\n".join(lines))

    def per_kernel(sub, counter):
        acc = {}
        for r in _csv(_find(os.path.join(d, sub), "counter_collection.csv")):
            if r["Counter_Name"] != counter:
                continue
            k = _short(r["Kernel_Name"])
            v = acc.setdefault(k, [0.0, 0])
            v[0] += float(r["Counter_Value"])
            v[1] += 1
        return acc

    def copy_kib(sub, counter):
        vals = [float(v[0]) / v[1] for k, v in per_kernel(sub, counter).items() if "copyBuffer" in k]
        return max(vals)
    copy_kib_total = COPY_BYTES / 1024
    f_scale = copy_kib_total / copy_kib("copy_fetch", "FETCH_SIZE")
    w_scale = copy_kib_total / copy_kib("copy_write", "WRITE_SIZE")
    fetch, write = per_kernel("fetch", "FETCH_SIZE"), per_kernel("write", "WRITE_SIZE")
    lines = [f"# HBM traffic per launch, {name} workload (MI355X, rocprofv3 counters)", "",
             "Commands (repository root), one counter per run:", ""]
    lines += [f"    {cmd[k]}" for k in ("fetch", "write", "copy_fetch", "copy_write")]
    lines += ["", f"Scale: a {COPY_BYTES} B device copy reads FETCH_SIZE x {f_scale:.3f} and "
              f"WRITE_SIZE x {w_scale:.3f} of its bytes; every figure below is scaled by these factors.", "",
              "| kernel | launches | read GB/launch | written GB/launch |", "|---|---:|---:|---:|"]
    for k in sorted(fetch, key=lambda k: -fetch[k][0]):
        if k not in write:
            continue
        rd = fetch[k][0] / fetch[k][1] * 1024 * f_scale
        wr = write[k][0] / write[k][1] * 1024 * w_scale
        lines.append(f"| {k} | {fetch[k][1]} | {rd / 1e9:.4f} | {wr / 1e9:.4f} |")
    open(os.path.join(ROOT, "profiles", f"clha_step_{name}_hbm_traffic.md"), "w").write("\n".join(lines) + "\n")

    # matrix-core and LDS counters per kernel (sums over all units, per launch)
    trace = _csv(_find(os.path.join(d, "trace"), "kernel_trace.csv"))
    dur = {}
    for r in trace:
        v = dur.setdefault(_short(r["Kernel_Name"]), [])
        v.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    avg_ns = {k: sorted(v)[len(v) // 2] for k, v in dur.items()}
    m = {c: per_kernel("mfma", c) for c in MFMA_COUNTERS.split()}
    ld = {c: per_kernel("lds", c) for c in LDS_COUNTERS.split()}
    per = lambda tab, c, k: tab[c][k][0] / tab[c][k][1] if k in tab[c] else 0.0
    lines = [f"# Matrix-core and LDS counters per launch, {name} workload (MI355X, rocprofv3)", "",
             "Commands (repository root), one pass each:", "", f"    {cmd['mfma']}", f"    {cmd['lds']}", "",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 256 CUs), the share of CU cycles with",
             "the matrix pipe busy while the kernel ran (counters serialise kernels, so each launch has the",
             "GPU alone).  Executed TFLOP/s = 512 x SQ_INSTS_VALU_MFMA_MOPS_<type> over the launch's median",
             "duration in the kernel trace (tile overcompute included, so it is at least the algorithmic",
             "rate).  LDS bank conflicts are SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE (cycles).", "",
             "| kernel | launches | MFMA busy | bf16 TFLOP/s | int8 TOP/s | fp32 TFLOP/s | fp64 TFLOP/s | "
             "LDS conflict / active |", "|---|---:|---:|---:|---:|---:|---:|---:|"]
    ks = sorted(m["GRBM_GUI_ACTIVE"], key=lambda k: -per(m, "SQ_VALU_MFMA_BUSY_CYCLES", k))
    rec_counters = {}
    for k in ks:
        busy = per(m, "SQ_VALU_MFMA_BUSY_CYCLES", k)
        gui = per(m, "GRBM_GUI_ACTIVE", k)
        if busy == 0 and per(ld, "SQ_LDS_IDX_ACTIVE", k) == 0:
            continue
        t = avg_ns.get(k)
        rate = {ty: (512 * per(m, f"SQ_INSTS_VALU_MFMA_MOPS_{ty}", k) / (t * 1e-9) / 1e12 if t else 0.0)
                for ty in ("BF16", "I8", "F32", "F64")}
        act, conf = per(ld, "SQ_LDS_IDX_ACTIVE", k), per(ld, "SQ_LDS_BANK_CONFLICT", k)
        u = busy / (gui * 256) if gui else 0.0
        rec_counters[k] = {"mfma_busy": u, "lds_conflict_per_active": conf / act if act else 0.0,
                           **{f"{ty.lower()}_rate": v for ty, v in rate.items()}}
        lines.append(f"| {k} | {m['GRBM_GUI_ACTIVE'][k][1]} | {u:.3f} | {rate['BF16']:.1f} | {rate['I8']:.1f} | "
                     f"{rate['F32']:.1f} | {rate['F64']:.2f} | {conf / act if act else 0.0:.4f} |")
    open(os.path.join(ROOT, "profiles", f"clha_step_{name}_mfma_lds_counters.md"), "w").write("\n".join(lines) + "\n")

    # the collection's Gram-sum kernel (operands read from x by token id)
    sk = "clha::syrk_kernel<true>"
    rec = {"workload": name, "kernel": "syrk_kernel<true>", "syrk_source_sha256_16": syrk_source_hash(),
           "fetch_kib_per_launch": fetch[sk][0] / fetch[sk][1], "write_kib_per_launch": write[sk][0] / write[sk][1],
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_bytes_per_launch": (fetch[sk][0] / fetch[sk][1] * f_scale + write[sk][0] / write[sk][1] * w_scale) * 1024,
           "counters": rec_counters.get(sk),
           "commands": [cmd[k] for k in ("fetch", "write", "copy_fetch", "copy_write", "mfma", "lds")]}
    json.dump(rec, open(traffic_file(name), "w"), indent=1)
    print(json.dumps(rec))


EXPERIMENT_TAUS = (0.01, 0.03, 0.1, 0.3, 1.0, 3.0, 10.0)


def experiment(args):
    """The CLHA summary's section-4 experiments on the drift-stress shapes (d 4096,
    128 routed experts top-8, 262,144 tokens per layer, 2048x4096 bf16 weights,
    2-bit, group 64), every expert quantized under PLIC, CLHA-rt and CLHA-eq:
      drift      layer b's activations (1 - t) x_a + t z for t in 0, .25, .5, .75, 1,
                 router logits x R of each layer's own activations;
      sharpness  the activations at t = 0.5 with sampled routing, logits
                 x R / tau + Gumbel noise per layer, over a range of tau.
    Each row: routing divergence (JSD of the expert loads, top-K overlap) and, per
    weighting, the summed loss over the experts under the combined Hessian and
    under each layer's own (the calibration-Hessian error).  Writes one JSON file."""
    import numpy as np
    import torch
    import gen
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.sweep import drift_sweep, sharpness_sweep

    wl = gen.WORKLOADS[5]
    dev = torch.device("cuda", 0)

    def bits_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, 0, max_tokens=wl.n_tokens, device=dev)
    weights = {e: bits_dev(w) for e, w in gen.all_expert_weights(wl, 0, range(wl.n_routed)).items()}
    t0 = time.perf_counter()
    if args.experiment == "drift":
        def inputs_for(t):
            inp = gen.pair_inputs(wl, 0, t=t)
            log(f"drift t={t}: inputs after {time.perf_counter() - t0:.1f} s")
            return (bits_dev(inp["x"][0]), bits_dev(inp["x"][1]),
                    torch.from_numpy(inp["logits"][0]).to(dev), torch.from_numpy(inp["logits"][1]).to(dev))
        rows = drift_sweep(ctx, inputs_for, wl.drift, weights, wl.bits, wl.group, wl.block, wl.damp)
        what = "drift t"
    else:
        xa, xb = gen.activations(wl, 0, t=0.5)
        rk = wl.scaled(logit_kind="router")
        base = [gen.router_logits(rk, 0, 0, xa), gen.router_logits(rk, 0, 1, xb)]
        x = [bits_dev(xa), bits_dev(xb)]

        def logits_for(tau):
            log(f"sharpness tau={tau}: logits after {time.perf_counter() - t0:.1f} s")
            return [torch.from_numpy(gen.sharpness_logits(wl, 0, l, (xa, xb)[l], tau, base=base[l])).to(dev)
                    for l in range(2)]
        rows = sharpness_sweep(ctx, x, logits_for, EXPERIMENT_TAUS, weights, wl.bits, wl.group, wl.block,
                               wl.damp)
        what = "router temperature tau"
    cmd = f"python3 bench.py --experiment {args.experiment}"
    table = {"experiment": args.experiment, "command": cmd, "varied": what,
             "workload": {"name": wl.name, "d": wl.d, "routed_experts": wl.n_routed, "top_k": wl.top_k,
                          "tokens_per_layer": wl.n_tokens, "matrix_shape": [wl.rows, wl.d], "bits": wl.bits,
                          "group": wl.group, "damp": wl.damp,
                          "activations": "x_a ~ N(0,1); x_b = (1 - t) x_a + t z",
                          "logits": ("x R per layer" if args.experiment == "drift"
                                     else "x R / tau + Gumbel(0,1) per layer, t = 0.5")},
             "losses": "sums over the experts of tr[(Wq - W) H (Wq - W)^T]: comb = the weighting's own "
                       "H_comb, a / b = layer a's / b's Hessian",
             "rows": rows}
    out = args.out or os.path.join(ROOT, "profiles", f"experiment_{args.experiment}.json")
    json.dump(table, open(out, "w"), indent=1)
    log(f"wrote {out} after {time.perf_counter() - t0:.1f} s")
    print(json.dumps({"experiment": args.experiment, "rows": len(rows), "out": out}), flush=True)
    return 0


def down_proj_bench(args):
    """The down_proj calibration step of the mid-MoE block (see the module docstring)."""
    import numpy as np
    import torch
    import gen
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.calibrate import SharedGroupCalibration

    wl = gen.WORKLOADS[2]
    n, E, K, nsh, f, dm = wl.n_tokens, wl.n_routed, wl.top_k, wl.n_shared, wl.rows, wl.d
    dev = torch.device("cuda", 0)
    inp = gen.pair_inputs(wl)
    x = [torch.from_numpy(inp["x"][l].view(np.int16)).to(dev) for l in range(2)]
    lg = [torch.from_numpy(inp["logits"][l]).to(dev) for l in range(2)]
    main_ctx = clha.Context(dm, E, K, 0, n, device=dev)
    down = clha.Context(f, E + nsh, K, 0, n, device=dev)
    wgu = [torch.from_numpy(gen.expert_weights(wl, 0, e).view(np.int16)).to(dev) for e in range(E + nsh)]
    w_down = [torch.from_numpy(gen.swiglu_weights(2000 + e, 1, dm // 2, f)[0].view(np.int16)).to(dev)
              .view(torch.bfloat16) for e in range(E + nsh)]
    routing = []
    for l in range(2):
        main_ctx.register_layer(l, *main_ctx.new_layer_buffers())
        ids = torch.empty(n * K, dtype=torch.int32, device=dev)
        off = torch.empty(E + 1, dtype=torch.int64, device=dev)
        main_ctx.collect_hessians(l, x[l], lg[l], offsets_out=off, token_ids_out=ids)
        routing.append((ids, off))
    cal = SharedGroupCalibration(down, [0, 1])
    outputs = cal.make_outputs(range(E + nsh), dm, wl.group)
    jobs = [{"H": cal.H[e], "W": w_down[e], "bits": wl.bits, **outputs[e]} for e in range(E + nsh)]
    prep = down.prepare_gptq(jobs, f)

    def step():
        cal.reset()
        for l in range(2):
            down.collect_down_hessians(l, x[l], routing[l][0], routing[l][1], wgu, E)
        cal.aggregate("rt")
        down.run_gptq(prep, wl.group, 128, wl.damp)

    for _ in range(args.warmup):
        step()
    down.sync()
    down.set_timing(True)
    down.read_timing()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    stages = {k: v[0] / args.steps for k, v in down.read_timing().items() if v[1]}
    rows = 2 * (n * K + nsh * n)
    gemm_flops = rows * 2 * dm * 2 * f / 2          # per collection (one layer)
    gemm_ms = stages.get("gather", 0.0) / 2
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None
    line = {"metric": "down_proj matrices calibrated/sec (SwiGLU inputs + Hessians + CLHA-GPTQ)",
            "value": round((E + nsh) / (ms * 1e-3), 2), "unit": "matrices/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "mid_moe_block_down_proj", "layers": 2, "tokens_per_layer": n, "d_model": dm,
                       "f": f, "routed_experts": E, "top_k": K, "shared_experts": nsh, "matrices": E + nsh,
                       "matrix_shape": [dm, f], "bits": wl.bits, "group": wl.group, "alpha": "rt"},
            "roofline": {"kernel": "down_gemm_kernel", "bound": "mfma",
                         "achieved": round(achieved, 2) if achieved else None, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4) if achieved else None,
                         "traffic": down_traffic(), "avg_launch_ms": round(gemm_ms, 4),
                         "flops_per_launch": gemm_flops},
            "stages_ms_per_step": {k: round(v, 4) for k, v in stages.items()}}
    print(json.dumps(line), flush=True)
    return 0


def main():
    args = parse()
    if args.profile_commands:
        for _, c in PROFILE_RUNS:
            print(c.format(dir=args.profile_commands, wid=args.workload))
        return 0
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return 0
    if args.summarize_options_profile:
        summarize_options_profile(*args.summarize_options_profile)
        return 0
    if args.summarize_down_profile:
        summarize_down_profile(*args.summarize_down_profile)
        return 0
    if args.down_counter_commands:
        for _, c in DOWN_COUNTER_RUNS:
            print(c.format(dir=args.down_counter_commands))
        return 0
    if args.summarize_down_traffic:
        summarize_down_traffic(args.summarize_down_traffic)
        return 0
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the multi-GPU "
              "exchange is designed, not built)", file=sys.stderr)
        return 2
    if args.down_proj:
        return down_proj_bench(args)
    if args.experiment:
        return experiment(args)
    return calibration_bench(args)


def traffic_file(wl_name):
    return os.path.join(ROOT, "profiles", f"syrk_{wl_name}_traffic.json")


def calibration_bench(args):
    """The CLHA calibration step over one CLWS pair; see the module docstring."""
    import numpy as np
    import torch
    import gen
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.calibrate import SharedGroupCalibration

    wl = gen.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    # the step's units: CLWS pairs, or for the drift workload one pair at each drift t
    units = list(wl.drift) if wl.drift else list(range(wl.n_pairs))
    if args.pairs:
        units = units[:args.pairs]
    experts = list(range(wl.n_experts_total))

    def bits_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, wl.n_shared, max_tokens=wl.n_tokens, device=dev)
    H = torch.empty(ctx.slots, wl.d, wl.d, dtype=torch.float32, device=dev)
    x, lg, W, cals, host0 = [], [], [], [], None
    t0 = time.perf_counter()
    for u, unit in enumerate(units):
        if wl.drift:
            inp = gen.pair_inputs(wl, 0, t=unit)
            w_host = gen.all_expert_weights(wl, 0, experts) if u == 0 else host0[1]
        else:
            inp = gen.pair_inputs(wl, unit)
            w_host = gen.all_expert_weights(wl, unit, experts)
        if u == 0 or (wl.drift and u == len(units) - 1):
            host0 = (inp, w_host)
        x += [bits_dev(b) for b in inp["x"]]
        lg += [torch.from_numpy(a).to(dev) for a in inp["logits"]]
        if not wl.drift or u == 0:
            W.append({e: (bits_dev(w) if wl.w_dtype == "bf16" else torch.from_numpy(w).to(dev))
                      for e, w in w_host.items()})
        cals.append(SharedGroupCalibration(ctx, [2 * u, 2 * u + 1], H=H))
        del inp
        log(f"unit {u + 1}/{len(units)} ({'t=' + str(unit) if wl.drift else 'pair ' + str(unit)}) "
            f"resident after {time.perf_counter() - t0:.1f} s")
    # one GPTQ workspace for every pair's batch: the batches run one after another
    outputs = [cals[0].make_outputs(experts, W[i][0].shape[0], wl.group) for i in range(len(W))]
    jobs0 = cals[0].quantize_jobs(W[0], wl.bits, wl.shared_bits, outputs[0])
    ws = torch.empty(ctx.gptq_workspace_bytes(jobs0, wl.d, args.act_order, args.static_groups),
                     dtype=torch.uint8, device=dev)
    preps = [cals[0].prepare_quantize(W[i], wl.bits, wl.shared_bits, wl.group, outputs=outputs[i],
                                      act_order=args.act_order, static_groups=args.static_groups,
                                      workspace=ws)[0] for i in range(len(W))]
    ctx.workspace("collect", ctx.collect_workspace_bytes())
    n_mats = len(experts) * len(wl.mats)

    def step(i):
        u = i % len(units)
        cal = cals[u]
        cal.reset()
        cal.collect(2 * u, x[2 * u], lg[2 * u])
        cal.collect(2 * u + 1, x[2 * u + 1], lg[2 * u + 1])
        cal.aggregate(wl.alpha)
        ctx.run_gptq(preps[0 if wl.drift else u], wl.group, wl.block, wl.damp)

    for i in range(args.warmup):
        step(i)
    ctx.sync()
    log(f"warmup done ({args.warmup} steps)")
    ctx.set_timing(True)
    ctx.read_timing()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ctx.sync()
    stages = ctx.read_timing()
    ctx.set_timing(False)
    ms_per_step = (t1 - t0) / args.steps * 1e3
    value = n_mats / (ms_per_step / 1e3)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    # Gram-sum roofline: algorithmic flops = sum over the routed slots of n_e d (d+1), averaged
    # per launch (the shared slot's sums are formed from the routed ones, not by the kernel)
    launched = [i % len(units) for i in range(args.steps)]
    counts = {u: [cals[u].counts[l].cpu().numpy() for l in cals[u].layer_ids] for u in set(launched)}
    rows_per_launch = sum(float(c[:wl.n_routed].sum()) for u in launched for c in counts[u]) / (2 * args.steps)
    flops_per_launch = rows_per_launch * wl.d * (wl.d + 1)
    syrk_ms, syrk_calls = stages["syrk"]
    syrk_avg_ms = syrk_ms / max(syrk_calls, 1)
    achieved = flops_per_launch / (syrk_avg_ms / 1e3) / 1e12
    traffic = None
    tf = traffic_file(wl.name)
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("syrk_source_sha256_16") == syrk_source_hash():
            traffic = rec.get("hbm_bytes_per_launch")
    roofline = {"kernel": "syrk_kernel<true>", "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "avg_launch_ms": round(syrk_avg_ms, 4),
                "flops_per_launch": flops_per_launch}
    stages_ms = {k: round(v[0] / args.steps, 4) for k, v in stages.items() if v[1]}

    # end-to-end roofline: each step's algorithmic work at the published peak of its bound
    # (Gram sums on bf16 MFMA, their operands read straight from x; inverse Cholesky
    # (2/3)d^3 per distinct Hessian and GPTQ r c (c-1) per matrix on fp32 MFMA)
    n_hess = wl.n_routed + (1 if wl.n_shared else 0)
    rows_total = sum(int(W[0][e].shape[0]) for e in experts)
    terms = {"gram_sums": 2 * flops_per_launch / (PEAK_BF16_TFLOPS * 1e12),
             "inverse_cholesky": n_hess * (2.0 / 3.0) * wl.d ** 3 / (PEAK_FP32_TFLOPS * 1e12),
             "gptq": rows_total * wl.d * (wl.d - 1) / (PEAK_FP32_TFLOPS * 1e12)}
    t_roof_ms = sum(terms.values()) * 1e3
    end_to_end = {"t_roof_ms": round(t_roof_ms, 3), "frac": round(t_roof_ms / ms_per_step, 4),
                  "terms_ms": {k: round(v * 1e3, 3) for k, v in terms.items()},
                  "peaks": "bf16 MFMA 2500 TFLOP/s, fp32 MFMA 157.3 TFLOP/s"}

    n_layers = 2 * (wl.n_pairs if not wl.drift else 1)
    config = {"workload": wl.name, "layers": n_layers, "clws_pairs": wl.n_pairs,
              "pairs_resident": len(units) if not wl.drift else 1,
              "step": ("one CLWS pair at one drift t (cycling t over " + str(list(units)) + ")") if wl.drift
              else "one CLWS pair (cycling over the resident pairs)",
              "tokens_per_layer": wl.n_tokens, "d": wl.d,
              "routed_experts": wl.n_routed, "top_k": wl.top_k, "shared_experts": wl.n_shared,
              "router_load": {"normal": "N(0,1) logits", "zipf": "Zipf(1.1)",
                              "router": "logits = x R"}[wl.logit_kind],
              "matrices_per_step": n_mats, "matrix_shape": [wl.rows, wl.d], "bits": wl.bits,
              "shared_bits": wl.shared_bits, "group": wl.group, "alpha": wl.alpha}
    if args.act_order or args.static_groups:
        config["gptq_options"] = [o for o, on in (("act_order", args.act_order),
                                                   ("static_groups", args.static_groups)) if on]
    config["precision"] = ("Gram sums bf16 in / fp32 accumulate; Cholesky fp64 values, its long products "
                           "exact int8 digit products of 42-bit expansions; triangular inverse at fp32 "
                           "precision (three bf16 parts per operand); GPTQ fp32, trailing products exact "
                           "int8 digit products of 28-bit expansions")
    out = {"metric": METRIC, "value": round(value, 2), "unit": "matrices/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": config,
           "roofline": roofline, "stages_ms_per_step": stages_ms, "end_to_end_roofline": end_to_end}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl, host0[0], host0[1])
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
