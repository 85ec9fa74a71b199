#!/usr/bin/env python3
"""Throughput of the CLHA calibration hot path on one MI355X (gfx950).

One step is one full calibration pass of the mid-MoE-block workload (two
layers sharing 64 routed experts, top-6, plus 2 always-active shared experts;
d = 2048; 65,536 tokens per layer; gate and up 1408x2048 bf16 per expert;
3-bit, group 128, routing-frequency alpha):
  reset accumulators -> collect layer a -> collect layer b (route, bucket,
  gather, Gram sums) -> aggregate H_comb -> GPTQ of 66 stacked gate|up jobs
  (damping, factor of the inverse, column loop, lazy block updates, loss)
= 132 expert matrices.  Inputs are seeded synthetic arrays resident in HBM
before the timed region.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

--down-proj measures the experts' second matrices instead (the same block and
batch): one step resets the down_proj accumulators, collects both layers'
SwiGLU inputs h = bf16(silu(x Wg^T) * (x Wu^T)) and their Gram sums (routing
taken from the main context's collection of the same batch, done once before
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "syrk_mid_moe_block_traffic.json")
SYRK_SRC = os.path.join(ROOT, "gptq_calibration_moe_amd", "csrc", "syrk.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=2, help="workload id of gen.WORKLOADS (default 2)")
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
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def syrk_source_hash():
    return hashlib.sha256(open(SYRK_SRC, "rb").read()).hexdigest()[:16]


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


# Profiling runs behind the committed summaries.  The counter runs read
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) in passes of their own; the
# copy probe moves a known number of bytes so that each counter can be scaled
# to bytes.  `--profile-commands DIR` prints these lines; `--summarize-profiles
# DIR` turns their CSV output into the text summaries.
COPY_BYTES = 1 << 30
PROFILE_RUNS = [
    ("trace", "timeout -k 10 600 rocprofv3 --kernel-trace --stats --output-format csv -d {dir}/trace -o run "
              "-- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline"),
    ("fetch", "timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {dir}/fetch -o run "
              "-- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline"),
    ("write", "timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {dir}/write -o run "
              "-- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline"),
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
    """Kernel-time table of a traced bench run (1 warm-up + `timed` steps).  Each
    kernel's first launches (1/steps of them) belong to the warm-up step, whose
    first touch of fresh device memory is slow; they are left out.  With
    setup_free, kernels launched fewer than `steps` times ran only in the set-up
    before the steps and are left out too."""
    trace = _csv(_find(trace_dir, "kernel_trace.csv"))
    by_name = {}
    for r in trace:
        by_name.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    stats = []
    for name, ds in by_name.items():
        ds.sort()
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
             f"{steps} steps traced (1 warm-up + {timed} timed); the warm-up step's launches are left out "
             f"and per-step figures are totals / {timed}.", *notes, "",
             "| kernel | calls/step | ms/step | avg us/launch | % |", "|---|---:|---:|---:|---:|"]
    total = sum(float(r["TotalDurationNs"]) for r in stats)
    for r in stats:
        t = float(r["TotalDurationNs"])
        lines.append(f"| {_short(r['Name'])} | {int(r['Calls']) / timed:g} | {t / 1e6 / timed:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {100 * t / total:.1f} |")
    lines += ["", f"Sum of kernel time per step: {total / 1e6 / timed:.3f} ms", ""]
    return lines


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
                 "-- python3 bench.py --act-order --static-groups --steps 3 --warmup 1 --no-cpu-baseline")


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
           "    timeout -k 10 400 python3 -u bench.py --act-order --static-groups --no-cpu-baseline", "",
           "Output:", "", "```json", line, "```", ""]
    open(os.path.join(ROOT, "profiles", "bench_gptq_options_mid_moe_block.md"), "w").write("\n".join(out))


def summarize_profiles(d, workload_name="mid_moe_block"):
    """Writes the kernel-trace summary and the per-kernel HBM traffic summary
    (counter values scaled by the copy probe) under profiles/."""
    cmd = {k: c.format(dir=d) for k, c in PROFILE_RUNS}
    lines = _trace_lines(os.path.join(d, "trace"),
                         f"# Kernel time per step, {workload_name} workload (MI355X, rocprofv3 kernel trace)",
                         cmd["trace"],
                         ["The factorisation runs as four Hessian groups on concurrent streams, overlapped with the",
                          "GPTQ kernels, so per-kernel times overlap in wall time; wall-clock stage times are",
                          "`stages_ms_per_step` in the bench line."])
    open(os.path.join(ROOT, "profiles", f"clha_step_{workload_name}_kernel_trace.md"), "w").write("\n".join(lines))

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
    lines = [f"# HBM traffic per launch, {workload_name} workload (MI355X, rocprofv3 counters)", "",
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
    open(os.path.join(ROOT, "profiles", f"clha_step_{workload_name}_hbm_traffic.md"), "w").write("\n".join(lines) + "\n")
    sk = "clha::syrk_kernel"
    rec = {"workload": workload_name, "kernel": "syrk_kernel", "syrk_source_sha256_16": syrk_source_hash(),
           "fetch_kib_per_launch": fetch[sk][0] / fetch[sk][1], "write_kib_per_launch": write[sk][0] / write[sk][1],
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_bytes_per_launch": (fetch[sk][0] / fetch[sk][1] * f_scale + write[sk][0] / write[sk][1] * w_scale) * 1024,
           "commands": [cmd[k] for k in ("fetch", "write", "copy_fetch", "copy_write")]}
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(rec))


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
                         "traffic": None, "avg_launch_ms": round(gemm_ms, 4), "flops_per_launch": gemm_flops},
            "stages_ms_per_step": {k: round(v, 4) for k, v in stages.items()}}
    print(json.dumps(line), flush=True)
    return 0


def main():
    args = parse()
    if args.profile_commands:
        for _, c in PROFILE_RUNS:
            print(c.format(dir=args.profile_commands))
        return 0
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return 0
    if args.summarize_options_profile:
        summarize_options_profile(*args.summarize_options_profile)
        return 0
    if args.summarize_down_profile:
        summarize_down_profile(*args.summarize_down_profile)
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
    import numpy as np
    import torch
    import gen
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.calibrate import SharedGroupCalibration

    wl = gen.WORKLOADS[args.workload]
    if wl.n_pairs != 1 and args.workload != 2:
        wl = wl.scaled(n_pairs=1)
    dev = torch.device("cuda", 0)
    t0 = time.perf_counter()
    inp = gen.pair_inputs(wl, t=wl.drift[-1] if wl.drift else None)
    experts = list(range(wl.n_experts_total))
    w_host = {e: gen.expert_weights(wl, 0, e) for e in experts}
    log(f"generated {wl.name} inputs in {time.perf_counter() - t0:.1f} s")

    def bits_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

    x = [bits_dev(b) for b in inp["x"]]
    lg = [torch.from_numpy(a).to(dev) for a in inp["logits"]]
    W = {e: (bits_dev(w) if wl.w_dtype == "bf16" else torch.from_numpy(w).to(dev)) for e, w in w_host.items()}
    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, wl.n_shared, max_tokens=wl.n_tokens, device=dev)
    cal = SharedGroupCalibration(ctx, [0, 1])
    prep, outputs = cal.prepare_quantize(W, wl.bits, wl.shared_bits, wl.group,
                                         act_order=args.act_order, static_groups=args.static_groups)
    ctx.workspace("collect", ctx.collect_workspace_bytes())
    n_mats = len(experts) * len(wl.mats)

    def step():
        cal.reset()
        cal.collect(0, x[0], lg[0])
        cal.collect(1, x[1], lg[1])
        cal.aggregate(wl.alpha)
        ctx.run_gptq(prep, wl.group, wl.block, wl.damp)

    for i in range(args.warmup):
        step()
    ctx.sync()
    log(f"warmup done ({args.warmup} steps)")
    ctx.set_timing(True)
    ctx.read_timing()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ctx.sync()
    stages = ctx.read_timing()
    ctx.set_timing(False)
    ms_per_step = (t1 - t0) / args.steps * 1e3
    value = n_mats / (ms_per_step / 1e3)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    # Gram-sum roofline: algorithmic flops = sum over slots of n_e d (d+1), per launch
    counts = [cal.counts[l].cpu().numpy() for l in (0, 1)]
    flops_per_launch = sum(float(c.sum()) for c in counts) * wl.d * (wl.d + 1) / 2.0
    syrk_ms, syrk_calls = stages["syrk"]
    syrk_avg_ms = syrk_ms / max(syrk_calls, 1)
    achieved = flops_per_launch / (syrk_avg_ms / 1e3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("syrk_source_sha256_16") == syrk_source_hash() and rec.get("workload") == wl.name:
            traffic = rec.get("hbm_bytes_per_launch")
    roofline = {"kernel": "syrk_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "avg_launch_ms": round(syrk_avg_ms, 4),
                "flops_per_launch": flops_per_launch}
    stages_ms = {k: round(v[0] / args.steps, 4) for k, v in stages.items() if v[1]}

    # gather rate on algorithmic bytes (each token read once, each routed row written once)
    routed = [float(c[:wl.n_routed].sum()) for c in counts]
    gather_bytes = sum(wl.n_tokens * wl.d * 2 + p * wl.d * 2 for p in routed)
    gather_gbs = gather_bytes / (stages_ms["gather"] / 1e3) / 1e9 if stages_ms.get("gather") else None
    # end-to-end roofline: each step's algorithmic work at the published peak of its bound
    # (Gram sums on bf16 MFMA; inverse Cholesky (2/3)d^3 per distinct Hessian and GPTQ
    # r c (c-1) per matrix on fp32 MFMA; the gather on HBM)
    n_hess = wl.n_routed + (1 if wl.n_shared else 0)
    rows_total = sum(int(W[e].shape[0]) for e in experts)
    terms = {"gram_sums": 2 * flops_per_launch / (PEAK_BF16_TFLOPS * 1e12),
             "inverse_cholesky": n_hess * (2.0 / 3.0) * wl.d ** 3 / (PEAK_FP32_TFLOPS * 1e12),
             "gptq": rows_total * wl.d * (wl.d - 1) / (PEAK_FP32_TFLOPS * 1e12),
             "gather": gather_bytes / (PEAK_HBM_GBS * 1e9)}
    t_roof_ms = sum(terms.values()) * 1e3
    end_to_end = {"t_roof_ms": round(t_roof_ms, 3), "frac": round(t_roof_ms / ms_per_step, 4),
                  "terms_ms": {k: round(v * 1e3, 3) for k, v in terms.items()},
                  "peaks": "bf16 MFMA 2500 TFLOP/s, fp32 MFMA 157.3 TFLOP/s, HBM 8000 GB/s"}

    out = {"metric": METRIC, "value": round(value, 2), "unit": "matrices/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": wl.name, "layers": 2, "tokens_per_layer": wl.n_tokens, "d": wl.d,
                      "routed_experts": wl.n_routed, "top_k": wl.top_k, "shared_experts": wl.n_shared,
                      "matrices": n_mats, "matrix_shape": [wl.rows, wl.d], "bits": wl.bits,
                      "shared_bits": wl.shared_bits, "group": wl.group, "alpha": wl.alpha,
                      **({"gptq_options": [o for o, on in (("act_order", args.act_order),
                                                            ("static_groups", args.static_groups)) if on]}
                         if args.act_order or args.static_groups else {}),
                      "precision": "Gram sums bf16 in / fp32 accumulate; Cholesky fp64 values, its "
                                   "long products exact int8 digit products of 42-bit expansions; "
                                   "triangular inverse at fp32 precision (three bf16 parts per operand); "
                                   "GPTQ fp32, trailing products exact int8 digit products of 28-bit "
                                   "expansions"},
           "roofline": roofline, "stages_ms_per_step": stages_ms,
           "gather_gbs": round(gather_gbs, 1) if gather_gbs else None, "end_to_end_roofline": end_to_end}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl, inp, w_host)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
