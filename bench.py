#!/usr/bin/env python3
"""Throughput of the CLHA calibration hot path on one MI355X (gfx950).

One step is one full calibration pass of the mid-MoE-block workload (two
layers sharing 64 routed experts, top-6, plus 2 always-active shared experts;
d = 2048; 65,536 tokens per layer; gate and up 1408x2048 bf16 per expert;
3-bit, group 128, routing-frequency alpha):
  reset accumulators -> collect layer a -> collect layer b (route, bucket,
  gather, Gram sums) -> aggregate H_comb -> GPTQ of 66 stacked gate|up jobs
  (damping, fp64 factor of the inverse, column loop, lazy block updates, loss)
= 132 expert matrices.  Inputs are seeded synthetic arrays resident in HBM
before the timed region.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "syrk_mid_moe_block_traffic.json")
SYRK_SRC = os.path.join(ROOT, "gptq_calibration_moe_amd", "csrc", "syrk.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=2, help="workload id of gen.WORKLOADS (default 2)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def syrk_source_hash():
    return hashlib.sha256(open(SYRK_SRC, "rb").read()).hexdigest()[:16]


def cpu_baseline(wl, inp, w_expert0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    routing and bucketing of all tokens of both layers, then Gram sums of routed
    expert 0 in both layers, aggregation, GPTQ of its gate|up job and its loss."""
    import numpy as np
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
    S, n = [], []
    for l in range(2):
        tk = oracle.route(inp["logits"][l], wl.top_k)
        s_l, c_l = oracle.layer_hessians(inp["x"][l], tk, wl.n_routed, wl.n_shared, slots=[0])
        S.append(s_l[0])
        n.append(c_l[0])
    H, _ = oracle.aggregate(S, n, wl.alpha)
    import gen
    wv = gen.weights_value(wl, w_expert0).astype(np.float64)
    g = oracle.gptq(wv, H, wl.bits, wl.group, wl.damp, wl.block)
    oracle.loss(wv, g["wq"], H)
    dt = time.perf_counter() - t0
    mats = len(wl.mats)
    return {"value": round(mats / dt, 4), "unit": "matrices/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"oracle (fp64 NumPy) on routed expert 0 of the {wl.name} workload: routing and "
                       f"bucketing of all {wl.n_tokens} tokens of both layers, that expert's Gram sums in "
                       f"both layers, aggregation, GPTQ of its {wl.job_rows}x{wl.d} gate|up job and the "
                       f"loss = {mats} matrices in {dt:.2f} s")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (every run here uses "
              "exactly one MI355X; the multi-GPU design is described, not built)", file=sys.stderr)
        return 2
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
    prep, outputs = cal.prepare_quantize(W, wl.bits, wl.shared_bits, wl.group)
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

    out = {"metric": METRIC, "value": round(value, 2), "unit": "matrices/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": wl.name, "layers": 2, "tokens_per_layer": wl.n_tokens, "d": wl.d,
                      "routed_experts": wl.n_routed, "top_k": wl.top_k, "shared_experts": wl.n_shared,
                      "matrices": n_mats, "matrix_shape": [wl.rows, wl.d], "bits": wl.bits,
                      "shared_bits": wl.shared_bits, "group": wl.group, "alpha": wl.alpha,
                      "precision": "Gram sums bf16 in / fp32 accumulate; factor of the inverse fp64; "
                                   "GPTQ propagation fp32"},
           "roofline": roofline, "stages_ms_per_step": stages_ms}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl, inp, w_host[0])
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
