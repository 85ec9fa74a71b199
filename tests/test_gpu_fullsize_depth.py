"""Parity at the full sizes of the full-depth, CLHA-MP and drift-stress
workloads, in the launch configuration the benchmark times.

Full depth (d 2048, 64 routed experts top-6 under a Zipf(1.1) router load, 2
shared experts, 262,144 tokens per layer, equal weighting, 2-bit, group 128),
one CLWS pair of the twelve (every pair has the same shapes):
  * routing, counts, offsets and token lists of every token bit-exact;
  * all 65 combined Hessians on sampled rows (24 rows of each, every column);
  * GPTQ codes, grids and loss of the most and the least loaded routed expert
    and of both shared experts, from one batch of all 66 jobs.
CLHA-MP on the same arrays (routing-frequency weighting, shared experts at
3 bits, routed at 2): the shared jobs use the 3-bit range and match the oracle,
as does the most loaded routed expert.
Drift stress (d 4096, 128 routed experts top-8, router logits from the
activations, group 64, 2048x4096 matrices, 262,144 tokens per layer) at each
t in {0, 0.25, 0.5, 0.75, 1}: routing of every token, the sampled expert's
PLIC, CLHA-rt and CLHA-eq Hessians and GPTQ results, and its losses under the
combined Hessian and under each layer's own Hessian (the calibration-Hessian
error of the CLHA summary, section 4); at t = 0 CLHA equals PLIC bit for bit.

Tolerances as everywhere: routing bit-exact; Hessians 1e-4 normalised by
sqrt(H_ii H_jj); codes >= 99.9 % identical; loss within 1e-3 relative.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import (HESS_TOL, LOSS_RTOL, bits_to_dev, check_all_slots, check_gptq, dev, full_hessian,
                      say, slot_rows, to_dev, weights_to_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_calibration_moe_amd  # noqa: F401  (fails loudly if the library is missing)


# --------------------------------------------------------------------------- full depth, CLHA-MP

@pytest.fixture(scope="module")
def depth_pair():
    wl = gen.WORKLOADS[3]
    say("full depth: generating pair 0 at 262,144 tokens per layer")
    inp = gen.pair_inputs(wl, 0)
    buckets = []
    for l in range(2):
        tk = oracle.route(inp["logits"][l], wl.top_k)
        buckets.append(oracle.bucket(tk, wl.n_routed) + (tk,))
    w_host = gen.all_expert_weights(wl, 0, range(wl.n_experts_total))
    say("full depth: inputs and oracle routing ready")
    return {"wl": wl, "inp": inp, "buckets": [b[:3] for b in buckets], "topk": [b[3] for b in buckets],
            "w": w_host, "grams": {}}


def _collect_pair(wl, inp, modes):
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.calibrate import SharedGroupCalibration
    n, E, K = wl.n_tokens, wl.n_routed, wl.top_k
    ctx = clha.Context(wl.d, E, K, wl.n_shared, max_tokens=n, device=dev())
    cal = SharedGroupCalibration(ctx, [0, 1])
    routing = []
    cal.reset()
    for l in range(2):
        r = {"topk_out": torch.empty(n, K, dtype=torch.int32, device=dev()),
             "offsets_out": torch.empty(E + 1, dtype=torch.int64, device=dev()),
             "token_ids_out": torch.empty(n * K, dtype=torch.int32, device=dev())}
        cal.collect(l, bits_to_dev(inp["x"][l]), to_dev(inp["logits"][l]), **r)
        routing.append(r)
    H = {}
    for m in modes:
        H[m] = torch.empty(ctx.slots, wl.d, wl.d, dtype=torch.float32, device=dev())
        ctx.aggregate([0, 1], m, H[m])
    ctx.sync()
    return ctx, cal, routing, H


def _grams(P, e):
    """Per-layer full Gram sums of job e's slot (cached in the fixture)."""
    wl = P["wl"]
    slot = min(e, wl.n_routed)
    if slot not in P["grams"]:
        P["grams"][slot] = full_hessian(P["inp"]["x"], P["buckets"], slot, wl.n_routed)
    return P["grams"][slot]


def test_full_depth_pair_full_size(depth_pair):
    P = depth_pair
    wl, inp = P["wl"], P["inp"]
    E = wl.n_routed
    ctx, cal, routing, H = _collect_pair(wl, inp, ["eq"])
    for l in range(2):
        counts, offsets, ids = P["buckets"][l]
        assert np.array_equal(routing[l]["topk_out"].cpu().numpy(), P["topk"][l])
        assert np.array_equal(routing[l]["offsets_out"].cpu().numpy(), offsets)
        assert np.array_equal(routing[l]["token_ids_out"].cpu().numpy(), ids)
        got = cal.counts[l].cpu().numpy()
        assert np.array_equal(got[:E], counts) and got[E] == wl.n_tokens
    say("full depth: routing of every token bit-exact")
    check_all_slots(H["eq"], inp["x"], P["buckets"], E, ctx.slots, "eq", seed=31, label="full depth eq")
    # the benchmark's GPTQ batch: all 66 jobs on H_eq
    experts = list(range(wl.n_experts_total))
    W = {e: weights_to_dev(wl, P["w"][e]) for e in experts}
    outputs = cal.quantize(W, wl.bits, wl.shared_bits, wl.group, block=wl.block, damp=wl.damp, H=H["eq"])
    ctx.sync()
    load = P["buckets"][0][0] + P["buckets"][1][0]
    sample = [int(np.argmax(load)), int(np.argmin(load)), E, E + 1]
    assert load[sample[0]] > 20 * load[sample[1]]          # the Zipf skew is really there
    for e in sample:
        S, n = _grams(P, e)
        H_ref, _ = oracle.aggregate(S, n, "eq")
        check_gptq(wl, P["w"][e], H_ref, outputs[e], wl.bits, f"full depth expert {e} (rows {sum(n)})")


def test_clha_mp_full_size(depth_pair):
    P = depth_pair
    wl3 = P["wl"]
    wl = gen.WORKLOADS[4]
    assert wl.seed_base + wl.wid == wl3.seed_base + wl3.wid and wl.shared_bits == wl.bits + 1
    E = wl.n_routed
    ctx, cal, routing, H = _collect_pair(wl, P["inp"], ["rt"])
    experts = list(range(wl.n_experts_total))
    W = {e: weights_to_dev(wl, P["w"][e]) for e in experts}
    outputs = cal.quantize(W, wl.bits, wl.shared_bits, wl.group, block=wl.block, damp=wl.damp, H=H["rt"])
    ctx.sync()
    load = P["buckets"][0][0] + P["buckets"][1][0]
    for e in [int(np.argmax(load)), E, E + 1]:
        bits = wl.shared_bits if e >= E else wl.bits
        S, n = _grams(P, e)
        H_ref, _ = oracle.aggregate(S, n, "rt")
        _, codes = check_gptq(wl, P["w"][e], H_ref, outputs[e], bits, f"CLHA-MP expert {e} ({bits} bits)")
        if e >= E:
            assert codes.max() >= 1 << wl.bits, f"shared expert {e} does not use the {bits}-bit range"


# --------------------------------------------------------------------------- drift stress

@pytest.fixture(scope="module")
def drift_cache():
    return {}


@pytest.mark.parametrize("t", [0.0, 0.25, 0.5, 0.75, 1.0])
def test_drift_stress_full_size(t, drift_cache):
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.calibrate import SharedGroupCalibration
    wl = gen.WORKLOADS[5]
    n, E, K, d = wl.n_tokens, wl.n_routed, wl.top_k, wl.d
    say(f"drift t={t}: generating 262,144 tokens per layer at d={d}")
    inp = gen.pair_inputs(wl, 0, t=t)
    if "bucket_a" not in drift_cache:
        drift_cache["bucket_a"] = oracle.bucket(oracle.route(inp["logits"][0], K), E)
    buckets = [drift_cache["bucket_a"], oracle.bucket(oracle.route(inp["logits"][1], K), E)]
    if t == 0.0:                        # equal values (1 * x + 0 * z turns a -0 into +0)
        assert np.array_equal(gen.bf16_value(inp["x"][0]), gen.bf16_value(inp["x"][1]))
    ctx = clha.Context(d, E, K, 0, max_tokens=n, device=dev())
    cal = SharedGroupCalibration(ctx, [0, 1])
    cal.reset()
    for l in range(2):
        cal.collect(l, bits_to_dev(inp["x"][l]), to_dev(inp["logits"][l]))
    H = {}
    for name, layers, mode, alpha in (("a", [0], "explicit", [1.0]), ("b", [1], "explicit", [1.0]),
                                      ("rt", [0, 1], "rt", None), ("eq", [0, 1], "eq", None)):
        H[name] = torch.empty(ctx.slots, d, d, dtype=torch.float32, device=dev())
        ctx.aggregate(layers, mode, H[name], alpha=alpha)
    ctx.sync()
    for l in range(2):
        assert np.array_equal(cal.counts[l].cpu().numpy(), buckets[l][0]), l
    say(f"drift t={t}: counts of both layers bit-exact")
    # one sampled expert per t; PLIC is layer a's own Hessian
    e = [3, 41, 77, 100, 126][int(t * 4)]
    jobs = []
    wb = gen.expert_weights(wl, 0, e)
    Wd = weights_to_dev(wl, wb)
    for name in ("a", "rt", "eq"):
        jobs.append({"H": H[name][e], "W": Wd, "bits": wl.bits, "H_eval": H["a"][e],
                     "loss_eval": torch.empty(1, dtype=torch.float32, device=dev()),
                     "codes": torch.empty(wl.rows, d, dtype=torch.uint8, device=dev()),
                     "scales": torch.empty(wl.rows, d // wl.group, dtype=torch.float32, device=dev()),
                     "zeros": torch.empty(wl.rows, d // wl.group, dtype=torch.uint8, device=dev()),
                     "loss": torch.empty(1, dtype=torch.float32, device=dev()),
                     "status": torch.empty(1, dtype=torch.int32, device=dev())})
    ctx.gptq_quantize(jobs, d, wl.group, wl.block, wl.damp)
    loss_b = []
    for j in jobs:
        lb = torch.empty(1, dtype=torch.float32, device=dev())
        ctx.loss(Wd, j["codes"], j["scales"], j["zeros"], H["b"][e], wl.group, lb)
        loss_b.append(lb)
    ctx.sync()
    assert all(int(j["status"].cpu()[0]) == clha.OK for j in jobs)
    # oracle: the expert's per-layer Gram sums, its Hessians and GPTQ per weighting
    S, cnt = [], []
    for l in range(2):
        xs = slot_rows(inp["x"][l], buckets[l], e, E)
        S.append(oracle.gram(oracle.bf16_to_f64(xs)))
        cnt.append(xs.shape[0])
    H_l = [oracle.aggregate([S[l]], [cnt[l]], "explicit", alpha=[1.0])[0] for l in range(2)]
    refs = {"a": H_l[0], "rt": oracle.aggregate(S, cnt, "rt")[0], "eq": oracle.aggregate(S, cnt, "eq")[0]}
    wv = gen.weights_value(wl, wb).astype(np.float64)
    for k, name in enumerate(("a", "rt", "eq")):
        G = H[name][e].cpu().numpy().astype(np.float64)
        R = refs[name]
        dg = np.sqrt(np.diag(R))
        herr = float(np.max(np.abs(G - R) / np.outer(dg, dg)))
        assert herr <= HESS_TOL, f"t={t} {name}: H error {herr:.3e}"
        ref, codes = check_gptq(wl, wb, R, jobs[k], wl.bits, f"drift t={t} expert {e} {name}")
        for lname, Hr, got in (("a", H_l[0], jobs[k]["loss_eval"]), ("b", H_l[1], loss_b[k])):
            want = oracle.loss(wv, ref["wq"], Hr)
            g = float(got.cpu()[0])
            assert abs(g - want) <= LOSS_RTOL * abs(want), f"t={t} {name} loss_{lname}: {g} vs {want}"
    if t == 0.0:
        for k in (1, 2):                # identical layers: CLHA-rt and CLHA-eq are PLIC exactly
            assert torch.equal(jobs[k]["codes"], jobs[0]["codes"]), k
            assert torch.equal(jobs[k]["scales"], jobs[0]["scales"]), k
        say("drift t=0: CLHA-rt and CLHA-eq codes equal PLIC bit for bit")
