"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the CPU oracle under the stated tolerances."""
import numpy as np
import torch

import gen
import oracle

HESS_TOL = 1e-4        # max |H_gpu - H_ref| / sqrt(H_ref_ii H_ref_jj)
CODE_AGREE = 0.999     # fraction of identical codes
LOSS_RTOL = 1e-3       # relative loss difference
# Scales of rows whose codes all agree: a scale is the range of up to g weights
# after fp32 propagation, whose error against the fp64 oracle grows like
# sqrt(cond(Hd)) * sqrt(c) * eps32 (about 2.4e-5 at cond 1.2e3, c = 128).
SCALE_RTOL = 5e-5


def dev():
    return torch.device("cuda", 0)


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def weights_to_dev(wl, w: np.ndarray) -> torch.Tensor:
    return bits_to_dev(w) if wl.w_dtype == "bf16" else to_dev(w.astype(np.float32))


def hess_err(G, R) -> float:
    """Max error over the lower triangle, normalised by sqrt(R_ii R_jj)."""
    G = np.asarray(G, np.float64)
    R = np.asarray(R, np.float64)
    dg = np.sqrt(np.maximum(np.diag(R), 0.0))
    den = np.outer(dg, dg)
    low = np.tril(np.ones_like(R, dtype=bool))
    zero = low & (den == 0)
    if np.any(G[zero] != 0) and np.any(R[zero] == 0):
        return float("inf")
    m = low & (den > 0)
    if not m.any():
        return 0.0
    return float(np.max(np.abs(G - R)[m] / den[m]))


def run_group(wl, inputs, jobs, *, mode=None, alpha=None, chunks=1, layers=(0, 1),
              block=128, keep_routing=True, agg_layers=None):
    """Runs collection for every layer, aggregation and GPTQ through the ABI.
    inputs: {"x": [bits per layer], "logits": [...]}; jobs: {expert: stored weights}."""
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.calibrate import SharedGroupCalibration

    n = inputs["x"][0].shape[0]
    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, wl.n_shared, max_tokens=n, device=dev())
    cal = SharedGroupCalibration(ctx, list(layers))
    out = {"topk": [], "offsets": [], "token_ids": []}
    for li, l in enumerate(layers):
        x = bits_to_dev(inputs["x"][li])
        lg = to_dev(inputs["logits"][li])
        if chunks == 1:
            tk = torch.empty(n, wl.top_k, dtype=torch.int32, device=dev()) if keep_routing else None
            of = torch.empty(wl.n_routed + 1, dtype=torch.int64, device=dev()) if keep_routing else None
            ti = torch.empty(n * wl.top_k, dtype=torch.int32, device=dev()) if keep_routing else None
            cal.collect(l, x, lg, topk_out=tk, offsets_out=of, token_ids_out=ti)
            if keep_routing:
                out["topk"].append(tk)
                out["offsets"].append(of)
                out["token_ids"].append(ti)
        else:
            bounds = np.linspace(0, n, chunks + 1).astype(int)
            for a, b in zip(bounds[:-1], bounds[1:]):
                cal.collect(l, x[a:b], lg[a:b])
    ctx.sync()
    res = {"ctx": ctx, "cal": cal}
    res["S"] = [cal.S[l].cpu().numpy() for l in layers]
    res["counts"] = [cal.counts[l].cpu().numpy() for l in layers]
    for k in ("topk", "offsets", "token_ids"):
        res[k] = [t.cpu().numpy() for t in out[k]]
    if mode is not None:
        cal.aggregate(mode, alpha=alpha, layers=agg_layers)
        ctx.sync()
        res["H"] = cal.H.cpu().numpy()
        res["alpha"] = cal.alpha.cpu().numpy()
    if jobs:
        wdev = {e: weights_to_dev(wl, w) for e, w in jobs.items()}
        o = cal.quantize(wdev, wl.bits, wl.shared_bits, wl.group, block=block, damp=wl.damp)
        ctx.sync()
        res["gptq"] = {e: {k: v.cpu().numpy() for k, v in d.items()} for e, d in o.items()}
    return res


def agree(a, b) -> float:
    return float(np.mean(np.asarray(a) == np.asarray(b)))


# A rounding of h to bf16 is decided in fp32 on both sides, but the two fp32
# sums (matrix-core order against BLAS order) can differ by a few fp32 ulps, so
# an h within that distance of a bf16 midpoint may round either way.  Every
# value whose fp32 h lies within a relative 2^-16 of a midpoint (16 times the
# fp32 error of a 2048-term sum) is taken as ambiguous: the GPU may hold its
# other neighbour, one bf16 step away.
BF16_TIE_MARGIN = 2.0 ** -16


def down_gram_flip_bound(hb, h32):
    """Largest change of sum_t h_t h_t^T that admissible bf16 flips of the
    ambiguous values can cause, per element (all from the oracle)."""
    hb = np.asarray(hb, np.float64)
    h32 = np.asarray(h32, np.float64)
    m, e = np.frexp(np.where(h32 == 0.0, 1.0, h32))
    step = np.ldexp(1.0, e - 8)                           # bf16 spacing around h
    frac = np.ldexp(np.abs(m), 8)                          # in [128, 256)
    dist = np.abs(frac - np.floor(frac) - 0.5) * step      # distance to the nearest midpoint
    amb = (dist <= BF16_TIE_MARGIN * np.abs(h32)) & (h32 != 0.0)
    A = np.where(amb, step, 0.0)
    H = np.abs(hb)
    return A.T @ H + H.T @ A + A.T @ A


def assert_down_gram(S_gpu, S_ref, bound, label):
    """|S_gpu - S_ref| <= flip bound + HESS_TOL sqrt(S_ii S_jj), elementwise."""
    S_gpu = np.asarray(S_gpu, np.float64)
    d = np.sqrt(np.clip(np.diag(S_ref), 1e-300, None))
    low = np.tril(np.ones_like(S_ref, dtype=bool))
    excess = np.abs(S_gpu - S_ref) - bound - HESS_TOL * np.outer(d, d)
    worst = float(np.max(np.where(low, excess, -np.inf)))
    assert worst <= 0.0, f"{label}: exceeds the bound by {worst:.3e}"


def say(msg):
    print(msg, flush=True)


def slot_rows(x_bits, bucket, slot, n_routed):
    """Token rows (bf16 bits) of one Hessian slot: a routed expert's tokens, or
    every token for the shared slot."""
    counts, offsets, ids = bucket
    if slot < n_routed:
        return x_bits[ids[offsets[slot]:offsets[slot + 1]]]
    return x_bits


def col_sq_sums(x_bits, chunk=16384):
    """sum_t x_tj^2 per column, float64 (the tolerance's normaliser)."""
    out = np.zeros(x_bits.shape[1])
    for t0 in range(0, x_bits.shape[0], chunk):
        x = oracle.bf16_to_f64(x_bits[t0:t0 + chunk])
        out += np.einsum("ti,ti->i", x, x)
    return out


def check_all_slots(H_dev, x_list, buckets, n_routed, slots, mode, seed, n_rows=24, label=""):
    """Every slot's combined Hessian on n_rows sampled rows against the oracle's
    aggregation of the per-layer Gram-sum rows."""
    rng = np.random.default_rng(seed)
    d = H_dev.shape[-1]
    worst = 0.0
    for s in range(slots):
        rows = np.sort(rng.choice(d, n_rows, replace=False))
        S, D, n = [], [], []
        for l, x in enumerate(x_list):
            xs = slot_rows(x, buckets[l], s, n_routed)
            S.append(oracle.gram_rows(xs, rows))
            D.append(col_sq_sums(xs))
            n.append(xs.shape[0])
        R, _ = oracle.aggregate(S, n, mode)
        Rd, _ = oracle.aggregate(D, n, mode)
        G = H_dev[s][torch.from_numpy(rows).to(H_dev.device)].cpu().numpy().astype(np.float64)
        den = np.sqrt(np.outer(Rd[rows], Rd))
        err = float(np.max(np.abs(G - R) / den))
        worst = max(worst, err)
        assert err <= HESS_TOL, f"{label} slot {s}: H_comb error {err:.3e}"
    say(f"{label}: all {slots} slots within {worst:.2e}")


def full_hessian(x_list, buckets, slot, n_routed):
    """Per-layer full Gram sums (float64) and token counts of one slot."""
    S, n = [], []
    for l, x in enumerate(x_list):
        xs = slot_rows(x, buckets[l], slot, n_routed)
        S.append(np.zeros((x.shape[1], x.shape[1])))
        for t0 in range(0, xs.shape[0], 32768):
            S[-1] += oracle.gram(oracle.bf16_to_f64(xs[t0:t0 + 32768]))
        n.append(xs.shape[0])
    return S, n


def check_gptq(wl, w_bits, H_ref, out, bits, label):
    wv = gen.weights_value(wl, w_bits).astype(np.float64)
    ref = oracle.gptq(wv, H_ref, bits, wl.group, wl.damp, wl.block)
    codes = out["codes"].cpu().numpy()
    a = agree(codes, ref["codes"])
    assert a >= CODE_AGREE, f"{label}: codes agree {a:.5f}"
    assert codes.max() <= (1 << bits) - 1
    ok = (codes == ref["codes"]).all(axis=1)
    assert ok.mean() >= 0.9, f"{label}: only {ok.mean():.3f} of the rows agree in every code"
    np.testing.assert_allclose(out["scales"].cpu().numpy()[ok], ref["scales"][ok], rtol=SCALE_RTOL)
    assert (out["zeros"].cpu().numpy()[ok] == ref["zeros"][ok]).all(), label
    want = oracle.loss(wv, ref["wq"], H_ref)
    got = float(out["loss"].cpu().numpy()[0])
    assert abs(got - want) <= LOSS_RTOL * abs(want), f"{label}: loss {got} vs {want}"
    say(f"{label}: codes agree {a:.5f}, loss {got:.6g} vs {want:.6g}")
    return ref, codes
