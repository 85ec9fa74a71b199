"""Experiments of the CLHA summary, section 4, on one CLWS pair.

sharpness_sweep: the routing-divergence experiment: how far the two layers'
routing diverges as the router is sharpened or flattened, and how the
quantization loss of PLIC, CLHA-rt and CLHA-eq behaves under each layer's own
Hessian as it does.
drift_sweep: the same losses as layer b's activations drift away from layer
a's (the calibration-Hessian error under each layer's Hessian, and the
combined objective).

Host-side orchestration; every arithmetic step of the calibration runs in the
library's kernels.  The two divergence measures are small host computations on
the routing the library returns:
  load_divergence   Jensen-Shannon divergence (natural log) of the layers'
                    expert-load distributions n_e / sum n
  topk_overlap      mean over tokens of the fraction of experts chosen in both layers
"""
from __future__ import annotations

from typing import Callable, Sequence

import numpy as np
import torch

from .calibrate import SharedGroupCalibration


def load_divergence(counts_a, counts_b) -> float:
    p = np.asarray(counts_a, np.float64)
    q = np.asarray(counts_b, np.float64)
    p, q = p / p.sum(), q / q.sum()
    m = 0.5 * (p + q)
    with np.errstate(divide="ignore", invalid="ignore"):
        kp = np.where(p > 0, p * np.log(p / m), 0.0).sum()
        kq = np.where(q > 0, q * np.log(q / m), 0.0).sum()
    return float(0.5 * (kp + kq))


def topk_overlap(topk_a, topk_b) -> float:
    a = np.sort(np.asarray(topk_a), axis=1)
    b = np.sort(np.asarray(topk_b), axis=1)
    k = a.shape[1]
    hits = (a[:, :, None] == b[:, None, :]).any(axis=2).sum(axis=1)
    return float(hits.mean() / k)


def sharpness_sweep(ctx, x: Sequence[torch.Tensor], logits_for: Callable[[float], Sequence[torch.Tensor]],
                    taus: Sequence[float], weights: dict, bits: int, group: int, block: int = 128,
                    damp: float = 0.01) -> list:
    """For each tau: route and collect both layers with logits_for(tau), combine
    under PLIC (alpha = (1, 0)), CLHA-rt and CLHA-eq, quantize `weights`
    ({routed expert: W}) under each, and measure every result's loss under the
    layer-a and layer-b Hessians.  Returns one dict per tau."""
    cal = SharedGroupCalibration(ctx, [0, 1])
    E, K, d, dev = ctx.n_routed, ctx.top_k, ctx.d, ctx.device
    H_layer = [torch.empty(ctx.slots, d, d, dtype=torch.float32, device=dev) for _ in range(2)]
    rows = []
    for tau in taus:
        lg = logits_for(tau)
        topk = [torch.empty(x[l].shape[0], K, dtype=torch.int32, device=dev) for l in range(2)]
        cal.reset()
        for l in range(2):
            cal.collect(l, x[l], lg[l], topk_out=topk[l])
        for l in range(2):
            cal.aggregate("explicit", alpha=[1.0], layers=[l])
            H_layer[l].copy_(cal.H)
        counts = [cal.counts[l].cpu().numpy()[:E] for l in range(2)]
        row = {"tau": float(tau), "load_divergence": load_divergence(*counts),
               "topk_overlap": topk_overlap(topk[0].cpu().numpy(), topk[1].cpu().numpy())}
        for name, mode, alpha in (("plic", "explicit", [1.0, 0.0]), ("rt", "rt", None), ("eq", "eq", None)):
            cal.aggregate(mode, alpha=alpha)
            out = cal.quantize(weights, bits, bits, group, block=block, damp=damp)
            for l, tag in ((0, "a"), (1, "b")):
                total = 0.0
                for e, w in weights.items():
                    o = out[e]
                    got = torch.empty(1, dtype=torch.float32, device=dev)
                    ctx.loss(w, o["codes"], o["scales"], o["zeros"], H_layer[l][e], group, got)
                    total += float(got.cpu()[0])
                row[f"loss_{name}_{tag}"] = total
        rows.append(row)
    return rows


def _quantize_and_score(ctx, cal, H, H_a, H_b, weights: dict, bits: int, group: int, block: int,
                        damp: float) -> dict:
    """GPTQ of every weight on its slot of H in one batch; returns the sums over
    the weights of the loss under H (the combined objective), under layer a's
    Hessian (each job's second Hessian) and under layer b's (the explicit loss
    entry point)."""
    dev = ctx.device
    outputs = cal.make_outputs(sorted(weights), next(iter(weights.values())).shape[0], group)
    jobs = []
    for e in sorted(weights):
        o = outputs[e]
        o["H_eval"] = H_a[e]
        o["loss_eval"] = torch.empty(1, dtype=torch.float32, device=dev)
        o["status"] = torch.empty(1, dtype=torch.int32, device=dev)
        jobs.append({"H": H[e], "W": weights[e], "bits": bits, **o})
    ctx.gptq_quantize(jobs, ctx.d, group, block, damp)
    loss_b = []
    for e, j in zip(sorted(weights), jobs):
        lb = torch.empty(1, dtype=torch.float32, device=dev)
        ctx.loss(weights[e], j["codes"], j["scales"], j["zeros"], H_b[e], group, lb)
        loss_b.append(lb)
    ctx.sync()
    if any(int(j["status"].cpu()[0]) != 0 for j in jobs):
        raise RuntimeError("a GPTQ job of the sweep failed")
    return {"comb": float(sum(float(j["loss"].cpu()[0]) for j in jobs)),
            "a": float(sum(float(j["loss_eval"].cpu()[0]) for j in jobs)),
            "b": float(sum(float(lb.cpu()[0]) for lb in loss_b))}


def drift_sweep(ctx, inputs_for: Callable[[float], tuple], ts: Sequence[float], weights: dict, bits: int,
                group: int, block: int = 128, damp: float = 0.01) -> list:
    """For each drift t: inputs_for(t) gives (x_a, x_b, logits_a, logits_b) on the
    device; collect both layers, combine under PLIC (layer a's Hessian), CLHA-rt
    and CLHA-eq, quantize every weight ({routed expert: W}) under each, and sum
    each result's loss under the combined Hessian and under each layer's own.
    Also the routing divergence of the two layers.  Returns one dict per t."""
    cal = SharedGroupCalibration(ctx, [0, 1])
    E, K, d, dev = ctx.n_routed, ctx.top_k, ctx.d, ctx.device
    H_a, H_b, H_rt, H_eq = (torch.empty(ctx.slots, d, d, dtype=torch.float32, device=dev) for _ in range(4))
    rows = []
    for t in ts:
        xa, xb, la, lb = inputs_for(t)
        topk = [torch.empty(xa.shape[0], K, dtype=torch.int32, device=dev) for _ in range(2)]
        cal.reset()
        cal.collect(0, xa, la, topk_out=topk[0])
        cal.collect(1, xb, lb, topk_out=topk[1])
        ctx.aggregate([0], "explicit", H_a, alpha=[1.0])
        ctx.aggregate([1], "explicit", H_b, alpha=[1.0])
        ctx.aggregate([0, 1], "rt", H_rt)
        ctx.aggregate([0, 1], "eq", H_eq)
        counts = [cal.counts[l].cpu().numpy()[:E] for l in range(2)]
        row = {"t": float(t), "load_divergence": load_divergence(*counts),
               "topk_overlap": topk_overlap(topk[0].cpu().numpy(), topk[1].cpu().numpy())}
        for name, H in (("plic", H_a), ("rt", H_rt), ("eq", H_eq)):
            r = _quantize_and_score(ctx, cal, H, H_a, H_b, weights, bits, group, block, damp)
            for k, v in r.items():
                row[f"loss_{name}_{k}"] = v
        rows.append(row)
    return rows
