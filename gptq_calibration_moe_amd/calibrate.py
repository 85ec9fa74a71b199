"""CLHA calibration of one group of layers that share their routed experts.

Host-side orchestration of the three phases of the CLHA summary (section 2.2)
through the C ABI; every arithmetic step runs in the library's kernels.
  collect(layer, x, logits)   phase 1, per layer and batch (layer-aware, section 2.4)
  aggregate(mode)             phase 2, H_comb per expert slot
  quantize(weights, ...)      phase 3, GPTQ per expert on its slot's H_comb,
                              shared experts at b+1 bits under CLHA-MP (section 2.3)
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import Context


class SharedGroupCalibration:
    """Accumulators of n_layers layers sharing one MoE block's experts."""

    def __init__(self, ctx: Context, layer_ids: Sequence[int], H: Optional[torch.Tensor] = None):
        """H: optional [slots, d, d] float32 buffer for H_comb, e.g. one shared by
        groups that are aggregated and quantized one after another."""
        self.ctx = ctx
        self.layer_ids = list(layer_ids)
        self.S, self.counts = {}, {}
        for l in self.layer_ids:
            S, n = ctx.new_layer_buffers()
            ctx.register_layer(l, S, n)
            self.S[l], self.counts[l] = S, n
        self.H = (torch.empty(ctx.slots, ctx.d, ctx.d, dtype=torch.float32, device=ctx.device)
                  if H is None else H)
        self.alpha = torch.empty(ctx.slots, len(self.layer_ids), dtype=torch.float32, device=ctx.device)

    def reset(self):
        """Starts a new accumulation: the next collection of each layer overwrites
        its sums (the library zeroes the counts now and S only where no token lands)."""
        for l in self.layer_ids:
            self.ctx.reset_layer(l)

    def collect(self, layer: int, x: torch.Tensor, logits: torch.Tensor, **kw):
        self.ctx.collect_hessians(layer, x, logits, **kw)

    def aggregate(self, mode: str, alpha: Optional[Sequence[float]] = None,
                  layers: Optional[Sequence[int]] = None):
        ids = self.layer_ids if layers is None else list(layers)
        alpha_out = self.alpha if len(ids) == len(self.layer_ids) else None
        self.ctx.aggregate(ids, mode, self.H, alpha=alpha, alpha_out=alpha_out)
        return self.H

    def slot_of(self, expert: int) -> int:
        return expert if expert < self.ctx.n_routed else self.ctx.n_routed

    def make_outputs(self, experts: Sequence[int], rows: int, group: int):
        d, dev = self.ctx.d, self.ctx.device
        out = {}
        for e in experts:
            out[e] = {
                "codes": torch.empty(rows, d, dtype=torch.uint8, device=dev),
                "scales": torch.empty(rows, d // group, dtype=torch.float32, device=dev),
                "zeros": torch.empty(rows, d // group, dtype=torch.uint8, device=dev),
                "loss": torch.empty(1, dtype=torch.float32, device=dev),
            }
        return out

    def prepare_quantize(self, weights: dict, bits: int, shared_bits: int, group: int,
                         outputs: Optional[dict] = None, H: Optional[torch.Tensor] = None,
                         act_order: bool = False, static_groups: bool = False,
                         workspace: Optional[torch.Tensor] = None):
        """Marshals the GPTQ job batch once; run it with ctx.run_gptq(prep, group, ...).
        act_order / static_groups select GPTQ's activation-order and static-group options;
        workspace may be shared with other batches run on the same stream."""
        H = self.H if H is None else H
        experts = sorted(weights)
        rows = weights[experts[0]].shape[0]
        if outputs is None:
            outputs = self.make_outputs(experts, rows, group)
        jobs = [{"H": H[self.slot_of(e)], "W": weights[e],
                 "bits": shared_bits if e >= self.ctx.n_routed else bits, **outputs[e]}
                for e in experts]
        return self.ctx.prepare_gptq(jobs, self.ctx.d, act_order, static_groups, workspace), outputs

    def quantize_jobs(self, weights: dict, bits: int, shared_bits: int, outputs: dict,
                      H: Optional[torch.Tensor] = None) -> list:
        """The job dicts of a GPTQ batch (each expert on its slot's H_comb, shared
        experts at shared_bits), e.g. to size a workspace shared by several batches."""
        H = self.H if H is None else H
        return [{"H": H[self.slot_of(e)], "W": weights[e],
                 "bits": shared_bits if e >= self.ctx.n_routed else bits, **outputs[e]}
                for e in sorted(weights)]

    def quantize(self, weights: dict, bits: int, shared_bits: int, group: int, block: int = 128,
                 damp: float = 0.01, outputs: Optional[dict] = None, H: Optional[torch.Tensor] = None,
                 act_order: bool = False, static_groups: bool = False):
        """weights: {expert: W [rows, d] float32 or bfloat16}.  Routed expert e uses
        H[e]; shared experts (e >= E) use H[E] and shared_bits."""
        H = self.H if H is None else H
        experts = sorted(weights)
        rows = weights[experts[0]].shape[0]
        if outputs is None:
            outputs = self.make_outputs(experts, rows, group)
        jobs = []
        for e in experts:
            o = outputs[e]
            jobs.append({"H": H[self.slot_of(e)], "W": weights[e],
                         "bits": shared_bits if e >= self.ctx.n_routed else bits, **o})
        self.ctx.gptq_quantize(jobs, self.ctx.d, group, block, damp, act_order=act_order,
                               static_groups=static_groups)
        return outputs


def storage_bits(rows: int, cols: int, bits: int, group: int, scale_bits: int = 32, zero_bits: int = 8) -> int:
    """Bits of one quantized matrix in packed storage: rows*cols codes of `bits`
    bits plus one scale and one zero point per (row, group)."""
    return rows * cols * bits + rows * (cols // group) * (scale_bits + zero_bits)


def mixed_precision_overhead(jobs, group: int, scale_bits: int = 32, zero_bits: int = 8) -> dict:
    """CLHA-MP accounting (section 2.3): `jobs` is a sequence of (rows, cols,
    bits, base_bits); returns the packed bits per parameter with each job at its
    own width, the same at every job's base width, and the relative overhead."""
    params = sum(r * c for r, c, _, _ in jobs)
    mixed = sum(storage_bits(r, c, b, group, scale_bits, zero_bits) for r, c, b, _ in jobs)
    base = sum(storage_bits(r, c, b0, group, scale_bits, zero_bits) for r, c, _, b0 in jobs)
    return {"bits_per_param": mixed / params, "base_bits_per_param": base / params,
            "overhead": mixed / base - 1.0}
