"""Seeded synthetic inputs for CLHA calibration (Cross-Layer Hessian Aggregation).

This module only draws random numbers and stores them in the formats the
calibration path consumes (bf16 bit patterns as uint16, fp32).  It holds none
of the method's arithmetic: no routing, no Gram sums, no aggregation, no GPTQ.
Both the CPU oracle (``oracle/``) and the GPU path consume the arrays it
returns, so the two sides always see identical inputs.

Workloads.  The CLHA summary ("CLHA - Cross-Layer Hessian Aggregation ...",
section 4) measures a 34.5M-parameter CLWS-MoE trained on WikiText-2.  Neither
the trained weights nor the dataset are available, so five synthetic
workloads stand in for it (their shapes are listed in ``WORKLOADS``):

1. tiny CLWS pair      - d=256, 8 routed experts, top-2, W fp32 512x256
2. mid MoE block       - d=2048, 64 routed + 2 shared experts, top-6,
                         gate/up bf16 1408x2048, Student-t(4) activations
3. full depth          - 12 CLWS pairs of config-2 shapes, Zipf(1.1) router load
4. CLHA-MP             - config 3's arrays, shared experts at b+1 bits
5. drift stress        - d=4096, 128 routed experts, top-8, layer-b activations
                         drifting from layer a by t in {0, .25, .5, .75, 1}

Random streams are addressed, not spawned in order:
``SeedSequence(seed_base + workload_id, spawn_key=(pair, stream, index))``,
so a subset of experts or pairs can be generated without drawing the rest.
Activations and router logits are drawn in chunks of 16,384 rows, chunk i
from index i of its stream, on a pool of host threads; an array of at most
16,384 rows is one chunk.

bf16 values are made from fp32 by round-to-nearest-even and stored as the
upper 16 bits of the fp32 pattern (uint16).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

# stream ids inside one pair's key space
_S_XA, _S_XB, _S_ROT, _S_LA, _S_LB, _S_PERM_A, _S_PERM_B, _S_W, _S_ROUTER, _S_Z = range(10)


@dataclass(frozen=True)
class Workload:
    """Shape sheet of one synthetic calibration workload (one or more CLWS pairs)."""

    wid: int                 # workload id (1..5) or a derived id for test shapes
    name: str
    d: int                   # hidden size = columns of every calibrated matrix
    n_routed: int            # E, routed experts shared by the pair
    top_k: int               # K, experts chosen per token
    n_shared: int            # always-active shared experts (one Hessian slot for all)
    n_tokens: int            # N, calibration tokens per layer
    n_pairs: int             # CLWS pairs (2 layers each)
    rows: int                # rows of one calibrated matrix
    mats: tuple              # matrices per expert stacked into one GPTQ job
    w_dtype: str             # 'f32' or 'bf16'
    bits: int                # b for routed experts
    shared_bits: int         # bits for the always-active shared experts (b or b+1)
    group: int               # quantization group size g
    alpha: str               # 'rt' (routing frequency) or 'eq' (0.5)
    x_kind: str              # 'rotated' | 'student_t' | 'drift' | 'normal'
    logit_kind: str          # 'normal' | 'zipf' | 'router'
    damp: float = 0.01
    block: int = 128
    drift: tuple = ()
    seed_base: int = 1000

    @property
    def job_rows(self) -> int:
        """Rows of one GPTQ job: the expert's matrices stacked (gate over up)."""
        return self.rows * len(self.mats)

    @property
    def n_slots(self) -> int:
        """Hessian slots per layer: E routed plus one shared-input slot if any."""
        return self.n_routed + (1 if self.n_shared > 0 else 0)

    @property
    def n_experts_total(self) -> int:
        return self.n_routed + self.n_shared

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny_clws_pair", d=256, n_routed=8, top_k=2, n_shared=0,
                n_tokens=4096, n_pairs=1, rows=512, mats=("W",), w_dtype="f32",
                bits=2, shared_bits=2, group=128, alpha="rt",
                x_kind="rotated", logit_kind="normal"),
    2: Workload(2, "mid_moe_block", d=2048, n_routed=64, top_k=6, n_shared=2,
                n_tokens=65536, n_pairs=1, rows=1408, mats=("gate", "up"),
                w_dtype="bf16", bits=3, shared_bits=3, group=128, alpha="rt",
                x_kind="student_t", logit_kind="normal"),
    3: Workload(3, "full_depth", d=2048, n_routed=64, top_k=6, n_shared=2,
                n_tokens=262144, n_pairs=12, rows=1408, mats=("gate", "up"),
                w_dtype="bf16", bits=2, shared_bits=2, group=128, alpha="eq",
                x_kind="rotated", logit_kind="zipf"),
    4: Workload(4, "clha_mp", d=2048, n_routed=64, top_k=6, n_shared=2,
                n_tokens=262144, n_pairs=12, rows=1408, mats=("gate", "up"),
                w_dtype="bf16", bits=2, shared_bits=3, group=128, alpha="rt",
                x_kind="rotated", logit_kind="zipf", seed_base=1000 - 1),
    5: Workload(5, "drift_stress", d=4096, n_routed=128, top_k=8, n_shared=0,
                n_tokens=262144, n_pairs=1, rows=2048, mats=("W",), w_dtype="bf16",
                bits=2, shared_bits=2, group=64, alpha="rt",
                x_kind="drift", logit_kind="router", drift=(0.0, 0.25, 0.5, 0.75, 1.0)),
}
# Workload 4 reuses workload 3's seeds (seed_base + wid equal): identical arrays.
assert WORKLOADS[4].seed_base + 4 == WORKLOADS[3].seed_base + 3


CHUNK_ROWS = 16384      # rows per independently seeded chunk of a row-major stream
_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def _by_chunks(n: int, fill) -> None:
    """Runs fill(lo, hi, i) for the row chunks [i*CHUNK_ROWS, ...) of an n-row
    array on the thread pool (numpy's generators and ufuncs release the GIL)."""
    bounds = [(lo, min(lo + CHUNK_ROWS, n), i) for i, lo in enumerate(range(0, n, CHUNK_ROWS))]
    for f in [_pool().submit(fill, *b) for b in bounds]:
        f.result()


# --------------------------------------------------------------------------- formats

def bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """bf16 bit pattern (uint16) -> fp32 value (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(wl: Workload, pair: int, stream: int, index: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=wl.seed_base + wl.wid, spawn_key=(pair, stream, index))
    return np.random.Generator(np.random.PCG64(ss))


def _haar_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    g = rng.standard_normal((d, d))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def _student_t_f32(rng, shape, nu: float) -> np.ndarray:
    """Student-t(nu) in float32 as Z * sqrt(nu / chi2_nu), chi2_nu = 2 Gamma(nu/2)."""
    z = rng.standard_normal(shape, dtype=np.float32)
    g = rng.standard_gamma(np.float32(nu / 2.0), shape, dtype=np.float32)
    z *= np.sqrt(np.float32(nu / 2.0) / g)
    return z


def _normal_f32(rng, shape, scale=1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


# --------------------------------------------------------------------------- activations

def activations(wl: Workload, pair: int = 0, t: Optional[float] = None,
                n_tokens: Optional[int] = None):
    """Layer-a and layer-b activations of one CLWS pair as bf16 bits [N, d].

    rotated:   X_a ~ N(0,1); X_b = X_a Q + 0.3 N(0,1), Q Haar orthogonal.
    student_t: X_a, X_b independent Student-t(nu=4).
    drift:     X_a ~ N(0,1); X_b = (1-t) X_a + t Z, Z ~ N(0,1) independent.
    normal:    X_a, X_b independent N(0,1).
    """
    n = wl.n_tokens if n_tokens is None else n_tokens
    d = wl.d
    xa = np.empty((n, d), np.uint16)
    xb = np.empty((n, d), np.uint16)
    if wl.x_kind == "rotated":
        def fa(lo, hi, i):
            xa[lo:hi] = bf16_bits(_normal_f32(_rng(wl, pair, _S_XA, i), (hi - lo, d)))
        _by_chunks(n, fa)
        q = _haar_orthogonal(_rng(wl, pair, _S_ROT), d).astype(np.float32)
        m = bf16_value(xa) @ q

        def fb(lo, hi, i):
            xb[lo:hi] = bf16_bits(m[lo:hi] + _normal_f32(_rng(wl, pair, _S_XB, i), (hi - lo, d), 0.3))
        _by_chunks(n, fb)
        del m
    elif wl.x_kind == "student_t":
        def fs(lo, hi, i):
            xa[lo:hi] = bf16_bits(_student_t_f32(_rng(wl, pair, _S_XA, i), (hi - lo, d), 4.0))
            xb[lo:hi] = bf16_bits(_student_t_f32(_rng(wl, pair, _S_XB, i), (hi - lo, d), 4.0))
        _by_chunks(n, fs)
    elif wl.x_kind == "drift":
        if t is None:
            raise ValueError("drift workload needs t")

        def fd(lo, hi, i):
            xa[lo:hi] = bf16_bits(_normal_f32(_rng(wl, pair, _S_XA, i), (hi - lo, d)))
            z = _normal_f32(_rng(wl, pair, _S_Z, i), (hi - lo, d))
            xb[lo:hi] = bf16_bits(np.float32(1.0 - t) * bf16_value(xa[lo:hi]) + np.float32(t) * z)
        _by_chunks(n, fd)
    elif wl.x_kind == "normal":
        def fn(lo, hi, i):
            xa[lo:hi] = bf16_bits(_normal_f32(_rng(wl, pair, _S_XA, i), (hi - lo, d)))
            xb[lo:hi] = bf16_bits(_normal_f32(_rng(wl, pair, _S_XB, i), (hi - lo, d)))
        _by_chunks(n, fn)
    else:
        raise ValueError(wl.x_kind)
    return xa, xb


def router_logits(wl: Workload, pair: int, layer: int, x_bits: Optional[np.ndarray] = None,
                  n_tokens: Optional[int] = None) -> np.ndarray:
    """Router logits [N, E] fp32 for layer 0 (a) or 1 (b) of a pair.

    normal: i.i.d. N(0,1).
    zipf:   log p_{pi(e)} + Gumbel(0,1), p_k proportional to k^-1.1, pi a random
            permutation per layer (top-K of these is a Zipf-weighted sample
            without replacement).
    router: fp32(X R) computed in fp64, R ~ N(0, 1/d) [d, E] shared by the pair.
    """
    n = wl.n_tokens if n_tokens is None else n_tokens
    e = wl.n_routed
    stream = _S_LA if layer == 0 else _S_LB
    if wl.logit_kind == "normal":
        out = np.empty((n, e), np.float32)

        def fn(lo, hi, i):
            out[lo:hi] = _normal_f32(_rng(wl, pair, stream, i), (hi - lo, e))
        _by_chunks(n, fn)
        return out
    if wl.logit_kind == "zipf":
        perm = _rng(wl, pair, _S_PERM_A if layer == 0 else _S_PERM_B).permutation(e)
        logp = -1.1 * np.log(np.arange(1, e + 1, dtype=np.float64))
        logp -= np.log(np.exp(logp).sum())
        out = np.empty((n, e), np.float32)

        def fz(lo, hi, i):
            u = _rng(wl, pair, stream, i).random((hi - lo, e))
            out[lo:hi] = (logp[perm][None, :] - np.log(-np.log(u))).astype(np.float32)
        _by_chunks(n, fz)
        return out
    if wl.logit_kind == "router":
        if x_bits is None:
            raise ValueError("router logits need the layer's activations")
        r = _rng(wl, pair, _S_ROUTER).standard_normal((wl.d, e)) / np.sqrt(wl.d)
        out = np.empty((x_bits.shape[0], e), np.float32)
        step = 16384
        for i in range(0, x_bits.shape[0], step):
            out[i:i + step] = (bf16_value(x_bits[i:i + step]).astype(np.float64) @ r).astype(np.float32)
        return out
    raise ValueError(wl.logit_kind)


def sharpness_logits(wl: Workload, pair: int, layer: int, x_bits: np.ndarray, tau: float,
                     base: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits of the routing-sharpness sweep: x R / tau + Gumbel(0, 1), with
    R ~ N(0, 1/d) [d, E] shared by the pair and the Gumbel noise drawn per layer.
    Top-K of these logits is a sample without replacement from softmax(x R / tau),
    so tau sets how sharp routing is: small tau follows x R in both layers, large
    tau makes the two layers' choices independent.  fp32 [N, E].  `base`, when
    given, is the x R of these activations (router_logits with the router
    kind), reused across tau."""
    if base is None:
        base = router_logits(wl.scaled(logit_kind="router"), pair, layer, x_bits)
    u = _rng(wl, pair, _S_LA if layer == 0 else _S_LB).random(base.shape)
    return (base.astype(np.float64) / tau - np.log(-np.log(u))).astype(np.float32)


# --------------------------------------------------------------------------- weights

def expert_weights(wl: Workload, pair: int, expert: int) -> np.ndarray:
    """Stacked weights of one expert's GPTQ job, [job_rows, d], N(0, 0.02^2).

    Experts 0..E-1 are routed, E..E+n_shared-1 the always-active shared experts.
    Returns fp32 values (w_dtype 'f32') or bf16 bits as uint16 (w_dtype 'bf16').
    """
    w = _normal_f32(_rng(wl, pair, _S_W, expert), (wl.job_rows, wl.d), 0.02)
    return w if wl.w_dtype == "f32" else bf16_bits(w)


def all_expert_weights(wl: Workload, pair: int, experts) -> dict:
    """expert_weights of several experts, drawn on the thread pool: {expert: W}."""
    experts = list(experts)
    futs = [_pool().submit(expert_weights, wl, pair, e) for e in experts]
    return {e: f.result() for e, f in zip(experts, futs)}


def weights_value(wl: Workload, w: np.ndarray) -> np.ndarray:
    """Stored weights -> fp32 values (identity for fp32, exact widening for bf16)."""
    return w if wl.w_dtype == "f32" else bf16_value(w)


def pair_inputs(wl: Workload, pair: int = 0, t: Optional[float] = None,
                n_tokens: Optional[int] = None) -> dict:
    """Activations and router logits of both layers of one CLWS pair."""
    xa, xb = activations(wl, pair, t=t, n_tokens=n_tokens)
    la = router_logits(wl, pair, 0, xa, n_tokens)
    if wl.logit_kind == "router":
        lb = router_logits(wl, pair, 1, xb, n_tokens)
    else:
        lb = router_logits(wl, pair, 1, None, n_tokens)
    return {"x": [xa, xb], "logits": [la, lb]}


def swiglu_weights(seed: int, slots: int, f: int, d: int, scale: float = 0.02) -> list:
    """Gate and up weights of `slots` experts, each [2f, d] bf16 bits: rows 0..f-1
    gate, rows f..2f-1 up, N(0, scale^2) (the configs' N(0, 0.02))."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return [bf16_bits(_normal_f32(rng, (2 * f, d), scale)) for _ in range(slots)]


def structured_activations(seed: int, n: int, d: int, log_spread: float = 3.0,
                           dead_cols=()) -> np.ndarray:
    """Correlated activations X = Z diag(s) Q (s log-uniform over 10^[-spread/2, spread/2]),
    optionally with all-zero ("dead") input columns.  Makes GPTQ's error
    propagation matter, unlike the near-isotropic workloads.  bf16 bits [n, d]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    s = 10.0 ** rng.uniform(-log_spread / 2, log_spread / 2, d)
    q = _haar_orthogonal(rng, d)
    x = (rng.standard_normal((n, d)) * s[None, :]) @ q
    x = x.astype(np.float32)
    for c in dead_cols:
        x[:, c] = 0.0
    return bf16_bits(x)
