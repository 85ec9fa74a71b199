"""Plain CPU oracle of the CLHA calibration path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the GPU
library (``gptq_calibration_moe_amd``); the two meet only in the seeded input
generator ``gen``, which holds none of the method's arithmetic.

Sources.  "CLHA - Cross-Layer Hessian Aggregation for quantizing
weight-shared MoE transformers" (gist.science summary, Dutch page, with the
Chinese page as a second witness):
  * section 2.1 - objective L(W_q) = sum_i alpha_i tr[(W_q-W) H_i (W_q-W)^T],
    H_i the activation covariance of layer i, alpha_i the routing frequency;
    Proposition 1: minimising L is GPTQ with H_comb = sum_i alpha_i H_i;
    PLIC uses the primary layer's H alone.
  * section 2.2 - collection of per-layer Hessians and token counts for every
    active expert; aggregation per shared pair with alpha = n_a/(n_a+n_b)
    ("rt") or alpha = 0.5 ("eq"); quantization by standard GPTQ
    column-sequential updates on H_comb.
  * section 2.3 - CLHA-MP: always-active shared experts see all N tokens and
    get b+1 bits.
  * section 2.4 - accumulators keyed by layer, not by the shared module.
The pages leave everything inside "standard GPTQ" open.  Those steps follow
the published GPTQ algorithm (Frantar et al., ICLR 2023): relative damping,
the upper Cholesky factor of the inverse Hessian, column-sequential
quantize-and-propagate with lazy block updates, min-max asymmetric groups.

Precision.  Everything is float64, except the quantizer's integer decisions
(scale, zero point, code), which are taken in float32 -- the precision the GPU
kernels take them in -- so a code is decided identically from the same
weight value on both sides.

Readings of silent points (each is a stated choice, not a page fact):
  * H_l = S_l / n_l with S_l the raw Gram sum sum_t x_t x_t^T (uncentred,
    per token); rt aggregation = (S_a + S_b)/(n_a + n_b).
  * top-K order: larger logit first, ties to the lower expert index.
  * shared experts: one Hessian slot per layer over all N tokens.
  * dead columns (H_ii == 0): H_ii := 1 and W[:, i] := 0.
  * damping: lambda = damp * mean(diag H) after the dead fix.
  * group statistics computed at each group's first column from the updated
    weights; natural column order; the group size divides the block size.
    Two common GPTQ options are also offered: activation order (columns by
    decreasing H_ii, dead columns counted as 1, ties by index; groups are
    runs of processed columns) and static groups (every natural group's grid
    fitted once on the weights after the dead fix, before any update).
  * quantizer grid: range widened to contain 0, an all-zero group uses
    (-1, 1); s = (max - min)/maxq, z = rint(-min/s); rint ties to even.
  * an empty layer (n = 0) drops out of the combination; if every layer is
    empty the combined Hessian is the identity.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64", "route", "bucket", "gram", "gram_rows", "layer_hessians", "aggregate",
    "inverse_cholesky_upper", "quant_params", "quantize", "gptq", "dequantize",
    "dequantize_idx", "act_order_perm",
    "loss", "calibrate_pair",
]


# --------------------------------------------------------------------------- inputs

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- collection

def route(logits, k: int) -> np.ndarray:
    """Top-K experts per token (CLHA section 2.2, "active experts"; section 2.3,
    routed experts see a K/E fraction of tokens).

    For each token the experts are ordered by (logit descending, index
    ascending) and the first K are kept.  Returns [N, K] int32.
    """
    lg = np.asarray(logits, dtype=np.float32)
    n, e = lg.shape
    if not 1 <= k <= e:
        raise ValueError("need 1 <= K <= E")
    if not np.all(np.isfinite(lg)):
        raise ValueError("non-finite router logit")
    key_idx = np.broadcast_to(np.arange(e), (n, e))
    order = np.lexsort((key_idx, -lg.astype(np.float64)), axis=-1)
    return order[:, :k].astype(np.int32)


def bucket(topk, n_experts: int):
    """Token lists per expert (CLHA section 2.2, per-expert token counts).

    counts[e] = number of tokens that chose e; offsets = exclusive prefix sum;
    token_ids lists, for each expert in turn, its tokens in ascending order.
    """
    tk = np.asarray(topk, dtype=np.int64)
    n, k = tk.shape
    flat = tk.ravel()
    tok = np.repeat(np.arange(n, dtype=np.int64), k)
    order = np.lexsort((tok, flat))
    counts = np.bincount(flat, minlength=n_experts).astype(np.int64)
    offsets = np.zeros(n_experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    return counts, offsets, tok[order].astype(np.int32)


def gram(x) -> np.ndarray:
    """S = X^T X in float64 (raw activation Gram sum of one expert's tokens)."""
    x64 = np.asarray(x, dtype=np.float64)
    return x64.T @ x64


def gram_rows(x_bits, rows, chunk: int = 16384) -> np.ndarray:
    """Rows `rows` of the Gram sum S = X^T X of bf16 activations, in float64:
    S[i, j] = sum_t x_ti x_tj for i in rows and every j.  Tokens are taken in
    chunks of `chunk` rows only to bound memory; every product of two bf16
    values is exact in float64."""
    xb = np.asarray(x_bits, dtype=np.uint16)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, xb.shape[1]))
    for t0 in range(0, xb.shape[0], chunk):
        x = bf16_to_f64(xb[t0:t0 + chunk])
        out += x[:, rows].T @ x
    return out


def layer_hessians(x_bits, topk, n_routed: int, n_shared: int, slots=None):
    """Per-layer Gram sums and token counts (CLHA section 2.2, collection).

    Slots 0..E-1 are the routed experts (their routed tokens); slot E, present
    when n_shared > 0, is the shared-expert input over all N tokens (section
    2.3: shared experts receive every token).  Returns ({slot: S}, counts).
    """
    x = bf16_to_f64(x_bits)
    n = x.shape[0]
    counts, offsets, ids = bucket(topk, n_routed)
    n_slots = n_routed + (1 if n_shared > 0 else 0)
    all_counts = np.zeros(n_slots, np.int64)
    all_counts[:n_routed] = counts
    if n_shared > 0:
        all_counts[n_routed] = n
    if slots is None:
        slots = range(n_slots)
    out = {}
    for s in slots:
        if s < n_routed:
            out[s] = gram(x[ids[offsets[s]:offsets[s + 1]]])
        else:
            out[s] = gram(x)
    return out, all_counts


def round_bf16(v) -> np.ndarray:
    """Nearest bf16 value (8 significant bits), ties to even, from fp64; returns
    fp64 values.  Zero stays zero; the bf16 subnormal range is not needed here."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                       # v = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def silu(g) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + e^-g), in the precision of g."""
    g = np.asarray(g)
    one = g.dtype.type(1) if np.issubdtype(g.dtype, np.floating) else 1.0
    return g / (one + np.exp(-g))


def swiglu_intermediate(x_bits, wgu_bits, f: int, with_fp32: bool = False):
    """The input of an expert's down_proj (CLHA section 2.2 collects every shared
    weight's Hessian over its own input): h = bf16(silu(x Wg^T) * (x Wu^T)) with
    Wg = rows 0..f-1 and Wu = rows f..2f-1 of the stacked [2f, d] weight.

    Rounding h to bf16 is a discrete decision taken by floating point, so it is
    taken in the kernel's precision: g and u are fp32 sums of the (exact) bf16
    products, silu and the product are fp32, and that fp32 h is rounded to the
    nearest bf16 (ties to even).  Returns fp64 values of the bf16 h (and, with
    with_fp32, the fp32 h before rounding)."""
    x = bf16_to_f64(x_bits).astype(np.float32)
    w = bf16_to_f64(wgu_bits).astype(np.float32)
    g = x @ w[:f].T
    u = x @ w[f:].T
    h = (silu(g) * u).astype(np.float32)
    hb = round_bf16(h.astype(np.float64))
    return (hb, h.astype(np.float64)) if with_fp32 else hb


def down_layer_hessians(x_bits, topk, wgu_list, n_routed: int, f: int, slots=None):
    """Per-layer Gram sums of the down_proj inputs: slot e < n_routed over expert
    e's routed tokens with its weights, slot n_routed + s over all tokens with
    shared expert s's weights.  Returns ({slot: S}, counts)."""
    n = np.asarray(x_bits).shape[0]
    counts, offsets, ids = bucket(topk, n_routed)
    n_slots = len(wgu_list)
    all_counts = np.zeros(n_slots, np.int64)
    all_counts[:n_routed] = counts
    all_counts[n_routed:] = n
    out = {}
    for s in (range(n_slots) if slots is None else slots):
        rows = np.asarray(x_bits)[ids[offsets[s]:offsets[s + 1]]] if s < n_routed else np.asarray(x_bits)
        out[s] = gram(swiglu_intermediate(rows, wgu_list[s], f)) if len(rows) else np.zeros((f, f))
    return out, all_counts


def aggregate(S_list, n_list, mode: str, alpha=None):
    """Combined Hessian of one shared weight (CLHA section 2.1 Proposition 1;
    section 2.2 aggregation).

    mode 'rt':       H = sum_i S_i / sum_i n_i, i.e. alpha_i = n_i / sum n.
    mode 'eq':       H = sum_i (1/m) S_i/n_i over the m non-empty layers.
    mode 'explicit': H = sum_i alpha_i S_i/n_i (alpha renormalised over the
                     non-empty layers if some weighted layer is empty).
    A single layer (PLIC) is any mode with one entry: H = S/n.
    The S_i may also be matching slices of the Gram sums (rows, or a diagonal):
    every step is elementwise.
    Returns (H, alpha_used).  All layers empty -> (I, zeros).
    """
    n = np.asarray(n_list, dtype=np.int64)
    d = S_list[0].shape[0]
    m = len(S_list)
    if n.sum() == 0:
        return np.eye(d), np.zeros(m)
    if mode == "rt":
        total = float(n.sum())
        H = sum(np.asarray(S, np.float64) for S in S_list) / total
        return H, n / total
    if mode == "eq":
        a = np.where(n > 0, 1.0, 0.0)
        a = a / a.sum()
    elif mode == "explicit":
        a = np.asarray(alpha, np.float64).copy()
        if a.shape != (m,):
            raise ValueError("alpha needs one weight per layer")
        lost = bool(np.any((a != 0.0) & (n == 0)))
        a = np.where(n > 0, a, 0.0)
        if lost:
            if a.sum() == 0.0:
                return np.eye(d), np.zeros(m)
            a = a / a.sum()
    else:
        raise ValueError(mode)
    H = np.zeros(np.shape(S_list[0]))
    for ai, S, ni in zip(a, S_list, n):
        if ni > 0 and ai != 0.0:
            H += ai * (np.asarray(S, np.float64) / float(ni))
    return H, a


# --------------------------------------------------------------------------- GPTQ

def inverse_cholesky_upper(H) -> np.ndarray:
    """U upper triangular with positive diagonal and U^T U = H^-1 (GPTQ's
    "Cholesky of H^-1"), written as its definition."""
    Hinv = np.linalg.inv(np.asarray(H, np.float64))
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T


def quant_params(x, maxq: int):
    """Per-row asymmetric min-max grid of one group, decided in float32.

    x: [rows, g] weights.  Returns (scale, zero) as float32 arrays; zero holds
    integer values in [0, maxq].
    """
    x32 = np.asarray(x, dtype=np.float32)
    xmin = np.minimum(x32.min(axis=1), np.float32(0))
    xmax = np.maximum(x32.max(axis=1), np.float32(0))
    empty = (xmin == 0) & (xmax == 0)
    xmin = np.where(empty, np.float32(-1), xmin).astype(np.float32)
    xmax = np.where(empty, np.float32(1), xmax).astype(np.float32)
    s = ((xmax - xmin) / np.float32(maxq)).astype(np.float32)
    z = np.rint((-xmin) / s).astype(np.float32)
    return s, z


def quantize(w, s, z, maxq: int) -> np.ndarray:
    """Codes of one column: clamp(rint(w/s) + z, 0, maxq), decided in float32."""
    w32 = np.asarray(w, dtype=np.float32)
    q = np.rint(w32 / s) + z
    return np.clip(q, np.float32(0), np.float32(maxq)).astype(np.float32)


def dequantize(codes, scales, zeros, group: int) -> np.ndarray:
    """W_q = s (q - z) per group, float64."""
    c = np.asarray(codes, np.float64)
    s = np.repeat(np.asarray(scales, np.float64), group, axis=1)
    z = np.repeat(np.asarray(zeros, np.float64), group, axis=1)
    return s * (c - z)


def act_order_perm(H) -> np.ndarray:
    """Processing order of GPTQ's activation-order option: columns by
    decreasing H_ii, with a dead column (H_ii == 0) counted as 1 (its value
    after the dead fix) and ties in increasing column index.  Returns perm with
    perm[j] = the column processed j-th.  H_ii are compared as the float32
    values they are stored as."""
    d = np.diag(np.asarray(H, np.float32)).astype(np.float64)
    key = np.where(d == 0, 1.0, d)
    idx = np.arange(d.size)
    return np.array(sorted(idx, key=lambda i: (-key[i], i)), dtype=np.int64)


def gptq(w, H, bits: int, group: int, damp: float = 0.01, block: int = 128,
         act_order: bool = False, static_groups: bool = False) -> dict:
    """GPTQ on one weight matrix with Hessian H (CLHA section 2.2 step 3,
    "standard GPTQ column-sequential updates" with H = H_comb).

    w: [r, c] weights, H: [c, c] symmetric PSD (undamped).  Steps:
      1. dead columns (H_ii == 0): H_ii := 1, W[:, i] := 0;
      2. static_groups: fit (s, z) of every row and natural group
         (columns g*group .. +group-1) once, on these weights;
      3. act_order: process the columns in act_order_perm(H) order, i.e.
         run the rest on W[:, perm] and H[perm][:, perm];
      4. lambda = damp * mean(diag H); H += lambda I;
      5. U = upper Cholesky factor of H^-1;
      6. blocks of `block` columns; inside a block, column by column:
         the column's grid is its static one (step 2), or else, at every
         group-th processed column, (s, z) fitted per row on the next `group`
         processed columns' current weights; quantize the column;
         err = (w - what)/U_jj; propagate err * U[j, j+1:] into the rest of
         the block; after the block, propagate the block's errors into all
         later columns through U[block, later].
    Returns, in natural column order, codes [r,c] uint8, and the grids
    scales [r,c/g] float32 and zeros [r,c/g] uint8 with g_idx [c] (column i
    uses grid g_idx[i]: i // group, except for act_order without static
    groups, where it is the column's processing position // group); also obs
    [r] (sum of err^2 per row), wq [r,c] float64, dead [c] bool, lam, perm,
    and U in processing order.
    """
    W = np.array(w, dtype=np.float64)
    Hd = np.array(H, dtype=np.float64)
    r, c = W.shape
    if c % group or block % group:
        raise ValueError("group must divide the column count and the block size")
    maxq = (1 << bits) - 1
    ng = c // group
    diag = np.diag(Hd).copy()
    dead = diag == 0
    Hd[dead, dead] = 1.0
    W[:, dead] = 0.0
    scales = np.zeros((r, ng), np.float32)
    zeros = np.zeros((r, ng), np.uint8)
    if static_groups:
        zs = np.zeros((r, ng), np.float32)
        for g in range(ng):
            scales[:, g], zs[:, g] = quant_params(W[:, g * group:(g + 1) * group], maxq)
        zeros = zs.astype(np.uint8)
    perm = act_order_perm(H) if act_order else np.arange(c)
    W = W[:, perm]
    Hd = Hd[np.ix_(perm, perm)]
    lam = damp * float(np.mean(np.diag(Hd)))
    Hd[np.diag_indices(c)] += lam
    U = inverse_cholesky_upper(Hd)

    codes_p = np.zeros((r, c), np.uint8)   # processing order
    obs = np.zeros(r)
    s = z = None
    for i1 in range(0, c, block):
        i2 = min(i1 + block, c)
        W1 = W[:, i1:i2].copy()
        E1 = np.zeros_like(W1)
        for j in range(i1, i2):
            jj = j - i1
            if static_groups:
                g = perm[j] // group
                s, z = scales[:, g], zeros[:, g].astype(np.float32)
            elif j % group == 0:
                s, z = quant_params(W1[:, jj:jj + group], maxq)
                scales[:, j // group] = s
                zeros[:, j // group] = z.astype(np.uint8)
            wcol = W1[:, jj]
            q = quantize(wcol, s, z, maxq)
            codes_p[:, j] = q.astype(np.uint8)
            what = s.astype(np.float64) * (q.astype(np.float64) - z.astype(np.float64))
            err = (wcol - what) / U[j, j]
            obs += err * err
            W1[:, jj + 1:] -= np.outer(err, U[j, j + 1:i2])
            E1[:, jj] = err
        W[:, i2:] -= E1 @ U[i1:i2, i2:]
    codes = np.zeros_like(codes_p)
    codes[:, perm] = codes_p
    g_idx = np.arange(c) // group
    if act_order and not static_groups:
        g_idx[perm] = np.arange(c) // group
    wq = dequantize_idx(codes, scales, zeros, g_idx)
    return {"codes": codes, "scales": scales, "zeros": zeros, "obs": obs,
            "wq": wq, "dead": dead, "lam": lam, "U": U, "perm": perm, "g_idx": g_idx}


def dequantize_idx(codes, scales, zeros, g_idx) -> np.ndarray:
    """W_q[:, i] = s[:, g_idx[i]] (q[:, i] - z[:, g_idx[i]]), float64."""
    gi = np.asarray(g_idx, np.int64)
    s = np.asarray(scales, np.float64)[:, gi]
    z = np.asarray(zeros, np.float64)[:, gi]
    return s * (np.asarray(codes, np.float64) - z)


def pack_codes(codes, bits: int) -> np.ndarray:
    """b-bit packed storage of a flat code stream (CLHA section 2.3 stores
    shared experts at b+1 bits, routed ones at b): code j contributes its bits,
    least significant first, at positions j*b .. j*b+b-1 of a bit stream whose
    bit 0 is the least significant bit of byte 0."""
    c = np.asarray(codes, dtype=np.int64).ravel()
    stream = ((c[:, None] >> np.arange(bits)[None, :]) & 1).ravel().astype(np.uint8)
    return np.packbits(stream, bitorder="little")


def unpack_codes(packed, bits: int, n: int) -> np.ndarray:
    """Inverse of pack_codes: the first n codes of the stream."""
    stream = np.unpackbits(np.asarray(packed, dtype=np.uint8), bitorder="little")[: n * bits]
    w = (1 << np.arange(bits)).astype(np.int64)
    return (stream.reshape(n, bits).astype(np.int64) @ w).astype(np.uint8)


def load_divergence(counts_a, counts_b) -> float:
    """Jensen-Shannon divergence (natural log) between two layers' expert-load
    distributions p = n / sum n: JSD = (KL(p||m) + KL(q||m)) / 2, m = (p + q)/2,
    with 0 log 0 = 0 (a divergence between the layers' routing, section 4)."""
    p = np.asarray(counts_a, np.float64)
    q = np.asarray(counts_b, np.float64)
    p, q = p / p.sum(), q / q.sum()
    m = (p + q) / 2
    def kl(a):
        return sum(ai * np.log(ai / mi) for ai, mi in zip(a, m) if ai > 0)
    return 0.5 * (kl(p) + kl(q))


def topk_overlap(topk_a, topk_b) -> float:
    """Mean over tokens of |choices in layer a and in layer b| / K."""
    a = np.asarray(topk_a)
    b = np.asarray(topk_b)
    k = a.shape[1]
    return float(np.mean([len(set(ra.tolist()) & set(rb.tolist())) / k for ra, rb in zip(a, b)]))


def loss(w, wq, H) -> float:
    """tr[(W_q - W) H (W_q - W)^T] = sum over rows of delta_r H delta_r^T
    (CLHA section 2.1 objective for one layer term)."""
    delta = np.asarray(wq, np.float64) - np.asarray(w, np.float64)
    return float(np.sum((delta @ np.asarray(H, np.float64)) * delta))


# --------------------------------------------------------------------------- whole pair

def calibrate_pair(x_bits_list, logits_list, jobs: dict, *, n_routed: int, top_k: int,
                   n_shared: int, mode: str, bits: int, shared_bits: int, group: int,
                   damp: float = 0.01, block: int = 128, alpha=None,
                   layer_losses: bool = False) -> dict:
    """The three CLHA phases on one shared-weight group (section 2.2).

    x_bits_list / logits_list: one entry per layer sharing the experts.
    jobs: {expert: [r, c] float array} -- the stacked matrices of each expert
    to quantize.  Routed expert e (< E) uses Hessian slot e; every shared
    expert (E <= e < E + n_shared) uses slot E, the all-token Hessian, and
    shared_bits bits (CLHA-MP, section 2.3).
    Returns routing, counts, per-layer S, H_comb and alpha per slot, GPTQ
    outputs and the loss under H_comb per expert (and per layer if asked).
    """
    def slot_of(e):
        return e if e < n_routed else n_routed

    slots = sorted({slot_of(e) for e in jobs})
    out = {"topk": [], "counts": [], "offsets": [], "token_ids": [], "S": [], "n": []}
    for x_bits, lg in zip(x_bits_list, logits_list):
        tk = route(lg, top_k)
        counts, offsets, ids = bucket(tk, n_routed)
        S, all_counts = layer_hessians(x_bits, tk, n_routed, n_shared, slots=slots)
        out["topk"].append(tk)
        out["counts"].append(counts)
        out["offsets"].append(offsets)
        out["token_ids"].append(ids)
        out["S"].append(S)
        out["n"].append(all_counts)
    out["H"], out["alpha"] = {}, {}
    for s in slots:
        H, a = aggregate([S[s] for S in out["S"]], [n[s] for n in out["n"]], mode, alpha)
        out["H"][s], out["alpha"][s] = H, a
    out["gptq"], out["loss"], out["layer_loss"] = {}, {}, {}
    for e, w in sorted(jobs.items()):
        s = slot_of(e)
        b = shared_bits if e >= n_routed else bits
        g = gptq(w, out["H"][s], b, group, damp, block)
        out["gptq"][e] = g
        out["loss"][e] = loss(w, g["wq"], out["H"][s])
        if layer_losses:
            out["layer_loss"][e] = [
                loss(w, g["wq"], S[s] / n[s]) if n[s] > 0 else 0.0
                for S, n in zip(out["S"], out["n"])]
    return out
