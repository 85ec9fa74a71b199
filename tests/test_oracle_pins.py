"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one oracle function to something independent: a hand-computed
fixture, a closed form, a brute-force enumeration, a mathematical identity
fixed by the CLHA summary (Proposition 1, section 2.1) or by GPTQ's
derivation, or a special case that reduces to a textbook routine.  The
planted-mistake tests at the end re-run some pins on deliberately broken
copies of the oracle and require them to fail.
"""
import inspect
import itertools
import json
import os
import types

import numpy as np
import pytest

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _spd(rng, c, spread=2.0, n=None):
    """Random SPD matrix X^T X / n with a spread-out spectrum."""
    n = n or 4 * c
    s = 10.0 ** rng.uniform(-spread / 2, spread / 2, c)
    x = rng.standard_normal((n, c)) * s
    q, _ = np.linalg.qr(rng.standard_normal((c, c)))
    x = x @ q
    return x.T @ x / n


# =========================================================================== routing

def test_route_golden():
    g = json.load(open(os.path.join(GOLDEN, "route_small.json")))
    lg = np.array(g["logits"], np.float32)
    tk = oracle.route(lg, g["k"])
    assert tk.tolist() == g["topk"]
    counts, offsets, ids = oracle.bucket(tk, lg.shape[1])
    assert counts.tolist() == g["counts"]
    assert offsets.tolist() == g["offsets"]
    assert ids.tolist() == g["token_ids"]


def _route_by_repeated_argmax(lg, k):
    """Textbook selection: K rounds of 'largest remaining logit, lowest index'."""
    n, e = lg.shape
    out = np.zeros((n, k), np.int32)
    for t in range(n):
        taken = set()
        for j in range(k):
            best = None
            for x in range(e):
                if x in taken:
                    continue
                if best is None or lg[t, x] > lg[t, best]:
                    best = x
            out[t, j] = best
            taken.add(best)
    return out


@pytest.mark.parametrize("seed,e,k", [(1, 8, 2), (2, 16, 6), (3, 5, 5), (4, 64, 1)])
def test_route_brute_force_with_ties(seed, e, k):
    rng = _rng(seed)
    # coarse values force many exact ties
    lg = rng.integers(-3, 4, (200, e)).astype(np.float32) * np.float32(0.5)
    assert (oracle.route(lg, k) == _route_by_repeated_argmax(lg, k)).all()


def test_route_invariants_and_errors():
    rng = _rng(5)
    lg = rng.standard_normal((500, 32)).astype(np.float32)
    tk = oracle.route(lg, 6)
    assert tk.shape == (500, 6)
    for t in range(500):
        assert len(set(tk[t])) == 6
        vals = lg[t, tk[t]]
        assert np.all(np.diff(vals) <= 0)
        assert lg[t].max() == vals[0]
    bad = lg.copy()
    bad[3, 4] = np.nan
    with pytest.raises(ValueError):
        oracle.route(bad, 2)
    bad[3, 4] = np.inf
    with pytest.raises(ValueError):
        oracle.route(bad, 2)
    with pytest.raises(ValueError):
        oracle.route(lg, 33)


def test_bucket_brute_force_and_invariants():
    rng = _rng(6)
    n, e, k = 300, 12, 3
    tk = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    counts, offsets, ids = oracle.bucket(tk, e)
    assert counts.sum() == n * k
    assert offsets[0] == 0 and offsets[-1] == n * k
    for x in range(e):
        want = [t for t in range(n) if x in tk[t]]
        got = ids[offsets[x]:offsets[x + 1]].tolist()
        assert got == want
        assert counts[x] == len(want)
    seen = np.bincount(ids, minlength=n)
    assert (seen == k).all()


# =========================================================================== Gram sums

def test_gram_hand_example():
    x = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert oracle.gram(x).tolist() == [[10.0, 14.0], [14.0, 20.0]]


def test_gram_equals_sum_of_outer_products():
    rng = _rng(7)
    x = rng.standard_normal((37, 9))
    s = np.zeros((9, 9))
    for t in range(37):
        s += np.outer(x[t], x[t])
    np.testing.assert_allclose(oracle.gram(x), s, rtol=1e-13, atol=1e-12)
    g = oracle.gram(x)
    assert (g == g.T).all()
    assert np.linalg.eigvalsh(g).min() >= -1e-12 * np.trace(g)


def test_gram_rows_brute_force():
    """Rows of S = X^T X, element by element as sums of products over tokens,
    across the chunk boundary (chunk 7 over 23 tokens)."""
    rng = _rng(8)
    xb = gen.bf16_bits(rng.standard_normal((23, 6)).astype(np.float32))
    x = gen.bf16_value(xb).astype(np.float64)
    rows = [4, 0, 4]
    got = oracle.gram_rows(xb, rows, chunk=7)
    for a, i in enumerate(rows):
        for j in range(6):
            want = 0.0
            for t in range(23):
                want += x[t, i] * x[t, j]
            assert abs(got[a, j] - want) <= 1e-14 * max(1.0, abs(want))


def test_bf16_widening():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F7F], np.uint16)
    v = oracle.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 0.0
    assert v[4] == 3.140625
    assert v[3] == 0.0 and np.signbit(v[3])
    assert v[5] == (2.0 - 2.0 ** -7) * 2.0 ** 127      # largest finite bf16


def test_layer_hessians_slots():
    rng = _rng(8)
    n, d, e, k = 64, 8, 4, 2
    x = rng.standard_normal((n, d)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)   # truncation: any bf16 pattern will do
    xv = oracle.bf16_to_f64(bits)
    lg = rng.standard_normal((n, e)).astype(np.float32)
    tk = oracle.route(lg, k)
    S, counts = oracle.layer_hessians(bits, tk, e, n_shared=2)
    assert len(counts) == e + 1 and counts[e] == n and counts[:e].sum() == n * k
    for ex in range(e):
        rows = [t for t in range(n) if ex in tk[t]]
        np.testing.assert_allclose(S[ex], xv[rows].T @ xv[rows], rtol=1e-14)
    np.testing.assert_allclose(S[e], xv.T @ xv, rtol=1e-14)


# =========================================================================== aggregation

def _layers(seed, d=12, na=50, nb=170, same=False):
    rng = _rng(seed)
    xa = rng.standard_normal((na, d))
    xb = xa.copy() if same else rng.standard_normal((nb, d)) * 1.7 + 0.2
    return oracle.gram(xa), na, oracle.gram(xb), (na if same else nb)


@pytest.mark.parametrize("mode", ["rt", "eq"])
def test_proposition1_identity(mode):
    """CLHA section 2.1, Proposition 1: sum_i alpha_i tr[D H_i D^T] = tr[D H_comb D^T]."""
    Sa, na, Sb, nb = _layers(9)
    H, a = oracle.aggregate([Sa, Sb], [na, nb], mode)
    alpha = [na / (na + nb), nb / (na + nb)] if mode == "rt" else [0.5, 0.5]
    np.testing.assert_allclose(a, alpha, rtol=1e-15)
    rng = _rng(10)
    for _ in range(5):
        D = rng.standard_normal((7, Sa.shape[0]))
        lhs = alpha[0] * np.trace(D @ (Sa / na) @ D.T) + alpha[1] * np.trace(D @ (Sb / nb) @ D.T)
        rhs = np.trace(D @ H @ D.T)
        assert abs(lhs - rhs) <= 1e-12 * abs(lhs)


@pytest.mark.parametrize("mode", ["rt", "eq", "explicit"])
def test_proposition1_identity_three_layers(mode):
    """Proposition 1 is stated for n layers: with three layers of different
    sizes, sum_i alpha_i tr[D H_i D^T] = tr[D H_comb D^T] and the weights are
    the token shares (rt), 1/3 (eq) or the given ones (explicit)."""
    rng = _rng(15)
    ns = [40, 130, 75]
    S = [oracle.gram(rng.standard_normal((n, 10)) * (1 + i)) for i, n in enumerate(ns)]
    given = [0.2, 0.5, 0.3]
    H, a = oracle.aggregate(S, ns, mode, alpha=given if mode == "explicit" else None)
    want = {"rt": [n / sum(ns) for n in ns], "eq": [1 / 3] * 3, "explicit": given}[mode]
    np.testing.assert_allclose(a, want, rtol=1e-15)
    for _ in range(5):
        D = rng.standard_normal((6, 10))
        lhs = sum(w * np.trace(D @ (Si / n) @ D.T) for w, Si, n in zip(want, S, ns))
        assert abs(lhs - np.trace(D @ H @ D.T)) <= 1e-12 * abs(lhs)


def test_plic_is_alpha_one():
    """alpha = 1 on the primary layer reduces exactly to PLIC = H_a (section 2.1)."""
    Sa, na, Sb, nb = _layers(11)
    H1, a = oracle.aggregate([Sa, Sb], [na, nb], "explicit", alpha=[1.0, 0.0])
    assert (H1 == Sa / na).all()
    Hp, _ = oracle.aggregate([Sa], [na], "rt")
    assert (Hp == Sa / na).all()
    Hq, _ = oracle.aggregate([Sa], [na], "eq")
    assert (Hq == Sa / na).all()


@pytest.mark.parametrize("mode", ["rt", "eq"])
def test_identical_layers_equal_plic(mode):
    Sa, na, Sb, nb = _layers(12, same=True)
    H, _ = oracle.aggregate([Sa, Sb], [na, nb], mode)
    assert (H == Sa / na).all()


def test_combined_hessian_symmetric_psd():
    Sa, na, Sb, nb = _layers(13)
    for mode in ("rt", "eq"):
        H, _ = oracle.aggregate([Sa, Sb], [na, nb], mode)
        assert (H == H.T).all()
        assert np.linalg.eigvalsh(H).min() >= -1e-12 * np.trace(H)


def test_empty_layers():
    Sa, na, Sb, nb = _layers(14)
    z = np.zeros_like(Sa)
    for mode in ("rt", "eq"):
        H, a = oracle.aggregate([Sa, z], [na, 0], mode)
        assert np.allclose(H, Sa / na, rtol=1e-15) and a[1] == 0.0
    H, a = oracle.aggregate([z, z], [0, 0], "rt")
    assert (H == np.eye(Sa.shape[0])).all() and (a == 0).all()


# =========================================================================== inverse Cholesky

def test_inverse_cholesky_2x2_closed_form():
    a, b, c = 4.0, 1.5, 2.0
    det = a * c - b * b
    U = oracle.inverse_cholesky_upper(np.array([[a, b], [b, c]]))
    u00 = np.sqrt(c / det)
    want = np.array([[u00, -b / (det * u00)], [0.0, 1.0 / np.sqrt(c)]])
    np.testing.assert_allclose(U, want, rtol=1e-14, atol=1e-15)


def test_inverse_cholesky_characterisation():
    """The upper-triangular U with positive diagonal and U^T U H = I is unique."""
    rng = _rng(15)
    for c in (3, 17, 64):
        H = _spd(rng, c)
        U = oracle.inverse_cholesky_upper(H)
        assert np.allclose(np.tril(U, -1), 0.0, atol=0)
        assert (np.diag(U) > 0).all()
        res = U.T @ U @ H - np.eye(c)
        assert np.abs(res).max() < 1e-9 * np.linalg.cond(H) ** 0.5 + 1e-10


def test_inverse_cholesky_diagonal():
    h = np.array([4.0, 0.25, 9.0, 1.0])
    U = oracle.inverse_cholesky_upper(np.diag(h))
    np.testing.assert_allclose(U, np.diag(1 / np.sqrt(h)), rtol=1e-15)


# =========================================================================== quantizer

def test_quantizer_golden():
    g = json.load(open(os.path.join(GOLDEN, "quantizer_cases.json")))
    for case in g["cases"]:
        maxq = (1 << case["bits"]) - 1
        x = np.array([case["x"]], np.float32)
        s, z = oracle.quant_params(x, maxq)
        assert s[0] == np.float32(case["scale"]), case["name"]
        assert z[0] == case["zero"], case["name"]
        q = oracle.quantize(x[0], s[0], z[0], maxq)
        assert q.tolist() == case["codes"], case["name"]
    for bits in g["all_zero"]["bits"]:
        maxq = (1 << bits) - 1
        x = np.zeros((1, 8), np.float32)
        s, z = oracle.quant_params(x, maxq)
        q = oracle.quantize(x[0], s[0], z[0], maxq)
        assert (q == z[0]).all() and 0 <= z[0] <= maxq
        assert (s[0] * (q - z[0]) == 0).all()


# =========================================================================== GPTQ

def _rtn(w, bits, group):
    """Round-to-nearest on the same per-group grid, groups fitted on W itself."""
    maxq = (1 << bits) - 1
    r, c = w.shape
    codes = np.zeros((r, c), np.uint8)
    for g0 in range(0, c, group):
        s, z = oracle.quant_params(w[:, g0:g0 + group], maxq)
        for j in range(g0, g0 + group):
            codes[:, j] = oracle.quantize(w[:, j], s, z, maxq)
    return codes


@pytest.mark.parametrize("bits,group,block", [(2, 16, 32), (3, 32, 32), (4, 8, 64)])
def test_gptq_diagonal_hessian_is_rtn(bits, group, block):
    rng = _rng(16)
    w = rng.normal(0, 0.02, (24, 64))
    H = np.diag(rng.uniform(0.5, 2.0, 64))
    out = oracle.gptq(w, H, bits, group, 0.01, block)
    assert (out["codes"] == _rtn(w, bits, group)).all()


def test_gptq_two_column_closed_form():
    """Two columns, one group: w1' = w1 + (w0 - what0) * H01/H11 on the damped H."""
    rng = _rng(17)
    for trial in range(20):
        w = rng.normal(0, 1.0, (5, 2))
        H = _spd(rng, 2, spread=1.0)
        damp = 0.01
        out = oracle.gptq(w, H, 3, 2, damp, 2)
        Hd = H + damp * np.mean(np.diag(H)) * np.eye(2)
        maxq = 7
        s, z = oracle.quant_params(w, maxq)
        q0 = oracle.quantize(w[:, 0], s, z, maxq)
        what0 = s.astype(np.float64) * (q0 - z)
        w1p = w[:, 1] + (w[:, 0] - what0) * Hd[0, 1] / Hd[1, 1]
        q1 = oracle.quantize(w1p, s, z, maxq)
        assert (out["codes"][:, 0] == q0).all()
        assert (out["codes"][:, 1] == q1).all()


def _gptq_by_conditional_optimum(w, H, bits, group, damp):
    """GPTQ re-derived without U: before column j is quantized, the remaining
    columns take the values that minimise (v - w) Hd (v - w)^T given the
    already-quantized columns:  v_{j:} = w_{j:} - Hd_{jj}^-1 Hd_{j,<j} (what_{<j} - w_{<j}).
    Group grids are fitted on v at each group's first column."""
    r, c = w.shape
    maxq = (1 << bits) - 1
    Hd = np.array(H, np.float64)
    dead = np.diag(Hd) == 0
    Hd[dead, dead] = 1.0
    w = np.array(w, np.float64)
    w[:, dead] = 0.0
    Hd = Hd + damp * np.mean(np.diag(Hd)) * np.eye(c)
    codes = np.zeros((r, c), np.uint8)
    what = np.zeros((r, c))
    s = z = None
    for j in range(c):
        if j == 0:
            v = w.copy()
        else:
            delta = what[:, :j] - w[:, :j]
            corr = np.linalg.solve(Hd[j:, j:], Hd[j:, :j] @ delta.T).T
            v = np.concatenate([what[:, :j], w[:, j:] - corr], axis=1)
        if j % group == 0:
            s, z = oracle.quant_params(v[:, j:j + group], maxq)
        q = oracle.quantize(v[:, j], s, z, maxq)
        codes[:, j] = q
        what[:, j] = s.astype(np.float64) * (q - z)
    return codes, what


@pytest.mark.parametrize("seed,c,group,block,bits", [
    (18, 16, 16, 16, 2), (19, 32, 8, 16, 2), (20, 24, 8, 24, 3), (21, 32, 16, 32, 4)])
def test_gptq_matches_conditional_optimum(seed, c, group, block, bits):
    rng = _rng(seed)
    w = rng.normal(0, 0.05, (6, c))
    H = _spd(rng, c, spread=3.0)
    out = oracle.gptq(w, H, bits, group, 0.01, block)
    codes, what = _gptq_by_conditional_optimum(w, H, bits, group, 0.01)
    assert (out["codes"] == codes).all()
    np.testing.assert_allclose(out["wq"], what, rtol=0, atol=1e-12)


def test_gptq_obs_identity_and_loss_identity():
    """sum_j err_j^2 = tr[(Wq - W) Hd (Wq - W)^T]; hence the undamped loss equals
    obs - lambda ||Wq - W||^2 (W after the dead-column fix)."""
    rng = _rng(22)
    c = 64
    w = rng.normal(0, 0.02, (10, c))
    H = _spd(rng, c, spread=3.0)
    H[5, :] = 0.0
    H[:, 5] = 0.0          # a dead input column
    out = oracle.gptq(w, H, 2, 16, 0.01, 32)
    wf = w.copy()
    wf[:, 5] = 0.0
    Hd = H.copy()
    Hd[5, 5] = 1.0
    Hd += out["lam"] * np.eye(c)
    D = out["wq"] - wf
    tr = np.sum((D @ Hd) * D)
    assert abs(out["obs"].sum() - tr) <= 1e-10 * tr
    undamped = oracle.loss(w, out["wq"], H)
    assert abs(out["obs"].sum() - out["lam"] * np.sum(D * D) - undamped) <= 1e-10 * tr


def test_gptq_dead_column():
    rng = _rng(23)
    c = 32
    w = rng.normal(0, 0.02, (8, c))
    H = _spd(rng, c)
    H[7, :] = 0.0
    H[:, 7] = 0.0
    out = oracle.gptq(w, H, 2, 16, 0.01, 32)
    assert out["dead"][7] and out["dead"].sum() == 1
    z = out["zeros"][:, 7 // 16]
    assert (out["codes"][:, 7] == z).all()
    assert (out["wq"][:, 7] == 0.0).all()


@pytest.mark.parametrize("group", [8, 16])
def test_gptq_lazy_blocks_equal_eager(group):
    rng = _rng(24)
    c = 64
    w = rng.normal(0, 0.02, (12, c))
    H = _spd(rng, c, spread=3.0)
    ref = oracle.gptq(w, H, 2, group, 0.01, group)["codes"]
    for block in (2 * group, 64):
        assert (oracle.gptq(w, H, 2, group, 0.01, block)["codes"] == ref).all()


def test_gptq_single_group_per_row():
    rng = _rng(25)
    w = rng.normal(0, 0.02, (5, 16))
    out = oracle.gptq(w, _spd(rng, 16), 2, 16, 0.01, 16)
    assert out["scales"].shape == (5, 1) and out["zeros"].shape == (5, 1)


@pytest.mark.parametrize("seed,c,group", [(26, 6, 6), (27, 8, 4), (28, 8, 8)])
def test_gptq_not_better_than_brute_force(seed, c, group):
    """Enumerate every code vector on GPTQ's own grid (2 bits): the minimum of
    tr[D Hd D^T] can never be above GPTQ's value."""
    rng = _rng(seed)
    r, bits = 3, 2
    w = rng.normal(0, 0.05, (r, c))
    H = _spd(rng, c, spread=2.0)
    out = oracle.gptq(w, H, bits, group, 0.01, group)
    Hd = H + out["lam"] * np.eye(c)
    s = np.repeat(out["scales"].astype(np.float64), group, axis=1)
    z = np.repeat(out["zeros"].astype(np.float64), group, axis=1)
    allq = np.array(list(itertools.product(range(1 << bits), repeat=c)), np.float64)
    for row in range(r):
        cand = s[row] * (allq - z[row]) - w[row]
        vals = np.einsum("ij,jk,ik->i", cand, Hd, cand)
        d = out["wq"][row] - w[row]
        g = d @ Hd @ d
        assert vals.min() <= g * (1 + 1e-12)
        # GPTQ's own point is on the grid, so the minimum is attained at or below it
        qrow = out["codes"][row].astype(np.float64)
        idx = int(sum(int(q) * (4 ** (c - 1 - i)) for i, q in enumerate(qrow)))
        assert abs(vals[idx] - g) <= 1e-12 * max(g, 1e-30)


# ---- activation order and static groups (two GPTQ options the CLHA pages leave
# open; their readings: columns by decreasing H_ii with dead columns counted as
# 1 and ties by index, groups as runs of processed columns; static grids fitted
# once per natural group on the weights after the dead fix)

def test_act_order_perm_hand_example():
    # H_ii = 2, 0 (dead: counts as 1), 5, 2, 1 -> 5 (col 2), the tie 2, 2 in
    # column order (0, 3), then the tie 1, 1 (1, 4)
    H = np.diag([2.0, 0.0, 5.0, 2.0, 1.0]).astype(np.float32)
    assert oracle.act_order_perm(H).tolist() == [2, 0, 3, 1, 4]


@pytest.mark.parametrize("bits,group,block", [(2, 8, 32), (3, 16, 32), (4, 32, 64)])
def test_act_order_diagonal_hessian_is_rtn_on_sorted_groups(bits, group, block):
    """A diagonal H propagates nothing, so GPTQ is round-to-nearest; with
    activation order the groups are runs of columns by decreasing H_ii."""
    rng = _rng(40)
    c = 64
    w = rng.normal(0, 0.02, (12, c))
    d = rng.permutation(np.linspace(0.5, 2.0, c))     # distinct diagonal
    H = np.diag(d)
    out = oracle.gptq(w, H, bits, group, 0.01, block, act_order=True)
    order = np.argsort(-d)
    maxq = (1 << bits) - 1
    want = np.zeros((12, c), np.uint8)
    for g0 in range(0, c, group):
        cols = order[g0:g0 + group]
        s, z = oracle.quant_params(w[:, cols], maxq)
        for j in cols:
            want[:, j] = oracle.quantize(w[:, j], s, z, maxq)
        assert (out["g_idx"][cols] == g0 // group).all()
    assert (out["codes"] == want).all()
    # static groups: the natural groups' grids, so round-to-nearest as without
    # activation order
    st = oracle.gptq(w, H, bits, group, 0.01, block, act_order=True, static_groups=True)
    assert (st["codes"] == _rtn(w, bits, group)).all()
    assert (st["g_idx"] == np.arange(c) // group).all()


def _conditional_optimum_ordered(w, H, bits, group, damp, perm, static):
    """The conditional-optimum form of GPTQ (no U) over columns in the order
    perm: before processed column j is quantized, the unprocessed columns take
    their best values given the processed ones.  Grids: the natural group's,
    fitted on the dead-fixed weights (static), or fitted on the next `group`
    processed columns' current values.  Returns codes and W_q in natural
    column order."""
    r, c = w.shape
    maxq = (1 << bits) - 1
    Hn = np.array(H, np.float64)
    dead = np.diag(Hn) == 0
    Hn[dead, dead] = 1.0
    wn = np.array(w, np.float64)
    wn[:, dead] = 0.0
    Hn = Hn + damp * np.mean(np.diag(Hn)) * np.eye(c)
    sgrid = [oracle.quant_params(wn[:, g:g + group], maxq) for g in range(0, c, group)]
    codes = np.zeros((r, c), np.uint8)
    what = np.zeros((r, c))
    s = z = None
    for j in range(c):
        done, rest = list(perm[:j]), list(perm[j:])
        if j == 0:
            v = wn.copy()
        else:
            delta = what[:, done] - wn[:, done]
            corr = np.linalg.solve(Hn[np.ix_(rest, rest)], Hn[np.ix_(rest, done)] @ delta.T).T
            v = wn.copy()
            v[:, done] = what[:, done]
            v[:, rest] = wn[:, rest] - corr
        col = perm[j]
        if static:
            s, z = sgrid[col // group]
        elif j % group == 0:
            s, z = oracle.quant_params(v[:, list(perm[j:j + group])], maxq)
        q = oracle.quantize(v[:, col], s, z, maxq)
        codes[:, col] = q
        what[:, col] = s.astype(np.float64) * (q - z)
    return codes, what


@pytest.mark.parametrize("seed,c,group,block,bits,act,static", [
    (41, 32, 8, 16, 2, True, False), (42, 24, 8, 24, 3, True, True),
    (43, 32, 16, 32, 2, False, True), (44, 32, 4, 16, 4, True, False)])
def test_gptq_options_match_conditional_optimum(seed, c, group, block, bits, act, static):
    rng = _rng(seed)
    w = rng.normal(0, 0.05, (6, c))
    H = _spd(rng, c, spread=3.0)
    H[3, :] = 0.0
    H[:, 3] = 0.0          # a dead column, counted as H_ii = 1 in the order
    out = oracle.gptq(w, H, bits, group, 0.01, block, act_order=act, static_groups=static)
    perm = oracle.act_order_perm(H) if act else np.arange(c)
    codes, what = _conditional_optimum_ordered(w, H, bits, group, 0.01, perm, static)
    assert (out["codes"] == codes).all()
    np.testing.assert_allclose(out["wq"], what, rtol=0, atol=1e-12)


@pytest.mark.parametrize("act,static", [(True, False), (False, True), (True, True)])
def test_gptq_options_obs_identity(act, static):
    """sum_j err_j^2 = tr[(Wq - W) Hd (Wq - W)^T] in natural column order: the
    codes, grids and g_idx come back in the columns they belong to."""
    rng = _rng(45)
    c = 64
    w = rng.normal(0, 0.02, (10, c))
    H = _spd(rng, c, spread=3.0)
    out = oracle.gptq(w, H, 3, 16, 0.01, 32, act_order=act, static_groups=static)
    Hd = H + out["lam"] * np.eye(c)
    D = out["wq"] - w
    tr = np.sum((D @ Hd) * D)
    assert abs(out["obs"].sum() - tr) <= 1e-10 * tr


def test_act_order_ignores_input_column_order():
    """With distinct H_ii, activation order processes the same columns in the
    same order whatever order they arrive in; codes follow their columns."""
    rng = _rng(46)
    c = 48
    w = rng.normal(0, 0.02, (7, c))
    H = _spd(rng, c, spread=3.0)
    P = rng.permutation(c)
    a = oracle.gptq(w, H, 3, 8, 0.01, 16, act_order=True)
    b = oracle.gptq(w[:, P], H[np.ix_(P, P)], 3, 8, 0.01, 16, act_order=True)
    assert (b["codes"] == a["codes"][:, P]).all()
    assert (b["g_idx"] == a["g_idx"][P]).all()
    assert (b["scales"] == a["scales"]).all() and (b["zeros"] == a["zeros"]).all()


def test_static_grids_do_not_depend_on_h():
    rng = _rng(47)
    w = rng.normal(0, 0.02, (5, 32))
    a = oracle.gptq(w, _spd(rng, 32, spread=3.0), 2, 8, 0.01, 16, static_groups=True)
    b = oracle.gptq(w, _spd(rng, 32, spread=1.0), 2, 8, 0.01, 16, static_groups=True, act_order=True)
    assert (a["scales"] == b["scales"]).all() and (a["zeros"] == b["zeros"]).all()
    for g in range(4):
        s, z = oracle.quant_params(w[:, 8 * g:8 * g + 8], 3)
        assert (a["scales"][:, g] == s).all() and (a["zeros"][:, g] == z).all()


def _options_pins_hold(gptq_fn):
    rng = _rng(48)
    c = 24
    w = rng.normal(0, 0.05, (5, c))
    H = _spd(rng, c, spread=3.0)
    ok = True
    for act, static in ((True, False), (True, True)):
        try:
            out = gptq_fn(w, H, 2, 8, 0.01, 8, act_order=act, static_groups=static)
        except np.linalg.LinAlgError:
            return False          # a mutant that breaks the factorisation is caught too
        perm = oracle.act_order_perm(H)
        codes, _ = _conditional_optimum_ordered(w, H, 2, 8, 0.01, perm, static)
        Hd = H + out["lam"] * np.eye(c)
        D = out["wq"] - w
        ok &= bool((out["codes"] == codes).all())
        ok &= bool(abs(out["obs"].sum() - np.sum((D @ Hd) * D)) <= 1e-10 * np.sum((D @ Hd) * D))
    return ok


@pytest.mark.parametrize("old,new", [
    ("codes[:, perm] = codes_p", "codes[:] = codes_p"),                           # order not undone
    ("Hd = Hd[np.ix_(perm, perm)]", "Hd = Hd[perm]"),                             # rows only
    ("g = perm[j] // group", "g = j // group"),                                   # static grid by position
    ("g_idx[perm] = np.arange(c) // group", "g_idx[:] = np.arange(c) // group"),  # natural g_idx
])
def test_planted_gptq_option_mistakes_are_caught(old, new):
    assert _options_pins_hold(oracle.gptq)
    assert not _options_pins_hold(_mutant(oracle.gptq, old, new))


def test_loss_equals_projected_residual():
    """tr[D (X^T X / n) D^T] = ||D X^T||_F^2 / n."""
    rng = _rng(29)
    x = rng.standard_normal((40, 16))
    H = oracle.gram(x) / 40
    w = rng.normal(0, 0.02, (6, 16))
    wq = w + rng.normal(0, 0.001, (6, 16))
    want = np.sum(((wq - w) @ x.T) ** 2) / 40
    assert abs(oracle.loss(w, wq, H) - want) <= 1e-12 * want


# =========================================================================== planted mistakes

def _mutant(func, old, new):
    """Copy of an oracle function with one textual change, run in the oracle's namespace."""
    src = inspect.getsource(func)
    assert src.count(old) == 1, old
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns[func.__name__]


def _conditional_pin_holds(gptq_fn):
    rng = _rng(30)
    w = rng.normal(0, 0.05, (6, 32))
    H = _spd(rng, 32, spread=3.0)
    out = gptq_fn(w, H, 2, 8, 0.01, 16)
    codes, _ = _gptq_by_conditional_optimum(w, H, 2, 8, 0.01)
    return bool((out["codes"] == codes).all())


def _obs_pin_holds(gptq_fn):
    rng = _rng(31)
    w = rng.normal(0, 0.02, (8, 32))
    H = _spd(rng, 32, spread=3.0)
    out = gptq_fn(w, H, 2, 8, 0.01, 16)
    Hd = H + out["lam"] * np.eye(32)
    D = out["wq"] - w
    tr = np.sum((D @ Hd) * D)
    return abs(out["obs"].sum() - tr) <= 1e-10 * tr


@pytest.mark.parametrize("old,new", [
    ("W[:, i2:] -= E1 @ U[i1:i2, i2:]", "pass"),                                  # lazy update dropped
    ("W1[:, jj + 1:] -= np.outer(err, U[j, j + 1:i2])",
     "W1[:, jj + 1:] += np.outer(err, U[j, j + 1:i2])"),                          # sign flip
    ("W[:, i2:] -= E1 @ U[i1:i2, i2:]", "W[:, i2:] -= E1 @ U[i2:, i1:i2].T"),     # transposed operand
    ("err = (wcol - what) / U[j, j]", "err = (wcol - what) * U[j, j]"),            # wrong scaling
    ("Hd[np.diag_indices(c)] += lam", "Hd[np.diag_indices(c)] += 2 * lam"),        # wrong damping
])
def test_planted_gptq_mistakes_are_caught(old, new):
    assert _conditional_pin_holds(oracle.gptq)
    bad = _mutant(oracle.gptq, old, new)
    assert not (_conditional_pin_holds(bad) and _obs_pin_holds(bad))


def test_planted_inverse_cholesky_mistake_is_caught():
    bad_u = _mutant(oracle.inverse_cholesky_upper, "return np.linalg.cholesky(Hinv).T",
                    "return np.linalg.cholesky(np.asarray(H, np.float64)).T")
    ns = dict(vars(oracle))
    ns["inverse_cholesky_upper"] = bad_u
    src = inspect.getsource(oracle.gptq)
    exec(compile(src, "<mutant>", "exec"), ns)
    assert not _conditional_pin_holds(ns["gptq"])


def test_planted_aggregation_mistake_is_caught():
    """Averaging the per-layer H_i with equal weight under 'rt' breaks Proposition 1."""
    bad = _mutant(oracle.aggregate, "H = sum(np.asarray(S, np.float64) for S in S_list) / total",
                  "H = sum(np.asarray(S, np.float64) / float(k) for S, k in zip(S_list, n)) / len(S_list)")
    Sa, na, Sb, nb = _layers(32)
    H, _ = bad([Sa, Sb], [na, nb], "rt")
    D = _rng(33).standard_normal((4, Sa.shape[0]))
    lhs = na / (na + nb) * np.trace(D @ (Sa / na) @ D.T) + nb / (na + nb) * np.trace(D @ (Sb / nb) @ D.T)
    assert abs(lhs - np.trace(D @ H @ D.T)) > 1e-6 * abs(lhs)


def test_planted_route_mistake_is_caught():
    bad = _mutant(oracle.route, "np.lexsort((key_idx, -lg.astype(np.float64)), axis=-1)",
                  "np.lexsort((-key_idx, -lg.astype(np.float64)), axis=-1)")     # ties to the higher index
    g = json.load(open(os.path.join(GOLDEN, "route_small.json")))
    assert bad(np.array(g["logits"], np.float32), g["k"]).tolist() != g["topk"]


# =========================================================================== packed storage

def test_pack_codes_hand_example():
    """Section 2.3 stores codes at b (or b+1) bits.  Worked by hand, bits least
    significant first: 3-bit codes 1,2,3,4,5,6,7,0 are the stream
    100 010 110 001 101 011 111 000, i.e. bytes 10001011 00011010 11111000
    read from bit 0 up: 1+16+64+128 = 209, 8+16+64 = 88, 1+2+4+8+16 = 31.
    2-bit codes 0,1,2,3: stream 00 10 01 11 -> 4+32+64+128 = 228."""
    assert oracle.pack_codes([1, 2, 3, 4, 5, 6, 7, 0], 3).tolist() == [209, 88, 31]
    assert oracle.pack_codes([0, 1, 2, 3], 2).tolist() == [228]
    assert oracle.pack_codes([255] * 8, 8).tolist() == [255] * 8


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_pack_codes_round_trip_and_size(bits):
    codes = _rng(40 + bits).integers(0, 1 << bits, 8 * 37)
    packed = oracle.pack_codes(codes, bits)
    assert packed.size == codes.size * bits // 8
    assert np.array_equal(oracle.unpack_codes(packed, bits, codes.size), codes)


def test_mixed_precision_accounting():
    """Packed bits per parameter: b + (32 + 8)/g; shared experts at b+1 raise the
    total by their share of the parameters (section 2.3)."""
    from gptq_calibration_moe_amd.calibrate import mixed_precision_overhead, storage_bits
    assert storage_bits(2, 256, 3, 128) == 2 * 256 * 3 + 2 * 2 * 40
    jobs = [(1408, 2048, 3, 3)] * 64 + [(1408, 2048, 4, 3)] * 2
    r = mixed_precision_overhead(jobs, 128)
    assert abs(r["base_bits_per_param"] - (3 + 40 / 128)) < 1e-12
    assert abs(r["bits_per_param"] - (3 + 40 / 128 + 2 / 66)) < 1e-12
    assert abs(r["overhead"] - (2 / 66) / (3 + 40 / 128)) < 1e-12


# =========================================================================== down_proj inputs

def test_round_bf16_hand_values():
    """bf16 keeps 8 significant bits: on [1, 2) the spacing is 2^-7, on [256, 512) it is 2.
    1 + 2^-8 is a tie and goes to the even neighbour 1; 1 + 0.75 * 2^-7 rounds up;
    -257.5 lies between -256 and -258 and rounds to -258."""
    got = oracle.round_bf16([1.0, 1.0 + 2.0 ** -8, 1.0 + 0.75 * 2.0 ** -7, 1.0 + 2.0 ** -9, -257.5, 0.0])
    assert got.tolist() == [1.0, 1.0, 1.0078125, 1.0, -258.0, 0.0]


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12 and abs(oracle.silu(-40.0)) < 1e-15


def test_swiglu_intermediate_hand_example():
    """x = (1, 0) picks column 0 of the weights: g = (1, 0), u = (3, 0), so
    h = (bf16(3 sigmoid(1)), 0) = (bf16(2.19318), 0) = (2.1875, 0) (spacing 2^-6 on [2, 4))."""
    x = gen.bf16_bits(np.array([[1.0, 0.0]], np.float32))
    w = gen.bf16_bits(np.array([[1.0, 0.0], [0.0, 2.0], [3.0, 0.0], [0.0, 0.5]], np.float32))
    h = oracle.swiglu_intermediate(x, w, 2)
    assert h.tolist() == [[2.1875, 0.0]]


def test_down_layer_hessians_one_token_per_expert():
    """Two routed experts with one token each and one shared expert over both:
    each routed Gram sum is h h^T of its token, the shared one the sum of both."""
    x = gen.bf16_bits(np.array([[1.0, 0.0], [0.0, 1.0]], np.float32))
    topk = np.array([[0], [1]])
    ws = [gen.bf16_bits(np.array([[1.0, 1.0], [0.5, 0.0], [2.0, 2.0], [1.0, 4.0]], np.float32))] * 3
    S, n = oracle.down_layer_hessians(x, topk, ws, 2, 2)
    assert n.tolist() == [1, 1, 2]
    h0 = oracle.swiglu_intermediate(x[:1], ws[0], 2)[0]
    h1 = oracle.swiglu_intermediate(x[1:], ws[1], 2)[0]
    assert (S[0] == np.outer(h0, h0)).all() and (S[1] == np.outer(h1, h1)).all()
    assert np.allclose(S[2], np.outer(h0, h0) + np.outer(h1, h1), rtol=1e-15)


# =========================================================================== routing divergence

def test_load_divergence_closed_forms():
    """JSD = 0 for equal loads, ln 2 for disjoint ones, and for p = (1, 0),
    q = (1/2, 1/2): m = (3/4, 1/4), KL(p||m) = ln(4/3), KL(q||m) = ln(4/3)/2,
    so JSD = (3/4) ln(4/3)."""
    assert oracle.load_divergence([3, 5, 2], [6, 10, 4]) == 0.0
    assert abs(oracle.load_divergence([4, 0], [0, 9]) - np.log(2.0)) < 1e-15
    assert abs(oracle.load_divergence([8, 0], [5, 5]) - 0.75 * np.log(4.0 / 3.0)) < 1e-15


def test_topk_overlap_hand_example():
    a = np.array([[0, 1], [2, 3], [4, 5]])
    b = np.array([[1, 0], [3, 6], [7, 8]])
    assert oracle.topk_overlap(a, b) == (1.0 + 0.5 + 0.0) / 3
    assert oracle.topk_overlap(a, a) == 1.0


def test_sweep_metrics_match_oracle():
    """The package's vectorised host metrics against the oracle's definitions."""
    from gptq_calibration_moe_amd.sweep import load_divergence, topk_overlap
    rng = _rng(60)
    for _ in range(5):
        ca, cb = rng.integers(0, 50, 16), rng.integers(0, 50, 16)
        ca[3] = 0
        assert abs(load_divergence(ca, cb) - oracle.load_divergence(ca, cb)) < 1e-14
        ta = np.stack([rng.permutation(16)[:4] for _ in range(200)])
        tb = np.stack([rng.permutation(16)[:4] for _ in range(200)])
        assert topk_overlap(ta, tb) == oracle.topk_overlap(ta, tb)


def test_sharpness_logits_limits():
    """Sampled routing: with the same activations in both layers, a small tau
    follows x R in both (overlap 1), a large tau is close to independent sampling
    (overlap near K/E)."""
    wl = gen.WORKLOADS[1].scaled(n_tokens=2048, x_kind="drift", drift=(0.0,))
    xa, xb = gen.activations(wl, 0, t=0.0)
    assert np.array_equal(xa, xb)
    sharp = [oracle.route(gen.sharpness_logits(wl, 0, l, xa, 1e-5), wl.top_k) for l in range(2)]
    assert oracle.topk_overlap(*sharp) == 1.0
    flat = [oracle.route(gen.sharpness_logits(wl, 0, l, xa, 1e3), wl.top_k) for l in range(2)]
    assert abs(oracle.topk_overlap(*flat) - wl.top_k / wl.n_routed) < 0.05


# =========================================================================== whole pair

def _pair_case():
    """Two layers of 12 tokens over d = 8, two routed experts at top-1 and one
    shared expert (CLHA section 2.3: it sees every token).  The winning expert
    of each token is planted in the logits, so the routed token sets are known
    without the oracle's routing."""
    rng = _rng(70)
    d, n = 8, 12
    x = [gen.bf16_bits(rng.standard_normal((n, d)).astype(np.float32)) for _ in range(2)]
    win = [np.array([0, 1, 1, 0, 0, 1, 0, 1, 1, 1, 0, 1]), np.array([1, 1, 0, 0, 1, 1, 1, 1, 0, 1, 1, 1])]
    logits = []
    for wv in win:
        lg = rng.uniform(-1.0, 0.0, (n, 2)).astype(np.float32)
        lg[np.arange(n), wv] += 2.0
        logits.append(lg)
    jobs = {e: rng.normal(0, 0.02, (4, d)) for e in range(3)}    # 2 = the shared expert
    return x, logits, win, jobs


def _brute_hessians(x, win, mode):
    """Sums of outer products over each job's tokens, per layer and combined:
    routed expert e over the tokens whose planted winner is e, the shared
    expert over all tokens."""
    xs = [gen.bf16_value(b).astype(np.float64) for b in x]
    per_layer = {}
    for e in range(3):
        S, n = [], []
        for l in range(2):
            rows = [t for t in range(xs[l].shape[0]) if e == 2 or win[l][t] == e]
            S.append(sum(np.outer(xs[l][t], xs[l][t]) for t in rows))
            n.append(len(rows))
        per_layer[e] = (S, n)
    H = {}
    for e, (S, n) in per_layer.items():
        if mode == "rt":
            H[e] = (S[0] + S[1]) / (n[0] + n[1])
        else:
            H[e] = 0.5 * S[0] / n[0] + 0.5 * S[1] / n[1]
    return per_layer, H


def _calibrate_pair_pins_hold(fn, mode="rt"):
    """The CLHA phases wired together: each job's Hessian is the brute-force
    combination of its own tokens (the shared job's over all tokens), GPTQ ran
    on that Hessian (its lambda and U), the shared job at b+1 bits and the
    routed ones at b (CLHA-MP), and the losses are tr[D H D^T] under H_comb and
    under each layer's S_l / n_l."""
    x, logits, win, jobs = _pair_case()
    damp, bits, shared_bits = 0.01, 2, 3
    try:
        out = fn(x, logits, jobs, n_routed=2, top_k=1, n_shared=1, mode=mode, bits=bits,
                 shared_bits=shared_bits, group=8, damp=damp, block=8, layer_losses=True)
        per_layer, H = _brute_hessians(x, win, mode)
        slot = {0: 0, 1: 1, 2: 2}
        for e, w in jobs.items():
            He = H[e]
            if not np.allclose(out["H"][slot[e]], He, rtol=1e-12, atol=0):
                return False
            g = out["gptq"][e]
            if abs(g["lam"] - damp * np.mean(np.diag(He))) > 1e-15 * abs(g["lam"]):
                return False
            Hd = He + g["lam"] * np.eye(He.shape[0])
            if np.max(np.abs(g["U"].T @ g["U"] @ Hd - np.eye(He.shape[0]))) > 1e-9:
                return False
            b = shared_bits if e == 2 else bits
            maxq = (1 << b) - 1
            codes = g["codes"]
            if codes.max() > maxq or (e == 2 and codes.max() <= (1 << bits) - 1):
                return False
            # group 0's grid is fitted on the untouched first group: s = range / maxq
            w32 = w.astype(np.float32)
            rng_ = np.maximum(w32.max(axis=1), 0) - np.minimum(w32.min(axis=1), 0)
            if not np.array_equal(g["scales"][:, 0], (rng_ / np.float32(maxq)).astype(np.float32)):
                return False
            D = g["wq"] - w
            want = float(np.sum((D @ He) * D))
            if abs(out["loss"][e] - want) > 1e-12 * want:
                return False
            S, n = per_layer[e]
            for l in range(2):
                want_l = float(np.sum((D @ (S[l] / n[l])) * D))
                if abs(out["layer_loss"][e][l] - want_l) > 1e-12 * want_l:
                    return False
        return True
    except (KeyError, IndexError, ValueError, np.linalg.LinAlgError):
        return False


@pytest.mark.parametrize("mode", ["rt", "eq"])
def test_calibrate_pair_wiring(mode):
    assert _calibrate_pair_pins_hold(oracle.calibrate_pair, mode)


@pytest.mark.parametrize("old,new", [
    ("b = shared_bits if e >= n_routed else bits", "b = bits"),                  # CLHA-MP width dropped
    ("return e if e < n_routed else n_routed", "return e if e < n_routed else 0"),  # shared job on a routed slot
    ("loss(w, g[\"wq\"], S[s] / n[s])", "loss(w, g[\"wq\"], S[s])"),              # layer loss under S, not S/n
    ("out[\"loss\"][e] = loss(w, g[\"wq\"], out[\"H\"][s])",
     "out[\"loss\"][e] = loss(w, g[\"wq\"], out[\"S\"][0][s] / out[\"n\"][0][s])"),   # loss under layer a only
])
def test_planted_calibrate_pair_mistakes_are_caught(old, new):
    assert _calibrate_pair_pins_hold(oracle.calibrate_pair)
    bad = _mutant(oracle.calibrate_pair, old, new)
    assert not _calibrate_pair_pins_hold(bad)


@pytest.mark.parametrize("mode", ["rt", "eq"])
def test_aggregate_of_slices_is_the_slice_of_aggregate(mode):
    """Aggregation is elementwise: the full-size parity tests combine sampled
    rows (and diagonals) of the per-layer Gram sums."""
    Sa, na, Sb, nb = _layers(34)
    H, _ = oracle.aggregate([Sa, Sb], [na, nb], mode)
    rows = [1, 7, 3]
    Hr, _ = oracle.aggregate([Sa[rows], Sb[rows]], [na, nb], mode)
    Hd, _ = oracle.aggregate([np.diag(Sa), np.diag(Sb)], [na, nb], mode)
    assert np.array_equal(H[rows], Hr) and np.array_equal(np.diag(H), Hd)
