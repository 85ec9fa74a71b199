"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded inputs.

Bars: routing indices, counts, offsets and token lists bit-exact; Gram sums and
combined Hessians within 1e-4 (error normalised by sqrt(H_ii H_jj)); GPTQ codes
identical on >= 99.9% of entries; losses within 1e-3 relative.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import (CODE_AGREE, HESS_TOL, LOSS_RTOL, SCALE_RTOL, agree, bits_to_dev, dev, hess_err,
                      run_group, to_dev, weights_to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_calibration_moe_amd  # noqa: F401  (fails loudly if the library is missing)


def small(wid=1, **kw):
    return gen.WORKLOADS[wid].scaled(**kw)


def _jobs(wl, experts, pair=0):
    return {e: gen.expert_weights(wl, pair, e) for e in experts}


def _oracle(wl, inp, jobs, **kw):
    jv = {e: gen.weights_value(wl, w) for e, w in jobs.items()}
    return oracle.calibrate_pair(inp["x"], inp["logits"], jv, n_routed=wl.n_routed,
                                 top_k=wl.top_k, n_shared=wl.n_shared, mode=kw.pop("mode", wl.alpha),
                                 bits=wl.bits, shared_bits=wl.shared_bits, group=wl.group,
                                 damp=wl.damp, block=128, **kw)


# --------------------------------------------------------------------------- routing

ROUTE_CASES = [
    dict(wid=1),                                                        # tiny CLWS pair
    dict(wid=1, n_tokens=3001, n_routed=64, top_k=6, n_shared=2),       # ragged, E=64, K=6
    dict(wid=1, n_tokens=2500, n_routed=128, top_k=8),                  # E=128, K=8
    dict(wid=1, n_tokens=777, n_routed=5, top_k=5),                     # K = E
    dict(wid=1, n_tokens=1500, n_routed=256, top_k=16),                 # largest E and K
    dict(wid=1, n_tokens=300, n_routed=1, top_k=1),                     # one expert
]


@pytest.mark.parametrize("case", ROUTE_CASES)
def test_route_and_bucket_bit_exact(case):
    wl = small(**case)
    inp = gen.pair_inputs(wl)
    r = run_group(wl, inp, {})
    for l in range(2):
        tk = oracle.route(inp["logits"][l], wl.top_k)
        counts, offsets, ids = oracle.bucket(tk, wl.n_routed)
        assert (r["topk"][l] == tk).all()
        assert (r["offsets"][l] == offsets).all()
        assert (r["token_ids"][l] == ids).all()
        assert (r["counts"][l][:wl.n_routed] == counts).all()
        if wl.n_shared:
            assert r["counts"][l][wl.n_routed] == wl.n_tokens


def test_route_ties_bit_exact():
    wl = small(n_tokens=2048, n_routed=16, top_k=4)
    inp = gen.pair_inputs(wl)
    rng = np.random.default_rng(3)
    lg = (rng.integers(-2, 3, (2048, 16)) * 0.5).astype(np.float32)   # many exact ties
    lg[::7, 3] = -0.0
    inp["logits"] = [lg, lg.copy()]
    r = run_group(wl, inp, {})
    assert (r["topk"][0] == oracle.route(lg, 4)).all()


# --------------------------------------------------------------------------- Gram sums

HESS_CASES = [
    dict(wid=1),                                                           # d=256, 2 tiles
    dict(wid=1, d=384, n_tokens=3000, n_routed=5, top_k=2, n_shared=1),   # 3 tiles, ragged, shared
    dict(wid=2, d=256, n_tokens=2222, n_routed=8, top_k=3, n_shared=2),   # Student-t
]


@pytest.mark.parametrize("case", HESS_CASES)
def test_hessians(case):
    wl = small(**case)
    inp = gen.pair_inputs(wl)
    r = run_group(wl, inp, {})
    for l in range(2):
        tk = oracle.route(inp["logits"][l], wl.top_k)
        S, counts = oracle.layer_hessians(inp["x"][l], tk, wl.n_routed, wl.n_shared)
        assert (r["counts"][l] == counts).all()
        for s in range(wl.n_slots):
            assert hess_err(r["S"][l][s], S[s]) <= HESS_TOL, (l, s)
            assert np.all(np.triu(r["S"][l][s], 1) == 0)   # upper triangle never written


def test_chunked_collection_matches_single_call():
    """Resume/chunking: 16 calls on consecutive token ranges equal one call."""
    wl = small(n_tokens=4096, n_routed=8, top_k=2, n_shared=1)
    inp = gen.pair_inputs(wl)
    one = run_group(wl, inp, {})
    many = run_group(wl, inp, {}, chunks=16)
    for l in range(2):
        assert (one["counts"][l] == many["counts"][l]).all()
        for s in range(wl.n_slots):
            assert hess_err(many["S"][l][s], one["S"][l][s].astype(np.float64)) <= HESS_TOL


def test_layers_keep_separate_accumulators():
    """The hook-ambiguity fix (CLHA section 2.4): S of layer a sees layer a's tokens only."""
    import gptq_calibration_moe_amd as clha
    wl = small(n_tokens=1024, n_routed=4, top_k=2)
    inp = gen.pair_inputs(wl)
    r = run_group(wl, inp, {})
    tk = oracle.route(inp["logits"][0], 2)
    S, _ = oracle.layer_hessians(inp["x"][0], tk, 4, 0)
    for s in range(4):
        assert hess_err(r["S"][0][s], S[s]) <= HESS_TOL
    ctx = r["ctx"]
    S0, n0 = r["cal"].S[0], r["cal"].counts[0]
    with pytest.raises(clha.ClhaError) as ei:
        ctx.register_layer(5, S0, torch.zeros_like(n0))
    assert ei.value.status == clha.ERR_INVALID_ARG
    with pytest.raises(clha.ClhaError):
        ctx.register_layer(6, torch.zeros_like(S0), n0)
    with pytest.raises(clha.ClhaError) as ei:
        ctx.collect_hessians(9, bits_to_dev(inp["x"][0]), to_dev(inp["logits"][0]))
    assert ei.value.status == clha.ERR_INVALID_ARG


# --------------------------------------------------------------------------- aggregation

@pytest.mark.parametrize("mode,alpha", [("rt", None), ("eq", None), ("explicit", [0.3, 0.7])])
def test_aggregate(mode, alpha):
    wl = small(n_tokens=3000, n_routed=6, top_k=2, n_shared=1)
    inp = gen.pair_inputs(wl)
    r = run_group(wl, inp, {}, mode=mode, alpha=alpha)
    S, n = [], []
    for l in range(2):
        tk = oracle.route(inp["logits"][l], wl.top_k)
        s_l, c_l = oracle.layer_hessians(inp["x"][l], tk, wl.n_routed, wl.n_shared)
        S.append(s_l)
        n.append(c_l)
    for s in range(wl.n_slots):
        H, a = oracle.aggregate([S[0][s], S[1][s]], [n[0][s], n[1][s]], mode, alpha)
        assert hess_err(r["H"][s], H) <= HESS_TOL, s
        assert (r["H"][s] == r["H"][s].T).all()
        np.testing.assert_allclose(r["alpha"][s], a, rtol=1e-6)


def test_plic_and_identical_layers_bitwise():
    """alpha = (1, 0) gives H_a bit for bit; identical layers give H_a under rt and eq."""
    wl = small(n_tokens=2048, n_routed=4, top_k=2)
    inp = gen.pair_inputs(wl)
    plic = run_group(wl, inp, {}, mode="rt", agg_layers=[0])
    ex = run_group(wl, inp, {}, mode="explicit", alpha=[1.0, 0.0])
    assert (plic["H"] == ex["H"]).all()
    same = {"x": [inp["x"][0], inp["x"][0].copy()], "logits": [inp["logits"][0], inp["logits"][0].copy()]}
    for mode in ("rt", "eq"):
        r = run_group(wl, same, {}, mode=mode)
        assert (r["H"] == plic["H"]).all(), mode


# --------------------------------------------------------------------------- inverse Cholesky

def _spd(seed, c, spread=3.0, dead=()):
    rng = np.random.default_rng(seed)
    x = gen.bf16_value(gen.structured_activations(seed, 4 * c, c, spread, dead_cols=dead))
    return oracle.gram(x) / (4 * c)


@pytest.mark.parametrize("c,dead", [(128, ()), (256, (5, 200)), (512, ())])
def test_inverse_cholesky(c, dead):
    import gptq_calibration_moe_amd as clha
    Hs = [_spd(40 + i, c, dead=dead) for i in range(3)]
    ctx = clha.Context(c if c % 128 == 0 else 128, 4, 2, 0, 16, device=dev())
    Hd = [to_dev(h.astype(np.float32)) for h in Hs]
    U = torch.zeros(3, c, c, dtype=torch.float32, device=dev())
    lam = torch.empty(3, dtype=torch.float32, device=dev())
    dd = torch.empty(3, c, dtype=torch.uint8, device=dev())
    ctx.inverse_cholesky(Hd, U, 0.01, lam, dd)
    ctx.sync()
    U, lam, dd = U.cpu().numpy(), lam.cpu().numpy(), dd.cpu().numpy()
    for i, H in enumerate(Hs):
        H32 = H.astype(np.float32).astype(np.float64)
        # dead columns, lambda and U as the oracle's GPTQ makes them (one zero row)
        ref = oracle.gptq(np.zeros((1, c)), H32, 2, 64, damp=0.01, block=64)
        assert (dd[i].astype(bool) == ref["dead"]).all()
        assert abs(lam[i] - ref["lam"]) <= 1e-6 * ref["lam"]
        hd = H32.copy()
        hd[ref["dead"], ref["dead"]] = 1.0
        hd += ref["lam"] * np.eye(c)
        Uref = ref["U"]
        # the factor is computed in fp64 and rounded to fp32 once
        err = np.max(np.abs(np.triu(U[i]) - Uref)) / np.max(np.abs(Uref))
        assert err < 1e-6, err
        res = np.abs(np.triu(U[i]).T @ np.triu(U[i]) @ hd - np.eye(c)).max()
        assert res < 1e-3, res


def test_not_positive_definite_is_latched():
    import gptq_calibration_moe_amd as clha
    c = 128
    H = np.eye(c, dtype=np.float32)
    H[3, 3] = -5.0                      # indefinite even after damping
    ctx = clha.Context(128, 4, 2, 0, 16, device=dev())
    U = torch.zeros(1, c, c, dtype=torch.float32, device=dev())
    ctx.inverse_cholesky([to_dev(H)], U, 0.01)
    with pytest.raises(clha.ClhaError) as ei:
        ctx.sync()
    assert ei.value.status == clha.ERR_NOT_PD
    ctx.sync()                          # the latch is cleared


def test_nonfinite_logits_are_latched():
    import gptq_calibration_moe_amd as clha
    wl = small(n_tokens=512, n_routed=8, top_k=2)
    inp = gen.pair_inputs(wl)
    lg = inp["logits"][0].copy()
    lg[17, 3] = np.nan
    ctx = clha.Context(wl.d, 8, 2, 0, 512, device=dev())
    S, n = ctx.new_layer_buffers()
    ctx.register_layer(0, S, n)
    ctx.collect_hessians(0, bits_to_dev(inp["x"][0]), to_dev(lg))
    with pytest.raises(clha.ClhaError) as ei:
        ctx.sync()
    assert ei.value.status == clha.ERR_NONFINITE


def test_argument_errors():
    import gptq_calibration_moe_amd as clha
    ctx = clha.Context(256, 8, 2, 0, 1024, device=dev())
    S, n = ctx.new_layer_buffers()
    ctx.register_layer(0, S, n)
    x = torch.zeros(2048, 256, dtype=torch.bfloat16, device=dev())
    lg = torch.zeros(2048, 8, dtype=torch.float32, device=dev())
    with pytest.raises(clha.ClhaError) as ei:
        ctx.collect_hessians(0, x, lg)                         # more tokens than max_tokens
    assert ei.value.status == clha.ERR_SHAPE
    H = torch.eye(256, dtype=torch.float32, device=dev())
    W = torch.zeros(64, 256, dtype=torch.float32, device=dev())
    job = {"H": H, "W": W, "bits": 2, "codes": torch.empty(64, 256, dtype=torch.uint8, device=dev()),
           "scales": torch.empty(64, 2, dtype=torch.float32, device=dev()),
           "zeros": torch.empty(64, 2, dtype=torch.uint8, device=dev())}
    with pytest.raises(clha.ClhaError) as ei:
        ctx.gptq_quantize([job], 256, group=96, block=128)     # group does not divide block
    assert ei.value.status == clha.ERR_SHAPE
    with pytest.raises(clha.ClhaError) as ei:
        ctx.gptq_quantize([dict(job, bits=9)], 256, group=128, block=128)
    assert ei.value.status == clha.ERR_SHAPE
    with pytest.raises(clha.ClhaError) as ei:
        ctx.aggregate([0, 7], "rt", torch.empty(8, 256, 256, device=dev()))   # unregistered layer
    assert ei.value.status == clha.ERR_INVALID_ARG


# --------------------------------------------------------------------------- GPTQ

def _gptq_case(seed, rows, c, bits, group, dead=(), w_dtype="f32", spread=3.0):
    H = _spd(seed, c, spread, dead).astype(np.float32)
    rng = np.random.default_rng(seed + 1000)
    W = rng.normal(0, 0.02, (rows, c)).astype(np.float32)
    if w_dtype == "bf16":
        Wst = gen.bf16_bits(W)
        Wv = gen.bf16_value(Wst)
    else:
        Wst, Wv = W, W
    return H, Wst, Wv


@pytest.mark.parametrize("seed,rows,c,bits,group,block,wdt,dead", [
    (50, 64, 256, 2, 128, 128, "f32", ()),
    (51, 200, 384, 3, 64, 128, "bf16", (7,)),        # ragged rows, 3 blocks, 2 groups per block
    (52, 130, 256, 4, 32, 64, "f32", ()),            # block 64, small groups
    (53, 96, 512, 2, 128, 128, "bf16", (0, 300)),
    (54, 64, 128, 8, 128, 128, "f32", ()),           # 8 bits, a single block
    (55, 96, 256, 2, 16, 128, "f32", ()),            # small groups
    (56, 70, 128, 3, 4, 64, "bf16", (100,)),         # group 4, ragged rows, dead column
    (57, 300, 1024, 2, 128, 128, "bf16", ()),        # 5 slabs, 16 register blocks
    (58, 130, 448, 3, 32, 64, "bf16", (300,)),       # trailing tiles of 128 and 64 columns, dead
                                                     # column in the first trailing fill
    (59, 65, 320, 2, 64, 64, "f32", ()),             # one trailing tile of 64 columns, 2 slabs
])
def test_gptq_stage(seed, rows, c, bits, group, block, wdt, dead):
    import gptq_calibration_moe_amd as clha
    H, Wst, Wv = _gptq_case(seed, rows, c, bits, group, dead, wdt)
    ref = oracle.gptq(Wv, H.astype(np.float64), bits, group, 0.01, 128)
    ctx = clha.Context(c if c % 128 == 0 else 128, 4, 2, 0, 16, device=dev())
    Wd = to_dev(Wst.view(np.int16)).view(torch.bfloat16) if wdt == "bf16" else to_dev(Wst)
    job = {"H": to_dev(H), "W": Wd, "bits": bits,
           "codes": torch.empty(rows, c, dtype=torch.uint8, device=dev()),
           "scales": torch.empty(rows, c // group, dtype=torch.float32, device=dev()),
           "zeros": torch.empty(rows, c // group, dtype=torch.uint8, device=dev()),
           "loss": torch.empty(1, dtype=torch.float32, device=dev())}
    ctx.gptq_quantize([job], c, group, block, 0.01)
    ctx.sync()
    codes = job["codes"].cpu().numpy()
    assert agree(codes, ref["codes"]) >= CODE_AGREE
    assert codes.max() <= (1 << bits) - 1
    ok = (codes == ref["codes"]).all(axis=1)
    if ok.any():
        np.testing.assert_allclose(job["scales"].cpu().numpy()[ok], ref["scales"][ok], rtol=SCALE_RTOL)
        assert (job["zeros"].cpu().numpy()[ok] == ref["zeros"][ok]).all()
    want = oracle.loss(Wv, ref["wq"], H.astype(np.float64))
    got = float(job["loss"].cpu().numpy()[0])
    assert abs(got - want) <= LOSS_RTOL * want, (got, want)
    # explicit loss kernel on the GPU's own codes vs the oracle's loss of those codes
    lo = torch.empty(1, dtype=torch.float32, device=dev())
    ctx.loss(Wd, job["codes"], job["scales"], job["zeros"], job["H"], group, lo)
    ctx.sync()
    wq = oracle.dequantize(codes, job["scales"].cpu().numpy(), job["zeros"].cpu().numpy(), group)
    want2 = oracle.loss(Wv, wq, H.astype(np.float64))
    assert abs(float(lo.cpu().numpy()[0]) - want2) <= 1e-4 * want2


def test_gptq_diagonal_hessian_is_rtn():
    import gptq_calibration_moe_amd as clha
    c, rows = 256, 64
    rng = np.random.default_rng(60)
    H = np.diag(rng.uniform(0.5, 2.0, c)).astype(np.float32)
    W = rng.normal(0, 0.02, (rows, c)).astype(np.float32)
    ref = oracle.gptq(W, H.astype(np.float64), 2, 128, 0.01, 128)
    ctx = clha.Context(c, 4, 2, 0, 16, device=dev())
    job = {"H": to_dev(H), "W": to_dev(W), "bits": 2,
           "codes": torch.empty(rows, c, dtype=torch.uint8, device=dev()),
           "scales": torch.empty(rows, 2, dtype=torch.float32, device=dev()),
           "zeros": torch.empty(rows, 2, dtype=torch.uint8, device=dev())}
    ctx.gptq_quantize([job], c, 128, 128, 0.01)
    ctx.sync()
    assert (job["codes"].cpu().numpy() == ref["codes"]).all()


# --------------------------------------------------------------------------- end to end

def _e2e(wl, inp, experts, mode=None, **kw):
    jobs = _jobs(wl, experts)
    ref = _oracle(wl, inp, jobs, mode=mode or wl.alpha, layer_losses=False)
    r = run_group(wl, inp, jobs, mode=mode or wl.alpha, **kw)
    for l in range(2):
        assert (r["topk"][l] == ref["topk"][l]).all()
        assert (r["counts"][l][:wl.n_routed] == ref["counts"][l]).all()
    for s, H in ref["H"].items():
        assert hess_err(r["H"][s], H) <= HESS_TOL, s
    for e in experts:
        g, o = r["gptq"][e], ref["gptq"][e]
        assert agree(g["codes"], o["codes"]) >= CODE_AGREE, e
        got, want = float(g["loss"][0]), ref["loss"][e]
        assert abs(got - want) <= LOSS_RTOL * want, (e, got, want)
    return r, ref


def test_end_to_end_tiny_clws_pair():
    wl = gen.WORKLOADS[1]
    _e2e(wl, gen.pair_inputs(wl), list(range(wl.n_experts_total)))


def test_end_to_end_clha_mp_small():
    """CLHA-MP: shared experts at b+1 bits against the all-token Hessian."""
    wl = gen.WORKLOADS[4].scaled(d=256, n_tokens=4096, n_routed=8, top_k=2, rows=96, n_pairs=1)
    r, ref = _e2e(wl, gen.pair_inputs(wl), [0, 3, 8, 9])
    for e in (8, 9):                      # shared experts: the 3-bit range is used
        assert 4 <= r["gptq"][e]["codes"].max() <= 7, e
    for e in (0, 3):                      # routed experts stay at 2 bits
        assert r["gptq"][e]["codes"].max() <= 3, e


def test_drift_zero_clha_equals_plic_bitwise():
    wl = gen.WORKLOADS[5].scaled(d=256, n_tokens=4096, n_routed=8, top_k=2, rows=64)
    inp = gen.pair_inputs(wl, t=0.0)
    jobs = _jobs(wl, [0, 5])
    plic = run_group(wl, inp, jobs, mode="rt", agg_layers=[0])
    for mode in ("rt", "eq"):
        r = run_group(wl, inp, jobs, mode=mode)
        for e in jobs:
            assert (r["gptq"][e]["codes"] == plic["gptq"][e]["codes"]).all()


def test_runs_are_bit_identical():
    wl = small(n_tokens=4096, n_routed=8, top_k=2, n_shared=1, rows=128)
    inp = gen.pair_inputs(wl)
    jobs = _jobs(wl, [1, 8])
    a = run_group(wl, inp, jobs, mode="rt")
    b = run_group(wl, inp, jobs, mode="rt")
    for l in range(2):
        assert (a["S"][l] == b["S"][l]).all()
    assert (a["H"] == b["H"]).all()
    for e in jobs:
        for k in ("codes", "scales", "zeros", "loss"):
            assert (a["gptq"][e][k] == b["gptq"][e][k]).all()
