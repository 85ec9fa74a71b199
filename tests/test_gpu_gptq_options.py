"""GPTQ's activation-order and static-group options on the HIP path (through
clha_gptq_quantize_ex) against the CPU oracle.

Bars: g_idx bit-exact (the processing order is decided from the same fp32
H_ii on both sides); codes identical on >= 99.9% of entries; static grids
bit-exact (fitted in fp32 from the same weights before any update); other grids
as in the plain GPTQ tests; the returned loss within 1e-3 of the oracle's loss
of the oracle's W_q and of the GPU's own W_q.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import CODE_AGREE, LOSS_RTOL, SCALE_RTOL, agree, dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_calibration_moe_amd  # noqa: F401  (fails loudly if the library is missing)


def _hessian(seed, c, dead=(), ties=0):
    x = gen.bf16_value(gen.structured_activations(seed, 4 * c, c, 3.0, dead_cols=dead))
    H = oracle.gram(x) / (4 * c)
    if ties:
        # raise a few diagonal entries to one common value: still positive
        # definite, and the order has ties to break by column index
        rng = np.random.default_rng(seed + 7)
        idx = rng.choice([i for i in range(c) if i not in dead], ties, replace=False)
        H[idx, idx] = np.max(np.diag(H)[idx])
    return H.astype(np.float32)


def _weights(seed, rows, c, wdt):
    W = np.random.default_rng(seed + 1000).normal(0, 0.02, (rows, c)).astype(np.float32)
    if wdt == "bf16":
        bits = gen.bf16_bits(W)
        return to_dev(bits.view(np.int16)).view(torch.bfloat16), gen.bf16_value(bits)
    return to_dev(W), W.astype(np.float64)


def _job(H_dev, Wd, rows, c, bits, group):
    return {"H": H_dev, "W": Wd, "bits": bits,
            "codes": torch.empty(rows, c, dtype=torch.uint8, device=dev()),
            "scales": torch.empty(rows, c // group, dtype=torch.float32, device=dev()),
            "zeros": torch.empty(rows, c // group, dtype=torch.uint8, device=dev()),
            "loss": torch.empty(1, dtype=torch.float32, device=dev()),
            "g_idx": torch.empty(c, dtype=torch.int32, device=dev())}


def _check(job, ref, Wv, H, bits, group, static):
    codes = job["codes"].cpu().numpy()
    gi = job["g_idx"].cpu().numpy()
    sc, zp = job["scales"].cpu().numpy(), job["zeros"].cpu().numpy()
    assert (gi == ref["g_idx"]).all()
    assert agree(codes, ref["codes"]) >= CODE_AGREE
    assert codes.max() <= (1 << bits) - 1
    if static:
        assert (sc == ref["scales"]).all() and (zp == ref["zeros"]).all()
    else:
        ok = (codes == ref["codes"]).all(axis=1)
        if ok.any():
            np.testing.assert_allclose(sc[ok], ref["scales"][ok], rtol=SCALE_RTOL)
            assert (zp[ok] == ref["zeros"][ok]).all()
    got = float(job["loss"].cpu().numpy()[0])
    want = oracle.loss(Wv, ref["wq"], H.astype(np.float64))
    assert abs(got - want) <= LOSS_RTOL * want, (got, want)
    own = oracle.loss(Wv, oracle.dequantize_idx(codes, sc, zp, gi), H.astype(np.float64))
    assert abs(got - own) <= LOSS_RTOL * own, (got, own)


OPTIONS = [(True, False), (False, True), (True, True)]


@pytest.mark.parametrize("act,static", OPTIONS)
@pytest.mark.parametrize("seed,rows,c,bits,group,block,wdt,dead,ties", [
    (70, 200, 384, 3, 64, 128, "bf16", (7,), 0),        # ragged rows, dead column
    (71, 130, 256, 4, 32, 64, "f32", (), 6),            # block 64, ties in H_ii
    (72, 300, 1024, 2, 128, 128, "bf16", (0, 600), 0),  # 5 slabs, 4 superblocks
    (73, 70, 128, 3, 4, 64, "bf16", (100,), 3),         # group 4, one superblock
])
def test_gptq_options(act, static, seed, rows, c, bits, group, block, wdt, dead, ties):
    import gptq_calibration_moe_amd as clha
    print(f"gptq options act={act} static={static} seed={seed} rows={rows} c={c} group={group}", flush=True)
    H = _hessian(seed, c, dead, ties)
    Wd, Wv = _weights(seed, rows, c, wdt)
    ref = oracle.gptq(Wv, H.astype(np.float64), bits, group, 0.01, 128, act_order=act, static_groups=static)
    ctx = clha.Context(c if c % 128 == 0 else 128, 4, 2, 0, 16, device=dev())
    job = _job(to_dev(H), Wd, rows, c, bits, group)
    ctx.gptq_quantize([job], c, group, block, 0.01, act_order=act, static_groups=static)
    ctx.sync()
    _check(job, ref, Wv, H, bits, group, static)


@pytest.mark.parametrize("act,static", OPTIONS)
def test_gptq_options_several_hessians(act, static):
    """Three jobs in one call: two share a Hessian (one factorisation, one
    order), the third has its own."""
    import gptq_calibration_moe_amd as clha
    print(f"gptq options several Hessians act={act} static={static}", flush=True)
    c, group = 512, 128
    Hs = [_hessian(80, c, (3,), 4), _hessian(81, c)]
    Hd = [to_dev(h) for h in Hs]
    specs = [(0, 192, 3, 82, "bf16"), (1, 100, 2, 83, "f32"), (0, 64, 4, 84, "f32")]
    ctx = clha.Context(c, 4, 2, 0, 16, device=dev())
    jobs, refs = [], []
    for h, rows, bits, seed, wdt in specs:
        Wd, Wv = _weights(seed, rows, c, wdt)
        jobs.append(_job(Hd[h], Wd, rows, c, bits, group))
        refs.append((oracle.gptq(Wv, Hs[h].astype(np.float64), bits, group, 0.01, 128,
                                 act_order=act, static_groups=static), Wv, Hs[h], bits))
    ctx.gptq_quantize(jobs, c, group, 128, 0.01, act_order=act, static_groups=static)
    ctx.sync()
    for job, (ref, Wv, H, bits) in zip(jobs, refs):
        _check(job, ref, Wv, H, bits, group, static)


def test_options_off_is_plain_gptq_bitwise():
    """clha_gptq_quantize_ex with no flags (a g_idx output requested) returns
    exactly what clha_gptq_quantize returns, and g_idx = column // group."""
    import gptq_calibration_moe_amd as clha
    c, rows, group = 256, 96, 64
    H = _hessian(90, c)
    Wd, _ = _weights(90, rows, c, "f32")
    ctx = clha.Context(c, 4, 2, 0, 16, device=dev())
    a = _job(to_dev(H), Wd, rows, c, 3, group)
    b = _job(to_dev(H), Wd, rows, c, 3, group)
    del a["g_idx"]
    ctx.gptq_quantize([a], c, group, 128, 0.01)
    ctx.gptq_quantize([b], c, group, 128, 0.01)       # routed through the _ex entry point
    ctx.sync()
    for k in ("codes", "scales", "zeros", "loss"):
        assert torch.equal(a[k], b[k]), k
    assert (b["g_idx"].cpu().numpy() == np.arange(c) // group).all()


def test_static_diagonal_act_order_is_rtn():
    """A diagonal H propagates nothing: with static groups the codes are
    round-to-nearest on the natural groups whatever the order."""
    import gptq_calibration_moe_amd as clha
    c, rows, group, bits = 256, 64, 32, 3
    rng = np.random.default_rng(91)
    H = np.diag(rng.uniform(0.5, 2.0, c)).astype(np.float32)
    W = rng.normal(0, 0.02, (rows, c)).astype(np.float32)
    ctx = clha.Context(c, 4, 2, 0, 16, device=dev())
    job = _job(to_dev(H), to_dev(W), rows, c, bits, group)
    ctx.gptq_quantize([job], c, group, 128, 0.01, act_order=True, static_groups=True)
    ctx.sync()
    maxq = (1 << bits) - 1
    want = np.zeros((rows, c), np.uint8)
    for g0 in range(0, c, group):
        s, z = oracle.quant_params(W[:, g0:g0 + group], maxq)
        for j in range(g0, g0 + group):
            want[:, j] = oracle.quantize(W[:, j], s, z, maxq)
    assert (job["codes"].cpu().numpy() == want).all()


def test_option_argument_errors():
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd import lib
    import ctypes as C
    c, rows = 256, 64
    ctx = clha.Context(c, 4, 2, 0, 16, device=dev())
    job = _job(to_dev(np.eye(c, dtype=np.float32)), to_dev(np.zeros((rows, c), np.float32)), rows, c, 2, 128)
    arr = ctx._jobs([job], c)
    ws = torch.empty(int(lib.clha_gptq_workspace_bytes_ex(ctx._h, 1, arr, c, 3)), dtype=torch.uint8, device=dev())
    st = lib.clha_gptq_quantize_ex(ctx._h, 1, arr, c, 128, 128, 0.01, 4, None, ws.data_ptr(), ws.numel(), None)
    assert st == clha.ERR_INVALID_ARG                   # unknown flag
    bad = (C.c_void_p * 1)(job["g_idx"].data_ptr() + 2)
    st = lib.clha_gptq_quantize_ex(ctx._h, 1, arr, c, 128, 128, 0.01, 1, bad, ws.data_ptr(), ws.numel(), None)
    assert st == clha.ERR_ALIGN                         # misaligned g_idx
    st = lib.clha_gptq_quantize_ex(ctx._h, 1, arr, c, 128, 128, 0.01, 1, None, ws.data_ptr(), 256, None)
    assert st == clha.ERR_WORKSPACE                     # the permuted Hessian does not fit


def test_act_order_with_equal_diagonal_is_plain_gptq_bitwise():
    """All H_ii equal: every key ties, the order is the natural one, and the
    permuted Hessian is H itself, so activation order returns exactly the plain
    result (and g_idx = column // group)."""
    import gptq_calibration_moe_amd as clha
    c, rows, group = 256, 130, 32
    H = _hessian(92, c)
    np.fill_diagonal(H, np.max(np.diag(H)))       # raising the diagonal keeps H positive definite
    Wd, _ = _weights(92, rows, c, "bf16")
    ctx = clha.Context(c, 4, 2, 0, 16, device=dev())
    a = _job(to_dev(H), Wd, rows, c, 3, group)
    b = _job(to_dev(H), Wd, rows, c, 3, group)
    ctx.gptq_quantize([a], c, group, 128, 0.01)
    ctx.gptq_quantize([b], c, group, 128, 0.01, act_order=True)
    ctx.sync()
    for k in ("codes", "scales", "zeros", "loss"):
        assert torch.equal(a[k], b[k]), k
    assert (b["g_idx"].cpu().numpy() == np.arange(c) // group).all()


def test_options_runs_are_bit_identical():
    import gptq_calibration_moe_amd as clha
    c, rows, group = 512, 200, 64
    H = _hessian(93, c, (11,), 5)
    Wd, _ = _weights(93, rows, c, "bf16")
    ctx = clha.Context(c, 4, 2, 0, 16, device=dev())
    runs = []
    for _ in range(2):
        j = _job(to_dev(H), Wd, rows, c, 3, group)
        ctx.gptq_quantize([j], c, group, 128, 0.01, act_order=True, static_groups=True)
        runs.append(j)
    ctx.sync()
    for k in ("codes", "scales", "zeros", "loss", "g_idx"):
        assert torch.equal(runs[0][k], runs[1][k]), k
