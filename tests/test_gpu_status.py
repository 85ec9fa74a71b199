"""Per-job numerical status at the C ABI (GPTQ phase of the CLHA summary,
section 2.2: GPTQ runs once per shared weight, so one failing Hessian must not
hide which weight failed or spoil the others).

* One indefinite Hessian among three jobs: only its job reports NOT_PD, the
  context latch names that job, and the other two jobs match the oracle.
* A NaN on a Hessian's diagonal reports NONFINITE for its job.
* The optional second Hessian of a job (H_eval) gives the loss of the result
  under that Hessian, against the oracle's loss of the same codes; the dead
  flags come back in natural column order.
* A non-finite router logit names its layer.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import CODE_AGREE, LOSS_RTOL, agree, bits_to_dev, dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_calibration_moe_amd  # noqa: F401  (fails loudly if the library is missing)


def _spd(seed, c, dead=()):
    x = gen.bf16_value(gen.structured_activations(seed, 4 * c, c, 3.0, dead_cols=dead))
    return (oracle.gram(x) / (4 * c)).astype(np.float32)


def _job(H, W, bits, group, H_eval=None):
    rows, c = W.shape
    j = {"H": to_dev(H), "W": to_dev(W), "bits": bits,
         "codes": torch.empty(rows, c, dtype=torch.uint8, device=dev()),
         "scales": torch.empty(rows, c // group, dtype=torch.float32, device=dev()),
         "zeros": torch.empty(rows, c // group, dtype=torch.uint8, device=dev()),
         "loss": torch.empty(1, dtype=torch.float32, device=dev()),
         "dead": torch.empty(c, dtype=torch.uint8, device=dev()),
         "status": torch.full((1,), -1, dtype=torch.int32, device=dev())}
    if H_eval is not None:
        j["H_eval"] = to_dev(H_eval)
        j["loss_eval"] = torch.empty(1, dtype=torch.float32, device=dev())
    return j


def test_one_indefinite_hessian_among_three_jobs():
    import gptq_calibration_moe_amd as clha
    print("per-job status: jobs 0 and 2 valid, job 1 indefinite", flush=True)
    c, rows, bits, group = 256, 96, 2, 128
    H0, H2 = _spd(70, c, dead=(9,)), _spd(72, c)
    H1 = np.eye(c, dtype=np.float32)
    H1[5, 5] = -5.0                                     # indefinite even after damping
    rng = np.random.default_rng(73)
    W = [rng.normal(0, 0.02, (rows, c)).astype(np.float32) for _ in range(3)]
    jobs = [_job(H0, W[0], bits, group, H_eval=H2), _job(H1, W[1], bits, group), _job(H2, W[2], bits, group)]
    ctx = clha.Context(c, 4, 2, 0, 16, device=dev())
    ctx.gptq_quantize(jobs, c, group, 128, 0.01)
    with pytest.raises(clha.ClhaError) as ei:
        ctx.sync()
    assert ei.value.status == clha.ERR_NOT_PD
    assert "GPTQ job 1" in str(ei.value) and "Hessian 1" in str(ei.value), str(ei.value)
    ctx.sync()                                          # the record is cleared
    assert [int(j["status"].cpu()[0]) for j in jobs] == [clha.OK, clha.ERR_NOT_PD, clha.OK]
    for i in (0, 2):
        H = (H0, None, H2)[i]
        ref = oracle.gptq(W[i].astype(np.float64), H.astype(np.float64), bits, group, 0.01, 128)
        codes = jobs[i]["codes"].cpu().numpy()
        assert agree(codes, ref["codes"]) >= CODE_AGREE, i
        want = oracle.loss(W[i], ref["wq"], H.astype(np.float64))
        got = float(jobs[i]["loss"].cpu()[0])
        assert abs(got - want) <= LOSS_RTOL * want, (i, got, want)
        assert np.array_equal(jobs[i]["dead"].cpu().numpy().astype(bool), np.diag(H) == 0), i
    # job 0's result under a second Hessian: the oracle's loss of the GPU's own codes
    wq = oracle.dequantize(jobs[0]["codes"].cpu().numpy(), jobs[0]["scales"].cpu().numpy(),
                           jobs[0]["zeros"].cpu().numpy(), group)
    want = oracle.loss(W[0], wq, H2.astype(np.float64))
    got = float(jobs[0]["loss_eval"].cpu()[0])
    assert abs(got - want) <= 1e-4 * want, (got, want)


def test_nonfinite_hessian_diagonal():
    import gptq_calibration_moe_amd as clha
    print("per-job status: a NaN on job 0's diagonal", flush=True)
    c, rows = 128, 64
    Hbad = _spd(74, c)
    Hbad[17, 17] = np.nan
    rng = np.random.default_rng(75)
    W = rng.normal(0, 0.02, (rows, c)).astype(np.float32)
    jobs = [_job(Hbad, W, 3, 64), _job(_spd(76, c), W, 3, 64)]
    ctx = clha.Context(c, 4, 2, 0, 16, device=dev())
    ctx.gptq_quantize(jobs, c, 64, 128, 0.01)
    with pytest.raises(clha.ClhaError) as ei:
        ctx.sync()
    assert ei.value.status == clha.ERR_NONFINITE and "GPTQ job 0" in str(ei.value), str(ei.value)
    assert [int(j["status"].cpu()[0]) for j in jobs] == [clha.ERR_NONFINITE, clha.OK]


def test_nonfinite_logit_names_its_layer():
    import gptq_calibration_moe_amd as clha
    print("a NaN router logit in layer 7", flush=True)
    wl = gen.WORKLOADS[1].scaled(n_tokens=512)
    inp = gen.pair_inputs(wl)
    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, 0, 512, device=dev())
    for l in (6, 7):
        S, n = ctx.new_layer_buffers()
        ctx.register_layer(l, S, n)
    lg = inp["logits"][1].copy()
    lg[100, 2] = np.inf
    ctx.collect_hessians(6, bits_to_dev(inp["x"][0]), to_dev(inp["logits"][0]))
    ctx.collect_hessians(7, bits_to_dev(inp["x"][1]), to_dev(lg))
    with pytest.raises(clha.ClhaError) as ei:
        ctx.sync()
    assert ei.value.status == clha.ERR_NONFINITE and "layer 7" in str(ei.value), str(ei.value)
    ctx.sync()


def test_contexts_do_not_share_status_records():
    """A failure latched in one context is not seen by another on the same device."""
    import gptq_calibration_moe_amd as clha
    c = 128
    a = clha.Context(c, 4, 2, 0, 16, device=dev())
    b = clha.Context(c, 4, 2, 0, 16, device=dev())
    H = np.eye(c, dtype=np.float32)
    H[3, 3] = -5.0
    U = torch.zeros(1, c, c, dtype=torch.float32, device=dev())
    a.inverse_cholesky([to_dev(H)], U, 0.01)
    b.sync()                                            # b has nothing latched
    with pytest.raises(clha.ClhaError) as ei:
        a.sync()
    assert ei.value.status == clha.ERR_NOT_PD and "Hessian 0" in str(ei.value)
