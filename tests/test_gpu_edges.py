"""Edge cases of the HIP path through the C ABI, against the CPU oracle.

* an empty batch adds nothing;
* an expert that no token chooses: its combined Hessian is the identity
  (the reading for a slot with no tokens in any layer) and GPTQ on it is
  round-to-nearest on the same grid;
* all-zero weight rows: every group takes the (-1, 1) grid, every code is z;
* the largest hidden size, d = 8192: routing, Gram sums (sampled columns) and
  GPTQ of a 32-row matrix on a well-conditioned Hessian;
* a reset accumulator (stale sums left in S, counts zeroed) collects exactly
  what a zeroed one does, an unrouted slot included, and a layer reset but
  never collected drops out of the aggregation;
* the shared-expert slot, formed from the routed slots' sums, equals the
  oracle's X^T X over a reset layer with stale sums, an expert no token
  chooses and two batches, also when every token goes to every expert.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import (CODE_AGREE, HESS_TOL, LOSS_RTOL, SCALE_RTOL, agree, bits_to_dev, dev, hess_err,
                      to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_calibration_moe_amd  # noqa: F401  (fails loudly if the library is missing)


def _job(H, W, bits, group):
    rows, c = W.shape
    return {"H": H, "W": W, "bits": bits,
            "codes": torch.empty(rows, c, dtype=torch.uint8, device=dev()),
            "scales": torch.empty(rows, c // group, dtype=torch.float32, device=dev()),
            "zeros": torch.empty(rows, c // group, dtype=torch.uint8, device=dev()),
            "loss": torch.empty(1, dtype=torch.float32, device=dev())}


def test_empty_batch_adds_nothing():
    import gptq_calibration_moe_amd as clha
    wl = gen.WORKLOADS[1]
    inp = gen.pair_inputs(wl)
    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, wl.n_shared, wl.n_tokens, device=dev())
    S, n = ctx.new_layer_buffers()
    ctx.register_layer(0, S, n)
    ctx.collect_hessians(0, bits_to_dev(inp["x"][0]), to_dev(inp["logits"][0]))
    ctx.sync()
    S0, n0 = S.clone(), n.clone()
    ctx.collect_hessians(0, bits_to_dev(inp["x"][0][:0]), to_dev(inp["logits"][0][:0]))
    ctx.sync()
    assert torch.equal(S, S0) and torch.equal(n, n0)


def test_unrouted_expert_identity_and_rtn():
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.calibrate import SharedGroupCalibration
    wl = gen.WORKLOADS[1].scaled(n_tokens=2048)
    inp = gen.pair_inputs(wl)
    lg = [l.copy() for l in inp["logits"]]
    for l in lg:
        l[:, 7] = -100.0                     # expert 7 is never among the top 2
    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, 0, wl.n_tokens, device=dev())
    cal = SharedGroupCalibration(ctx, [0, 1])
    cal.reset()
    for l in range(2):
        cal.collect(l, bits_to_dev(inp["x"][l]), to_dev(lg[l]))
    H = cal.aggregate("rt")
    ctx.sync()
    for l in range(2):
        assert int(cal.counts[l][7]) == 0
    S_ref = [np.zeros((wl.d, wl.d)) for _ in range(2)]
    H_ref, al = oracle.aggregate(S_ref, [0, 0], "rt")
    assert np.array_equal(H[7].cpu().numpy(), H_ref.astype(np.float32))      # the identity
    assert np.all(cal.alpha[7].cpu().numpy() == 0)
    w = gen.weights_value(wl, gen.expert_weights(wl, 0, 7))
    job = _job(H[7], to_dev(w), wl.bits, wl.group)
    ctx.gptq_quantize([job], wl.d, wl.group, wl.block, wl.damp)
    ctx.sync()
    ref = oracle.gptq(w.astype(np.float64), H_ref, wl.bits, wl.group, wl.damp, wl.block)
    assert np.array_equal(job["codes"].cpu().numpy(), ref["codes"])          # RTN: no propagation
    np.testing.assert_array_equal(job["zeros"].cpu().numpy(), ref["zeros"])


def test_all_zero_weight_rows():
    import gptq_calibration_moe_amd as clha
    c, rows, bits, group = 256, 96, 3, 64
    rng = np.random.default_rng(71)
    x = gen.bf16_value(gen.structured_activations(71, 4 * c, c, 2.0))
    H = (oracle.gram(x) / (4 * c)).astype(np.float32)
    W = rng.normal(0, 0.02, (rows, c)).astype(np.float32)
    W[[0, 17, 95]] = 0.0
    ctx = clha.Context(c, 4, 2, 0, 16, device=dev())
    job = _job(to_dev(H), to_dev(W), bits, group)
    ctx.gptq_quantize([job], c, group, 128, 0.01)
    ctx.sync()
    ref = oracle.gptq(W.astype(np.float64), H.astype(np.float64), bits, group, 0.01, 128)
    codes = job["codes"].cpu().numpy()
    for r in (0, 17, 95):
        assert np.array_equal(codes[r], ref["codes"][r])
        assert np.array_equal(job["scales"].cpu().numpy()[r], ref["scales"][r])
        assert np.all(ref["codes"][r] == ref["zeros"][r][0])                    # every code is z
    assert agree(codes, ref["codes"]) >= CODE_AGREE


def test_largest_hidden_size():
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.calibrate import SharedGroupCalibration
    d, E, K, n = 8192, 4, 2, 2048
    wl = gen.WORKLOADS[1].scaled(d=d, n_routed=E, top_k=K, n_tokens=n, x_kind="normal")
    inp = gen.pair_inputs(wl)
    ctx = clha.Context(d, E, K, 0, n, device=dev())
    cal = SharedGroupCalibration(ctx, [0, 1])
    cal.reset()
    topk = torch.empty(n, K, dtype=torch.int32, device=dev())
    cal.collect(0, bits_to_dev(inp["x"][0]), to_dev(inp["logits"][0]), topk_out=topk)
    ctx.sync()
    tk = oracle.route(inp["logits"][0], K)
    assert np.array_equal(topk.cpu().numpy(), tk)
    counts, offsets, ids = oracle.bucket(tk, E)
    assert np.array_equal(cal.counts[0].cpu().numpy(), counts)
    # Gram sums of expert 1 on sampled columns (S[:, j] = X_e^T X_e[:, j])
    xe = oracle.bf16_to_f64(inp["x"][0][ids[offsets[1]:offsets[2]]])
    cols = np.array([0, 1, 777, 4095, 4096, 8191])
    ref = xe.T @ xe[:, cols]
    S = cal.S[0][1].cpu().numpy().astype(np.float64)
    got = np.stack([np.where(np.arange(d) >= j, S[:, j], S[j, :]) for j in cols], axis=1)  # lower half
    diag = np.sum(xe * xe, axis=0)
    den = np.sqrt(np.outer(diag, diag[cols]))
    assert np.max(np.abs(got - ref) / den) <= HESS_TOL
    # GPTQ at c = 8192 on a well-conditioned Hessian: diagonal plus rank 64
    rng = np.random.default_rng(72)
    V = rng.normal(size=(d, 64)) / 8.0
    Hm = (np.diag(rng.uniform(0.5, 2.0, d)) + V @ V.T).astype(np.float32)
    W = rng.normal(0, 0.02, (32, d)).astype(np.float32)
    job = _job(to_dev(Hm), to_dev(W), 2, 128)
    ctx.gptq_quantize([job], d, 128, 128, 0.01)
    ctx.sync()
    refq = oracle.gptq(W.astype(np.float64), Hm.astype(np.float64), 2, 128, 0.01, 128)
    codes = job["codes"].cpu().numpy()
    assert agree(codes, refq["codes"]) >= CODE_AGREE
    want = oracle.loss(W.astype(np.float64), refq["wq"], Hm.astype(np.float64))
    got_loss = float(job["loss"].cpu().numpy()[0])
    assert abs(got_loss - want) <= LOSS_RTOL * want


def test_reset_layer_matches_a_zeroed_accumulator():
    import gptq_calibration_moe_amd as clha
    wl = gen.WORKLOADS[1].scaled(n_tokens=4096)
    inp = gen.pair_inputs(wl)
    lg = [l.copy() for l in inp["logits"]]
    for l in lg:
        l[:, 5] = -100.0                     # expert 5 is never chosen: an empty slot
    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, wl.n_shared, wl.n_tokens, device=dev())
    Sz, nz = ctx.new_layer_buffers()         # zeroed: the plain accumulation
    Sr, nr = ctx.new_layer_buffers()
    Sr.fill_(3.0)                            # stale sums and counts of an earlier run
    nr.fill_(7)
    ctx.register_layer(0, Sz, nz)
    ctx.register_layer(1, Sr, nr)
    ctx.reset_layer(1)
    half = wl.n_tokens // 2
    for lo, hi in ((0, half), (half, wl.n_tokens)):   # two batches: overwrite, then add
        for layer in (0, 1):
            ctx.collect_hessians(layer, bits_to_dev(inp["x"][0][lo:hi]), to_dev(lg[0][lo:hi]))
    ctx.sync()
    assert torch.equal(nr, nz) and int(nr[5]) == 0
    low = torch.tril(torch.ones(wl.d, wl.d, dtype=torch.bool, device=dev()))
    for slot in range(ctx.slots):
        assert torch.equal(Sr[slot][low], Sz[slot][low]), f"slot {slot}"
    assert not bool(Sr[5][low].any())        # the empty slot was zeroed

    # a layer reset and never collected has zero counts: rt drops it
    ctx.reset_layer(0)
    H2 = torch.empty(ctx.slots, wl.d, wl.d, dtype=torch.float32, device=dev())
    H1 = torch.empty_like(H2)
    ctx.aggregate([0, 1], "rt", H2)
    ctx.aggregate([1], "rt", H1)
    ctx.sync()
    assert torch.equal(H2, H1)


@pytest.mark.parametrize("top_k", [2, 8])
def test_shared_slot_from_routed_sums_after_reset(top_k):
    """S_shared = (sum_e S_e) / K: every token goes to exactly K routed experts.
    Stale sums in S, an expert no token chooses (its slot zeroed before the
    shared slot is formed) and a second batch added to the first."""
    import gptq_calibration_moe_amd as clha
    wl = gen.WORKLOADS[1].scaled(n_tokens=4096, n_shared=1, top_k=top_k)
    inp = gen.pair_inputs(wl)
    lg = inp["logits"][0].copy()
    if top_k < wl.n_routed:
        lg[:, 5] = -100.0                    # expert 5 is never among the top K
    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, wl.n_shared, wl.n_tokens, device=dev())
    S, n = ctx.new_layer_buffers()
    S.fill_(3.0)                             # stale sums and counts of an earlier run
    n.fill_(7)
    ctx.register_layer(0, S, n)
    ctx.reset_layer(0)
    half = wl.n_tokens // 2
    for lo, hi in ((0, half), (half, wl.n_tokens)):
        ctx.collect_hessians(0, bits_to_dev(inp["x"][0][lo:hi]), to_dev(lg[lo:hi]))
    ctx.sync()
    E = wl.n_routed
    counts = n.cpu().numpy()
    assert int(counts[E]) == wl.n_tokens and int(counts[:E].sum()) == top_k * wl.n_tokens
    if top_k < wl.n_routed:
        assert int(counts[5]) == 0
    ref = oracle.gram_rows(inp["x"][0], np.arange(wl.d))
    assert hess_err(S[E].cpu().numpy(), ref) <= HESS_TOL
