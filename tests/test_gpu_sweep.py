"""Routing-sharpness sweep of one pair (the CLHA summary's divergence
experiment, section 4), GPU path against the oracle.

Both layers see the same activations; routing is sampled (Gumbel top-K of
x R / tau), so tau sets how far the layers' routing diverges.  Checked: the
divergence measures from the GPU's routing equal the oracle's (routing is
bit-exact); at a tiny tau routing agrees in both layers, so CLHA-rt and -eq
equal PLIC bit for bit; at a large tau the overlap falls toward K/E; there the
losses of PLIC, CLHA-rt and CLHA-eq under each layer's Hessian against the
oracle.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import LOSS_RTOL, bits_to_dev, dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_calibration_moe_amd  # noqa: F401  (fails loudly if the library is missing)


def test_sharpness_sweep():
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.sweep import sharpness_sweep
    wl = gen.WORKLOADS[1].scaled(n_tokens=2048, x_kind="drift", drift=(0.0,))
    xa, _ = gen.activations(wl, 0, t=0.0)
    x_dev = [bits_to_dev(xa), bits_to_dev(xa)]
    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, 0, wl.n_tokens, device=dev())
    experts = [1, 6]
    w_host = {e: gen.expert_weights(wl, 0, e) for e in experts}
    weights = {e: torch.from_numpy(w).to(dev()) for e, w in w_host.items()}
    taus = [1e-5, 1e3]
    logits = {t: [gen.sharpness_logits(wl, 0, l, xa, t) for l in range(2)] for t in taus}
    rows = sharpness_sweep(ctx, x_dev, lambda t: [to_dev(a) for a in logits[t]], taus, weights, wl.bits,
                           wl.group)
    for row, t in zip(rows, taus):
        tk = [oracle.route(logits[t][l], wl.top_k) for l in range(2)]
        cnt = [oracle.bucket(tk[l], wl.n_routed)[0] for l in range(2)]
        assert row["topk_overlap"] == oracle.topk_overlap(*tk)
        assert abs(row["load_divergence"] - oracle.load_divergence(*cnt)) < 1e-12
    sharp, flat = rows
    assert sharp["topk_overlap"] == 1.0
    for tag in ("a", "b"):
        assert sharp[f"loss_rt_{tag}"] == sharp[f"loss_plic_{tag}"] == sharp[f"loss_eq_{tag}"]
    assert flat["topk_overlap"] < 0.5 and flat["load_divergence"] >= 0.0
    # PLIC, CLHA-rt and CLHA-eq at the large tau against the oracle, each result
    # under each layer's own Hessian
    tk = [oracle.route(logits[1e3][l], wl.top_k) for l in range(2)]
    S = [oracle.layer_hessians(xa, tk[l], wl.n_routed, 0) for l in range(2)]
    for name in ("plic", "rt", "eq"):
        for tag, l in (("a", 0), ("b", 1)):
            want = 0.0
            for e in experts:
                Se = [S[0][0][e], S[1][0][e]]
                ne = [int(S[0][1][e]), int(S[1][1][e])]
                if name == "plic":
                    H_c, _ = oracle.aggregate(Se, ne, "explicit", alpha=[1.0, 0.0])
                else:
                    H_c, _ = oracle.aggregate(Se, ne, name)
                H_l, _ = oracle.aggregate([Se[l]], [ne[l]], "rt")
                wv = gen.weights_value(wl, w_host[e]).astype(np.float64)
                ref = oracle.gptq(wv, H_c, wl.bits, wl.group, 0.01, 128)
                want += oracle.loss(wv, ref["wq"], H_l)
            got = flat[f"loss_{name}_{tag}"]
            assert abs(got - want) <= LOSS_RTOL * abs(want), f"{name} under H_{tag}: {got} vs {want}"
