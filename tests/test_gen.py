"""Host-side checks of the seeded input generator (formats, determinism, shapes)."""
import numpy as np
import torch

import gen


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-20, 20, 100000)).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]      # exact ties: to even
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (gen.bf16_bits(x) == want).all()
    assert (gen.bf16_value(gen.bf16_bits(x)) == torch.from_numpy(x).to(torch.bfloat16).float().numpy()).all()


def test_streams_are_addressed_and_deterministic():
    wl = gen.WORKLOADS[1]
    a1 = gen.pair_inputs(wl)
    a2 = gen.pair_inputs(wl)
    for k in ("x", "logits"):
        for u, v in zip(a1[k], a2[k]):
            assert (u == v).all()
    w3 = gen.expert_weights(wl, 0, 3)
    assert (w3 == gen.expert_weights(wl, 0, 3)).all()
    assert not (w3 == gen.expert_weights(wl, 0, 4)).all()
    assert a1["x"][0].shape == (4096, 256) and a1["x"][0].dtype == np.uint16
    assert a1["logits"][0].shape == (4096, 8) and a1["logits"][0].dtype == np.float32
    assert w3.shape == (512, 256) and w3.dtype == np.float32


def test_workload_shapes():
    w2 = gen.WORKLOADS[2]
    assert w2.job_rows == 2816 and w2.n_slots == 65 and w2.n_experts_total == 66
    w4, w3 = gen.WORKLOADS[4], gen.WORKLOADS[3]
    assert w4.seed_base + w4.wid == w3.seed_base + w3.wid and w4.shared_bits == w4.bits + 1


def test_small_variants_of_each_kind():
    for wid in (2, 3, 5):
        wl = gen.WORKLOADS[wid].scaled(n_tokens=256, d=128, n_routed=8, top_k=2, rows=16)
        inp = gen.pair_inputs(wl, t=0.5 if wl.x_kind == "drift" else None)
        assert inp["x"][1].shape == (256, 128)
        assert np.isfinite(inp["logits"][1]).all()
    wl = gen.WORKLOADS[5].scaled(n_tokens=256, d=128, n_routed=8, top_k=2, rows=16)
    i0 = gen.pair_inputs(wl, t=0.0)
    assert (i0["x"][0] == i0["x"][1]).all() and (i0["logits"][0] == i0["logits"][1]).all()
