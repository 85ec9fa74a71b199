"""clha_loss_static (the allocation-free loss entry point) against clha_loss
(the workspace entry point) through the C ABI: two calls in a row, the second
smaller, each bit for bit equal to the workspace entry point's result; sizes
beyond the static scratch are rejected."""
import numpy as np
import pytest
import torch

import gen
from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_calibration_moe_amd  # noqa: F401  (fails loudly if the library is missing)


def _case(seed, rows, c, group, bits=3):
    rng = np.random.default_rng(seed)
    x = gen.bf16_value(gen.structured_activations(seed, 2 * c, c, 2.0))
    H = (x.astype(np.float64).T @ x / (2 * c)).astype(np.float32)
    W = gen.bf16_bits(rng.normal(0, 0.02, (rows, c)).astype(np.float32))
    codes = rng.integers(0, 1 << bits, (rows, c)).astype(np.uint8)
    scales = rng.uniform(0.005, 0.02, (rows, c // group)).astype(np.float32)
    zeros = rng.integers(0, 1 << bits, (rows, c // group)).astype(np.uint8)
    Wd = to_dev(W.view(np.int16)).view(torch.bfloat16)
    return Wd, to_dev(codes), to_dev(scales), to_dev(zeros), to_dev(H)


def test_static_loss_matches_workspace_loss_twice():
    import gptq_calibration_moe_amd as clha
    ctx = clha.Context(2048, 8, 2, 0, 16, device=dev())
    for seed, rows, c, group in ((80, 2816, 2048, 128), (81, 300, 512, 64)):   # second call smaller
        print(f"static loss: rows {rows}, cols {c}", flush=True)
        W, q, s, z, H = _case(seed, rows, c, group)
        want = torch.empty(1, dtype=torch.float32, device=dev())
        got = torch.full((1,), -1.0, dtype=torch.float32, device=dev())
        ctx.loss(W, q, s, z, H, group, want)
        ctx.loss_static(W, q, s, z, H, group, got)
        ctx.sync()
        assert float(want.cpu()[0]) > 0
        assert torch.equal(got, want), (float(got.cpu()[0]), float(want.cpu()[0]))


def test_static_loss_rejects_sizes_beyond_the_scratch():
    import gptq_calibration_moe_amd as clha
    ctx = clha.Context(2048, 8, 2, 0, 16, device=dev())
    rows, c = 65536 + 64, 8192               # 1025 row tiles x 128 column tiles > 131072
    W = torch.zeros(rows, c, dtype=torch.bfloat16, device=dev())
    q = torch.zeros(rows, c, dtype=torch.uint8, device=dev())
    s = torch.ones(rows, c // 128, dtype=torch.float32, device=dev())
    z = torch.zeros(rows, c // 128, dtype=torch.uint8, device=dev())
    H = torch.zeros(c, c, dtype=torch.float32, device=dev())
    out = torch.empty(1, dtype=torch.float32, device=dev())
    with pytest.raises(clha.ClhaError) as ei:
        ctx.loss_static(W, q, s, z, H, 128, out)
    assert ei.value.status == clha.ERR_WORKSPACE
