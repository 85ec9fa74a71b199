"""Packed storage of codes (CLHA summary, section 2.3: b bits for routed
experts, b+1 for shared ones), GPU against the oracle, bit-exact: every width
2..8 on a ragged code matrix, the round trip, and the empty stream."""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_calibration_moe_amd  # noqa: F401  (fails loudly if the library is missing)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_pack_matches_oracle_and_round_trips(bits):
    import gptq_calibration_moe_amd as clha
    wl = gen.WORKLOADS[1]
    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, wl.n_shared, wl.n_tokens, device=dev())
    rows, cols = 37, 136
    codes = np.random.default_rng(bits).integers(0, 1 << bits, (rows, cols)).astype(np.uint8)
    c_dev = torch.from_numpy(codes).to(dev())
    packed = ctx.pack_codes(c_dev, bits)
    ctx.sync()
    want = oracle.pack_codes(codes.ravel(), bits).reshape(rows, cols * bits // 8)
    assert np.array_equal(packed.cpu().numpy(), want)
    back = ctx.unpack_codes(packed, bits, cols)
    ctx.sync()
    assert np.array_equal(back.cpu().numpy(), codes)


def test_pack_empty_stream():
    import gptq_calibration_moe_amd as clha
    wl = gen.WORKLOADS[1]
    ctx = clha.Context(wl.d, wl.n_routed, wl.top_k, wl.n_shared, wl.n_tokens, device=dev())
    empty = torch.empty(0, 8, dtype=torch.uint8, device=dev())
    out = ctx.pack_codes(empty, 3)
    ctx.sync()
    assert out.shape == (0, 3)
