"""The experts' second matrix (down_proj), GPU against the oracle.

Its input is the SwiGLU intermediate h = bf16(silu(x Wg^T) * (x Wu^T)) of each
expert (routed experts over their routed tokens, each shared expert over all
tokens with its own weights), collected on a down_proj context (d = f) through
the routing of the block's main context, then aggregated and quantized as
usual (CLHA summary, section 2.2: every shared weight's Hessian over its own
input).  Checked: counts bit-exact; the down_proj Gram sums within 1e-4 normalised by
sqrt(S_ii S_jj) plus the largest change that admissible bf16 roundings of h can
make (both sides round an fp32 h, but the two fp32 sums differ in order, so an
h within a relative 2^-16 of a bf16 midpoint may round either way: the bound
is computed from the oracle's own h); H_comb likewise; GPTQ of down weights
against H_comb.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import (CODE_AGREE, LOSS_RTOL, agree, assert_down_gram, bits_to_dev, dev, down_gram_flip_bound,
                      to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_calibration_moe_amd  # noqa: F401  (fails loudly if the library is missing)


def _down_setup(wl, f, n_sh, seed):
    import gptq_calibration_moe_amd as clha
    E, K = wl.n_routed, wl.top_k
    main = clha.Context(wl.d, E, K, 0, wl.n_tokens, device=dev())
    down = clha.Context(f, E + n_sh, K, 0, wl.n_tokens, device=dev())
    wgu_bits = gen.swiglu_weights(seed, E + n_sh, f, wl.d)
    wgu = [bits_to_dev(w) for w in wgu_bits]
    return main, down, wgu_bits, wgu


def _down_ref(x_bits, logits, wgu_bits, E, K, f, slots):
    """Oracle Gram sums of the given slots, the counts, and each sum's flip bound."""
    counts, offsets, ids = oracle.bucket(oracle.route(logits, K), E)
    n = x_bits.shape[0]
    S, B = {}, {}
    for e in slots:
        rows = x_bits[ids[offsets[e]:offsets[e + 1]]] if e < E else x_bits
        hb, h32 = oracle.swiglu_intermediate(rows, wgu_bits[e], f, with_fp32=True)
        S[e] = oracle.gram(hb)
        B[e] = down_gram_flip_bound(hb, h32)
    all_counts = np.concatenate([counts, np.full(len(wgu_bits) - E, n)]).astype(np.int64)
    return S, all_counts, B


def _collect(main, down, layer, x_bits, logits, wgu, E, K):
    n = x_bits.shape[0]
    ids = torch.empty(n * K, dtype=torch.int32, device=dev())
    off = torch.empty(E + 1, dtype=torch.int64, device=dev())
    main.collect_hessians(layer, bits_to_dev(x_bits), to_dev(logits), offsets_out=off, token_ids_out=ids)
    down.collect_down_hessians(layer, bits_to_dev(x_bits), ids, off, wgu, E)


def _gptq_check(down, H_dev, H_ref, w_bits, bits, group, label):
    rows, cols = w_bits.shape
    job = {"H": H_dev, "W": bits_to_dev(w_bits), "bits": bits,
           "codes": torch.empty(rows, cols, dtype=torch.uint8, device=dev()),
           "scales": torch.empty(rows, cols // group, dtype=torch.float32, device=dev()),
           "zeros": torch.empty(rows, cols // group, dtype=torch.uint8, device=dev()),
           "loss": torch.empty(1, dtype=torch.float32, device=dev())}
    down.gptq_quantize([job], cols, group, 128, 0.01)
    down.sync()
    wv = oracle.bf16_to_f64(w_bits)
    ref = oracle.gptq(wv, H_ref, bits, group, 0.01, 128)
    a = agree(job["codes"].cpu().numpy(), ref["codes"])
    assert a >= CODE_AGREE, f"{label}: codes agree {a:.5f}"
    want = oracle.loss(wv, ref["wq"], H_ref)
    got = float(job["loss"].cpu().numpy()[0])
    assert abs(got - want) <= LOSS_RTOL * abs(want), f"{label}: loss {got} vs {want}"


def test_down_proj_small_block_two_layers():
    wl = gen.WORKLOADS[1].scaled(n_tokens=2048)
    f, n_sh = 128, 1
    E, K = wl.n_routed, wl.top_k
    main, down, wgu_bits, wgu = _down_setup(wl, f, n_sh, 71)
    inp = gen.pair_inputs(wl)
    S_d, n_d = {}, {}
    for l in range(2):
        main.register_layer(l, *main.new_layer_buffers())
        S_d[l], n_d[l] = down.new_layer_buffers()
        down.register_layer(l, S_d[l], n_d[l])
        _collect(main, down, l, inp["x"][l], inp["logits"][l], wgu, E, K)
    down.sync()
    ref, bound = [], []
    for l in range(2):
        S, n, B = _down_ref(inp["x"][l], inp["logits"][l], wgu_bits, E, K, f, range(E + n_sh))
        ref.append((S, n))
        bound.append(B)
        assert np.array_equal(n_d[l].cpu().numpy(), n)
        for e in range(E + n_sh):
            assert_down_gram(S_d[l][e].cpu().numpy(), S[e], B[e], f"layer {l} slot {e}")
    H = torch.empty(down.slots, f, f, dtype=torch.float32, device=dev())
    down.aggregate([0, 1], "rt", H)
    down.sync()
    Hn = H.cpu().numpy()
    H_ref = {}
    for e in range(E + n_sh):
        n = [int(ref[0][1][e]), int(ref[1][1][e])]
        H_ref[e], _ = oracle.aggregate([ref[0][0][e], ref[1][0][e]], n, "rt")
        assert_down_gram(Hn[e], H_ref[e], (bound[0][e] + bound[1][e]) / max(sum(n), 1), f"H slot {e}")
    # down weights [d_model, f], quantized against their H_comb (routed slot 2, the shared slot)
    w_down = gen.swiglu_weights(72, 1, wl.d // 2, f)[0]            # [d_model, f] bf16 bits
    for e in (2, E):
        _gptq_check(down, H[e], H_ref[e], w_down, 2, 128, f"slot {e}")


def test_down_proj_mid_moe_shapes_sampled():
    wl = gen.WORKLOADS[2].scaled(n_tokens=4096)
    f, n_sh = 1408, wl.n_shared
    E, K = wl.n_routed, wl.top_k
    main, down, wgu_bits, wgu = _down_setup(wl, f, n_sh, 73)
    inp = gen.pair_inputs(wl)
    main.register_layer(0, *main.new_layer_buffers())
    S_d, n_d = down.new_layer_buffers()
    down.register_layer(0, S_d, n_d)
    down.reset_layer(0)
    _collect(main, down, 0, inp["x"][0], inp["logits"][0], wgu, E, K)
    down.sync()
    sample = [5, 41, E, E + 1]                                     # two routed, both shared experts
    ref_S, ref_n, B = _down_ref(inp["x"][0], inp["logits"][0], wgu_bits, E, K, f, sample)
    assert np.array_equal(n_d.cpu().numpy(), ref_n)
    for e in sample:
        assert_down_gram(S_d[e].cpu().numpy(), ref_S[e], B[e], f"slot {e}")
    # GPTQ at c = f = 1408 (a partial last superblock) on the shared slot's Hessian
    H = torch.empty(down.slots, f, f, dtype=torch.float32, device=dev())
    down.aggregate([0], "rt", H)
    down.sync()
    H_ref, _ = oracle.aggregate([ref_S[E]], [int(ref_n[E])], "rt")
    assert_down_gram(H[E].cpu().numpy(), H_ref, B[E] / int(ref_n[E]), "H shared slot")
    w_down = gen.swiglu_weights(74, 1, 128, f)[0]                  # [256, f]
    _gptq_check(down, H[E], H_ref, w_down, 3, 128, "shared slot, c = 1408")


def test_down_proj_full_size_in_bench_configuration():
    """The down_proj step as the benchmark runs it (bench.py --down-proj): mid
    MoE block at 65,536 tokens per layer, both layers collected through their
    routing, routing-frequency aggregation, GPTQ of all 66 down_proj jobs in one
    batch; counts of both layers bit-exact, and one sampled routed expert's
    H_comb and GPTQ against the oracle."""
    import gptq_calibration_moe_amd as clha
    from gptq_calibration_moe_amd.calibrate import SharedGroupCalibration
    print("down_proj full size, bench configuration", flush=True)
    wl = gen.WORKLOADS[2]
    n, E, K, nsh, f, dm = wl.n_tokens, wl.n_routed, wl.top_k, wl.n_shared, wl.rows, wl.d
    inp = gen.pair_inputs(wl)
    main = clha.Context(dm, E, K, 0, n, device=dev())
    down = clha.Context(f, E + nsh, K, 0, n, device=dev())
    wgu_bits = [gen.expert_weights(wl, 0, e) for e in range(E + nsh)]
    wgu = [bits_to_dev(w) for w in wgu_bits]
    wd_bits = [gen.swiglu_weights(2000 + e, 1, dm // 2, f)[0] for e in range(E + nsh)]
    routing = []
    for l in range(2):
        main.register_layer(l, *main.new_layer_buffers())
        ids = torch.empty(n * K, dtype=torch.int32, device=dev())
        off = torch.empty(E + 1, dtype=torch.int64, device=dev())
        main.collect_hessians(l, bits_to_dev(inp["x"][l]), to_dev(inp["logits"][l]), offsets_out=off,
                              token_ids_out=ids)
        routing.append((ids, off))
    cal = SharedGroupCalibration(down, [0, 1])
    outputs = cal.make_outputs(range(E + nsh), dm, wl.group)
    jobs = [{"H": cal.H[e], "W": bits_to_dev(wd_bits[e]), "bits": wl.bits, **outputs[e]}
            for e in range(E + nsh)]
    prep = down.prepare_gptq(jobs, f)
    cal.reset()
    for l in range(2):
        down.collect_down_hessians(l, bits_to_dev(inp["x"][l]), routing[l][0], routing[l][1], wgu, E)
    cal.aggregate("rt")
    down.run_gptq(prep, wl.group, 128, wl.damp)
    down.sync()
    e = int(np.random.default_rng(12).integers(E))
    S, cnt, B = [], [], []
    for l in range(2):
        ref_S, ref_n, ref_B = _down_ref(inp["x"][l], inp["logits"][l], wgu_bits, E, K, f, [e])
        assert np.array_equal(cal.counts[l].cpu().numpy(), ref_n), f"layer {l} counts"
        S.append(ref_S[e])
        cnt.append(int(ref_n[e]))
        B.append(ref_B[e])
    H_ref, _ = oracle.aggregate(S, cnt, "rt")
    assert_down_gram(cal.H[e].cpu().numpy(), H_ref, (B[0] + B[1]) / (cnt[0] + cnt[1]), f"H_comb expert {e}")
    wv = oracle.bf16_to_f64(wd_bits[e])
    ref = oracle.gptq(wv, H_ref, wl.bits, wl.group, wl.damp, 128)
    codes = outputs[e]["codes"].cpu().numpy()
    a = agree(codes, ref["codes"])
    assert a >= CODE_AGREE, f"expert {e}: codes agree {a:.5f}"
    want = oracle.loss(wv, ref["wq"], H_ref)
    got = float(outputs[e]["loss"].cpu().numpy()[0])
    assert abs(got - want) <= LOSS_RTOL * abs(want), f"expert {e}: loss {got} vs {want}"
