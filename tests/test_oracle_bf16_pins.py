"""Pins of the oracle's BF16 x BF16 path ("DeepGEMM Mega MoE symmetric memory deep analysis", 5.3 and
10.1: the bf16 kernel takes bf16 tokens without scale factors): closed forms on integer values, a
textbook reduction through torch CPU routines, and brute force of the pooled against the direct
per-token path."""
import itertools

import numpy as np
import torch

import oracle
from inputs import MoEShape, make_inputs, to_numpy


def test_bf16_inputs_have_no_scales_and_exact_values():
    sh = MoEShape("b", 2, 16, 256, 128, 4, 4, 2, 64, weight_format="bf16")
    raw = make_inputs(sh)
    assert raw["x"].dtype == torch.bfloat16 and raw["w1"].dtype == torch.bfloat16
    assert raw["x_sf"] is None and raw["w1_sf"] is None and raw["w2_sf"] is None
    inp = to_numpy(raw)
    assert inp["x"].dtype == np.float32
    # the float32 copies hold the bf16 values exactly
    assert np.array_equal(oracle.bf16_round(inp["x"].astype(np.float64)), inp["x"].astype(np.float64))


def test_bf16_gemm1_exact_on_integer_values():
    """Integers -8..8: G equals an int64 matmul exactly."""
    sh = MoEShape("b", 1, 32, 512, 128, 2, 2, 1, 64, weight_format="bf16")
    inp = to_numpy(make_inputs(sh, integer_codes=True))
    a, w1, w2 = inp["x"][0], inp["w1"][1], inp["w2"][1]
    assert np.array_equal(a, np.round(a)) and np.abs(a).max() <= 8
    _, parts = oracle.expert_ffn_rows(a, None, w1, None, w2, None, sh.intermediate, return_parts=True)
    want = a.astype(np.int64) @ w1.astype(np.int64).T
    assert np.array_equal(parts["g"], want.astype(np.float64))


def test_bf16_textbook_single_expert():
    """S=1, E_l=1, K=1, w=1: y = bf16(W2 bf16(silu(W1g x) * W1u x)) through torch CPU routines."""
    sh = MoEShape("b", 1, 40, 384, 256, 1, 1, 1, 64, weight_format="bf16")
    inp = to_numpy(make_inputs(sh))
    inp["topk_idx"][:] = 0
    inp["topk_weights"][:] = 1.0
    out = oracle.forward(inp, 1, 1, 0, sh.block_m, keep_rows=True)
    x = torch.from_numpy(inp["x"][0]).to(torch.float64)
    W1 = torch.from_numpy(inp["w1"][0]).to(torch.float64)
    W2 = torch.from_numpy(inp["w2"][0]).to(torch.float64)
    I = sh.intermediate
    g = torch.matmul(x, W1.T)
    h = torch.nn.functional.silu(g[:, :I]) * g[:, I:]
    hb = h.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    want = torch.matmul(hb, W2.T).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(out["pool_meta"][:40, 1], np.arange(40))
    assert np.mean(out["parts"][0]["l2"] == hb.numpy()) > 0.999
    y = out["y"][0]
    ulp = np.abs(want) * 2.0 ** -7
    assert np.all(np.abs(y - want) <= ulp + 1e-30)


def test_bf16_pool_rows_are_the_tokens():
    sh = MoEShape("b", 2, 24, 256, 128, 4, 2, 2, 64, local_rank=1, weight_format="bf16")
    inp = to_numpy(make_inputs(sh))
    rt = oracle.route(inp["topk_idx"], inp["tokens_per_shard"], 4, 2, 1)
    px, psf, pm, off = oracle.fill_pool(inp["x"], None, rt, 64, 2)
    assert psf is None and px.dtype == np.float32
    for r in range(px.shape[0]):
        s, t, _ = pm[r]
        if s == oracle.layer.META_PAD:
            assert not px[r].any()
        else:
            assert np.array_equal(px[r], inp["x"][s, t])


def test_bf16_brute_force_pooled_equals_direct():
    """Every routing of tiny shapes through the pooled path and the direct per-token path."""
    K = 2
    choices = [(a, b) for a in (-1, 0, 1, 2) for b in (-1, 0, 1, 2) if a < 0 or b < 0 or a != b]
    for S, T in [(1, 3), (3, 1)]:
        sh = MoEShape("b", S, T, 128, 128, 3, 2, K, 64, weight_format="bf16")
        base = to_numpy(make_inputs(sh, seed=12))
        memo = {}
        for s in range(S):
            for t in range(T):
                for e in range(2):
                    one = dict(base)
                    one["topk_idx"] = np.full_like(base["topk_idx"], -1)
                    one["topk_idx"][s, t, 0] = e
                    one["topk_weights"] = np.ones_like(base["topk_weights"])
                    memo[(e, s, t)] = oracle.direct_token(one, s, t, 2, 0)
        for combo in itertools.product(choices, repeat=S * T):
            inp = dict(base)
            inp["topk_idx"] = np.array(combo, dtype=np.int64).reshape(S, T, K)
            out = oracle.forward(inp, 3, 2, 0, 64)
            for s in range(S):
                for t in range(T):
                    acc = np.zeros(128)
                    for k in range(K):
                        e = int(inp["topk_idx"][s, t, k])
                        if 0 <= e < 2:
                            acc += float(np.float32(inp["topk_weights"][s, t, k])) * memo[(e, s, t)]
                    assert np.array_equal(out["y"][s, t], oracle.bf16_round(acc)), (combo, s, t)
