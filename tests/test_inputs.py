"""The seeded input generator: shapes, determinism, distributions (no GPU)."""
import numpy as np
import torch

from inputs import SHAPES, MoEShape, make_inputs, digest


def test_shapes_and_determinism():
    sh = SHAPES["tiny"]
    a = make_inputs(sh)
    b = make_inputs(sh)
    assert digest(a) == digest(b)
    assert digest(make_inputs(sh, seed=5)) != digest(a)
    S, T, H, I, El, K = 1, 64, 256, 512, 8, 2
    assert a["x"].shape == (S, T, H) and a["x"].dtype == torch.uint8
    assert a["x_sf"].shape == (S, T, H // 128) and a["x_sf"].dtype == torch.float32
    assert a["w1"].shape == (El, 2 * I, H) and a["w1_sf"].shape == (El, 2 * I // 128, H // 128)
    assert a["w2"].shape == (El, H, I) and a["w2_sf"].shape == (El, H // 128, I // 128)
    assert a["topk_idx"].shape == (S, T, K) and a["topk_idx"].dtype == torch.int64
    assert a["tokens_per_shard"] == [T]


def test_routing_distinct_and_weights_normalised():
    sh = SHAPES["mid"].replace(max_tokens_per_shard=256, hidden=128, intermediate=128)
    inp = make_inputs(sh)
    idx = inp["topk_idx"]
    srt = idx.sort(-1).values
    assert bool((srt[..., 1:] != srt[..., :-1]).all())
    assert int(idx.min()) >= 0 and int(idx.max()) < sh.num_experts
    assert torch.allclose(inp["topk_weights"].sum(-1), torch.ones(1), atol=1e-5)
    # no NaN codes anywhere, scales positive
    for k in ("x", "w1", "w2"):
        c = inp[k]
        assert not bool(((c & 0x7F) == 0x7F).any())
    assert bool((inp["x_sf"] > 0).all())


def test_zipf_routing_is_skewed():
    sh = SHAPES["skewed"].replace(max_tokens_per_shard=512, hidden=128, intermediate=128)
    inp = make_inputs(sh)
    counts = torch.bincount(inp["topk_idx"].reshape(-1), minlength=sh.num_experts).numpy()
    mean = counts.mean()
    assert counts.max() > 10 * mean
    uni = make_inputs(sh.replace(routing="uniform"))
    cu = torch.bincount(uni["topk_idx"].reshape(-1), minlength=sh.num_experts).numpy()
    assert cu.max() < 2 * cu.mean()


def test_integer_codes_are_integers():
    sh = MoEShape("t", 1, 8, 128, 128, 2, 2, 1, 64)
    inp = make_inputs(sh, integer_codes=True)
    v = inp["x"].view(torch.float8_e4m3fn).to(torch.float32)
    assert bool((v == v.round()).all()) and float(v.abs().max()) <= 8
    assert bool((inp["w1_sf"] == 2.0 ** -6).all())
