"""GPU parity: the HIP layer against the CPU oracle, through the C ABI.

Layout (counts, table, pool offsets, block list, pool rows/scales/metadata): bit-exact.
Values (y and combine rows): max|d| <= 2e-2 * max|ref| + 1e-3, the layer's stated tolerance.
Small workloads are compared element by element over the whole output; the full-size workloads
(decode, skewed, prefill; the same launch configuration the benchmark times) on their whole layout
and on sampled tokens that the oracle evaluates one by one.
"""
import numpy as np
import pytest
import torch

import dispatch_fp8_grouped_amd as mm
import oracle
from inputs import SHAPES, MoEShape, make_inputs, to_numpy

from gpu_util import Run, check_layout, tol_check, sample_tokens, inputs_np

pytestmark = pytest.mark.gpu


def _print_case(name, shape):
    print(f"[case] {name}: S={shape.num_shards} T={shape.max_tokens_per_shard} H={shape.hidden} "
          f"I={shape.intermediate} E={shape.num_experts}/{shape.num_local_experts} K={shape.topk} "
          f"BM={shape.block_m} seed={shape.seed}", flush=True)


def full_compare(shape, inputs=None, flags=0, name=""):
    _print_case(name or shape.name, shape)
    run = Run(shape, inputs=inputs, flags=flags)
    inp = inputs_np(run)
    assert run.status == 0
    check_layout(run, inp)
    ref = oracle.forward(inp, shape.num_experts, shape.num_local_experts, shape.local_rank, shape.block_m,
                         num_shared_experts=shape.num_shared_experts)
    y = run.y_host()
    valid = ~np.isnan(ref["y"])
    tol_check(y[valid], ref["y"][valid], name)
    # rows t >= T_s untouched (still the NaN fill)
    assert np.all(np.isnan(y[~valid]))
    run.close()
    return run, ref


# --------------------------------------------------------------- small workloads, whole output
def test_tiny_whole_layer():
    full_compare(SHAPES["tiny"], name="tiny")


def test_ragged_multi_shard_whole_layer():
    """Several shards with ragged valid counts (one empty), remote experts, K=4, BM=64."""
    sh = MoEShape("ragged", 3, 200, 512, 384, 16, 8, 4, 64, local_rank=1, seed=7)
    inp = make_inputs(sh, device="cuda", tokens_per_shard=[200, 137, 0])
    full_compare(sh, inputs=inp, name="ragged")


def test_mid_whole_layer():
    full_compare(SHAPES["mid"], name="mid")


def test_bm128_ragged_tail():
    sh = MoEShape("bm128", 2, 700, 768, 256, 8, 4, 2, 128, seed=9)
    inp = make_inputs(sh, device="cuda", tokens_per_shard=[700, 555])
    full_compare(sh, inputs=inp, name="bm128")


# --------------------------------------------------------------- shared expert
@pytest.mark.parametrize("case", ["bm64_rank1", "bm128_rank0"])
def test_shared_expert_whole_layer(case):
    """A shared expert on the own shard's tokens (pool segment after the routed experts, combine slot
    K, weight 1): layout bit-exact, whole output within tolerance."""
    if case == "bm64_rank1":
        sh = MoEShape("shared64", 3, 150, 512, 256, 16, 8, 4, 64, local_rank=1, num_shared_experts=1, seed=51)
        tps = [150, 97, 3]
    else:
        sh = MoEShape("shared128", 2, 300, 768, 384, 8, 4, 2, 128, local_rank=0, num_shared_experts=1, seed=52)
        tps = [257, 300]
    inp = make_inputs(sh, device="cuda", tokens_per_shard=tps)
    full_compare(sh, inputs=inp, name=sh.name)


# --------------------------------------------------------------- MXFP4 weights (the FP8 x FP4 variant)
@pytest.mark.parametrize("case", ["bm64", "bm128_ragged", "bm64_shared_empty_shard", "bm128_zipf",
                                  "bm128_short_k", "bm64_short_k"])
def test_mxfp4_weights_whole_layer(case):
    """e2m1 weights with UE8M0 exponents per 32 K, applied by the MFMA's scale operand: layout
    bit-exact, whole output within tolerance against the oracle on the decoded weights.  Also with a
    shared expert (its MXFP4 weights packed after the routed experts') beside an empty shard, and with
    skewed routing (some experts with many blocks, some with none), and with K loops shorter than the
    load pipeline."""
    if case == "bm64":
        sh = MoEShape("mx64", 3, 120, 512, 256, 32, 8, 4, 64, local_rank=1, weight_format="mxfp4", seed=101)
        tps = [120, 77, 9]
    elif case == "bm128_ragged":
        sh = MoEShape("mx128", 2, 400, 1024, 512, 16, 8, 4, 128, weight_format="mxfp4", seed=102)
        tps = [400, 263]
    elif case == "bm64_shared_empty_shard":
        sh = MoEShape("mx64sh", 3, 130, 512, 384, 24, 8, 4, 64, local_rank=2, num_shared_experts=1,
                      weight_format="mxfp4", seed=103)
        tps = [130, 0, 71]
    elif case == "bm128_zipf":
        sh = MoEShape("mx128z", 4, 256, 768, 256, 32, 8, 4, 128, local_rank=0, routing="zipf",
                      weight_format="mxfp4", seed=104)
        tps = [256, 256, 190, 33]
    else:
        # K loops shorter than the load pipeline: GEMM1 has H/128 = 2 steps per tile and GEMM2 I/128 = 1
        bm = 128 if case == "bm128_short_k" else 64
        sh = MoEShape("mxshort", 2, 200, 256, 128, 8, 4, 2, bm, local_rank=1, weight_format="mxfp4", seed=105)
        tps = [200, 141]
    inp = make_inputs(sh, device="cuda", tokens_per_shard=tps)
    full_compare(sh, inputs=inp, name=sh.name)


def test_mxfp4_wide_exponent_range():
    """Exponent bytes drawn uniformly from [112, 142] (scales 2^-15 .. 2^15), independently per row and
    32-value block: a scale applied to the wrong lane, K block or byte of the packed word would be off
    by orders of magnitude, not by a rounding step."""
    sh = MoEShape("mxwide", 2, 150, 512, 256, 16, 8, 4, 64, local_rank=1, weight_format="mxfp4", seed=106)
    tps = [150, 99]
    inp = make_inputs(sh, device="cuda", tokens_per_shard=tps)
    g = torch.Generator().manual_seed(107)
    for k in ("w1_sf", "w2_sf"):
        inp[k] = torch.randint(112, 143, tuple(inp[k].shape), generator=g, dtype=torch.int32).to(torch.uint8).cuda()
    full_compare(sh, inputs=inp, name="mxfp4 wide exponents")


# --------------------------------------------------------------- seeded sweep of small configurations
def _sweep_cases(n=40, seed=2024):
    """Random small layers, alternating FP8 and MXFP4 weights: BLOCK_M 64/128, H 256-768, I 128-384,
    1-16 local experts on 1, 2 or 4 ranks, top-1..8, 1-4 shards with random (possibly zero) token
    counts, uniform or Zipf routing, with or without a shared expert."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        wf = "mxfp4" if i % 2 else "fp8"
        bm = int(rng.choice([64, 128]))
        H = int(rng.choice([256, 512, 768]))
        I = int(rng.choice([128, 256, 384]))
        El = int(rng.integers(1, 17))
        R = int(rng.choice([1, 2, 4]))
        E = El * R
        K = int(rng.integers(1, min(E, 8) + 1))
        S = int(rng.integers(1, 5))
        T = int(rng.integers(1, 257))
        rank = int(rng.integers(0, R))
        nsh = int(rng.integers(0, 2)) if rank < S else 0
        routing = "zipf" if rng.random() < 0.3 else "uniform"
        tps = [int(rng.integers(0, T + 1)) for _ in range(S)]
        out.append((MoEShape(f"sweep{i}", S, T, H, I, E, El, K, bm, local_rank=rank, routing=routing,
                             num_shared_experts=nsh, weight_format=wf, seed=300 + i), tps))
    return out


_SWEEP = _sweep_cases()


@pytest.mark.parametrize("case", range(len(_SWEEP)), ids=[sh.name for sh, _ in _SWEEP])
def test_random_configs_whole_layer(case):
    """Layout bit-exact and the whole output within tolerance on each seeded configuration."""
    sh, tps = _SWEEP[case]
    inp = make_inputs(sh, device="cuda", tokens_per_shard=tps)
    full_compare(sh, inputs=inp, name=f"{sh.name} {sh.weight_format} tps={tps}")


_SWEEP_FP8 = [i for i, (sh, _) in enumerate(_SWEEP) if sh.weight_format == "fp8"]


@pytest.mark.parametrize("case", _SWEEP_FP8, ids=[_SWEEP[i][0].name for i in _SWEEP_FP8])
def test_random_configs_fill_inside_gemm1(case):
    """The same FP8 configurations under the arrival-counted schedule (GEMM1's work-groups pull the
    pool themselves), including those with no routed rows at all."""
    sh, tps = _SWEEP[case]
    inp = make_inputs(sh, device="cuda", tokens_per_shard=tps)
    full_compare(sh, inputs=inp, flags=mm.FLAG_FILL_IN_GEMM1, name=f"{sh.name} fill-in-gemm1 tps={tps}")


@pytest.mark.parametrize("case", range(len(_SWEEP)), ids=[sh.name for sh, _ in _SWEEP])
def test_random_configs_one_gemm_launch(case):
    """Every configuration with GEMM1 and GEMM2 in one launch (and, for FP8 weights, the pool pulled in
    it too, and routing as well): the output bits equal the stream-ordered kernels', the status is
    clean and the schedule words are back at zero."""
    sh, tps = _SWEEP[case]
    print(f"[case] one GEMM launch {sh.name} {sh.weight_format} tps={tps}", flush=True)
    inp = make_inputs(sh, device="cuda", tokens_per_shard=tps)
    base = mm.MegaMoE.from_shape(sh)
    want = base(inp)
    torch.cuda.synchronize()
    assert base.status() == 0
    variants = [mm.FLAG_ONE_GEMM_LAUNCH]
    if sh.weight_format == "fp8":
        variants += [mm.FLAG_ONE_GEMM_LAUNCH | mm.FLAG_FILL_IN_GEMM1, mm.FLAG_ROUTE_IN_LAUNCH]
    for flags in variants:
        moe = mm.MegaMoE.from_shape(sh, flags=flags)
        for _ in range(2):
            got = moe(inp)
            torch.cuda.synchronize()
            assert moe.status() == 0
            for i, n in enumerate(tps):
                assert torch.equal(got[i, :n].view(torch.int16), want[i, :n].view(torch.int16)), (flags, i)
        words = moe.region("sched", torch.int32, (64 + 2 * moe.layout["max_pool_blocks"],))
        assert not words.any().item()
        moe.close()
    base.close()


@pytest.mark.parametrize("case", range(len(_SWEEP)), ids=[sh.name for sh, _ in _SWEEP])
def test_random_configs_routing_paths_agree(case):
    """The one-work-group routing (used where the counts fit in LDS) and the three-launch routing write
    the same counts, table, pool layout, row metadata and scatter targets, and give the same output
    bits."""
    sh, tps = _SWEEP[case]
    print(f"[case] routing paths {sh.name} tps={tps}", flush=True)
    inp = make_inputs(sh, device="cuda", tokens_per_shard=tps)
    runs = [Run(sh, inputs=inp, flags=f) for f in (0, mm.FLAG_DEBUG_ROUTE_LAUNCHES)]
    a, b = (r.layout_host() for r in runs)
    for k in a:
        if k != "table":
            assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k
    slots = np.arange(sh.max_tokens_per_shard)[None, None, :] < a["recv"][:, :, None]   # written slots
    assert np.array_equal(a["table"][slots], b["table"][slots]), "table"
    rows = a["nblocks"] * runs[0].moe.block_m
    for name, width in (("pool_meta", 3), ("pool_dst", 1)):
        ra, rb = (r.region(name, torch.int32, (rows * width,)).cpu().numpy() for r in runs)
        assert np.array_equal(ra, rb), name
    for i, n in enumerate(tps):
        assert torch.equal(runs[0].y[i, :n].view(torch.int16), runs[1].y[i, :n].view(torch.int16))
    for r in runs:
        assert r.status == 0
        r.close()


# --------------------------------------------------------------- full sizes, sampled values
_FULL_VARIANTS = {"decode_shared": dict(num_shared_experts=1), "decode_mxfp4": dict(weight_format="mxfp4"),
                  "prefill_mxfp4": dict(weight_format="mxfp4")}


@pytest.mark.parametrize("name", ["decode", "skewed", "prefill", "decode_shared", "decode_mxfp4", "prefill_mxfp4"])
def test_full_size_layout_and_sampled_tokens(name):
    shape = SHAPES[name] if name in SHAPES else SHAPES[name.split("_")[0]].replace(name=name, **_FULL_VARIANTS[name])
    _print_case(name, shape)
    run = Run(shape)
    inp = inputs_np(run)
    assert run.status == 0
    rt, off = check_layout(run, inp)
    y = run.y_host()
    cache = {}
    toks = sample_tokens(inp, shape, 12, seed=shape.seed)
    if shape.num_shared_experts:
        toks += [(shape.local_rank, t) for t in (0, 77, shape.max_tokens_per_shard - 1)]
    got = np.stack([y[s, t] for s, t in toks])
    want = np.stack([oracle.direct_token(inp, s, t, shape.num_local_experts, shape.local_rank, cache=cache,
                                         num_shared_experts=shape.num_shared_experts)
                     for s, t in toks])
    tol_check(got, want, f"{name} sampled y")
    # padding and unrouted rows of y: tokens without local experts are exact zeros
    for (s, t), row in zip(toks, want):
        if not np.any(row):
            assert np.all(y[s, t] == 0)
    run.close()


# --------------------------------------------------------------- combine rows of one expert
def test_comb_rows_and_requant_codes_mid():
    shape = SHAPES["mid"]
    _print_case("mid comb rows", shape)
    run = Run(shape)
    inp = inputs_np(run)
    rt, off = check_layout(run, inp)
    ref = oracle.forward(inp, shape.num_experts, shape.num_local_experts, 0, shape.block_m,
                         experts=[0, 13, 31], keep_rows=True)
    for le in [0, 13, 31]:
        base = int(off[le]) * shape.block_m
        n = int(rt.recv_tot[le])
        meta = ref["pool_meta"][base:base + n]
        o_ref = ref["rows"][le]
        got = np.stack([run.comb_row(int(k), int(s), int(t)) for s, t, k in meta])
        tol_check(got, o_ref, f"comb rows expert {le}")
        q, s = run.l2_host(slice(base, base + n))
        parts = ref["parts"][le]
        assert np.mean(q == parts["l2_codes"]) > 0.99
        # the scales follow each row's amax of h: fp32 accumulation over K = H on the GPU against
        # fp64 in the oracle moves amax by a few 1e-6 relative
        assert np.allclose(s, parts["l2_sf"], rtol=2e-4, atol=0)
    run.close()
