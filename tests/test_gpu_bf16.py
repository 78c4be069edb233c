"""BF16 x BF16 layer on the GPU (weight_format "bf16": bf16 tokens and weights, no scales; the pages'
bf16 kernel, "DeepGEMM Mega MoE symmetric memory deep analysis", 5.3 and 10.1) against the oracle's
bf16 path: routing layout and pool rows bit for bit, whole outputs within the layer tolerance, the
GEMMs bit-exact on integer values (exact fp32 sums), the L2 pool against the oracle's bf16-rounded
SwiGLU, and repeat / poisoned-workspace identity."""
import numpy as np
import pytest
import torch

import dispatch_fp8_grouped_amd as mm
import oracle
from inputs import SHAPES, MoEShape, make_inputs

from gpu_util import Run, inputs_np, sample_tokens, tol_check

pytestmark = pytest.mark.gpu


def _pool_rows(run):
    """The bf16 pool as float32 [nb*BM, H]: tiled [blocks][H/64][BM][64 values]."""
    sh, L, bm = run.shape, run.moe.layout, run.moe.block_m
    nb = int(run.region("status", torch.int32, (2,))[1].item())
    H = sh.hidden
    t = run.region("pool_x", torch.bfloat16, (L["max_pool_blocks"], H // 64, bm, 64))[:nb]
    return t.permute(0, 2, 1, 3).reshape(nb * bm, H).float().cpu().numpy()


def _l2_rows(run):
    """The bf16 L2 pool as float32 [nb*BM, I]: [blocks][I/64][4][BM][16 values]."""
    sh, L, bm = run.shape, run.moe.layout, run.moe.block_m
    nb = int(run.region("status", torch.int32, (2,))[1].item())
    I = sh.intermediate
    t = run.region("l2_x", torch.bfloat16, (L["max_pool_blocks"], I // 64, 4, bm, 16))[:nb]
    return t.permute(0, 3, 1, 2, 4).reshape(nb * bm, I).float().cpu().numpy()


def _check_layout_bf16(run, n):
    sh = run.shape
    nsh = sh.num_shared_experts
    rt = oracle.route(n["topk_idx"], n["tokens_per_shard"], sh.num_experts, sh.num_local_experts, sh.local_rank)
    got = run.layout_host()
    assert np.array_equal(got["send"], rt.send) and np.array_equal(got["recv"], rt.recv)
    px, psf, pm, off = oracle.fill_pool(n["x"], None, rt, run.moe.block_m, sh.topk,
                                        shared_shard=sh.local_rank if nsh else None,
                                        shared_tokens=n["tokens_per_shard"][sh.local_rank] if nsh else 0)
    assert psf is None
    assert np.array_equal(got["pool_off"], off), "pool offsets"
    gp = _pool_rows(run)
    assert gp.shape == px.shape
    assert np.array_equal(gp.view(np.uint32), px.view(np.uint32)), "pool rows"
    return rt, off, pm


def _whole(run, n):
    sh = run.shape
    ref = oracle.forward(n, sh.num_experts, sh.num_local_experts, sh.local_rank, sh.block_m,
                         num_shared_experts=sh.num_shared_experts)
    y = run.y_host()
    valid = ~np.isnan(ref["y"])
    tol_check(y[valid], ref["y"][valid], sh.name)
    assert np.all(np.isnan(y[~valid]))
    return ref


_CASES = {
    "bm64_ragged": (MoEShape("bf64", 3, 200, 512, 384, 16, 8, 4, 64, local_rank=1, weight_format="bf16", seed=201),
                    [200, 0, 137]),
    "bm128": (MoEShape("bf128", 2, 400, 1024, 512, 16, 8, 4, 128, weight_format="bf16", seed=202), [400, 263]),
    "bm64_shared": (MoEShape("bf64sh", 3, 130, 512, 256, 24, 8, 4, 64, local_rank=2, num_shared_experts=1,
                             weight_format="bf16", seed=203), [130, 71, 99]),
    "bm128_zipf": (MoEShape("bf128z", 4, 256, 768, 256, 32, 8, 4, 128, routing="zipf", weight_format="bf16",
                            seed=204), [256, 256, 190, 33]),
    "short_k": (MoEShape("bfshort", 2, 150, 256, 128, 8, 4, 2, 64, local_rank=1, weight_format="bf16", seed=205),
                [150, 88]),
}


@pytest.mark.parametrize("case", list(_CASES))
def test_bf16_whole_layer(case):
    """Layout and pool rows bit for bit, the whole output within tolerance (also K loops shorter than
    the load pipeline: GEMM1 has 2H/128 = 4 steps per tile and GEMM2 2 steps with "short_k")."""
    sh, tps = _CASES[case]
    print(f"[case] bf16 whole layer {case}", flush=True)
    inp = make_inputs(sh, tokens_per_shard=tps)
    run = Run(sh, inputs=inp)
    assert run.status == 0
    n = inputs_np(run)
    _check_layout_bf16(run, n)
    _whole(run, n)
    run.close()


def test_bf16_l2_pool_follows_the_bf16_swiglu():
    """The L2 pool holds GEMM1's SwiGLU rounded to bf16: against the oracle's (fp64 sums), nearly all
    values equal and the rest one bf16 step apart; comb rows within tolerance."""
    sh = MoEShape("bfmid", 2, 300, 1024, 512, 8, 8, 4, 64, weight_format="bf16", seed=206)
    print(f"[case] bf16 L2 pool {sh.name}", flush=True)
    run = Run(sh)
    n = inputs_np(run)
    rt, off, pm = _check_layout_bf16(run, n)
    ref = oracle.forward(n, sh.num_experts, sh.num_local_experts, 0, sh.block_m, keep_rows=True)
    l2 = _l2_rows(run)
    for le in range(sh.num_local_experts):
        base, cnt = int(off[le]) * sh.block_m, int(rt.recv_tot[le])
        if cnt == 0:
            continue
        got, want = l2[base:base + cnt], ref["parts"][le]["l2"]
        assert np.mean(got == want) > 0.99, le
        # one bf16 step of the value, plus an absolute term for values near zero, where the gate's sum
        # cancels and GEMM1's fp32 accumulation (against fp64 in the oracle) moves it by ~1e-8
        step = np.abs(want) * 2.0 ** -7 * 1.01 + 1e-5 * np.abs(want).max()
        d = np.abs(got - want)
        assert np.all(d <= step), (le, float((d / step).max()))
        rows = np.stack([run.comb_row(int(k), int(s), int(t)) for s, t, k in pm[base:base + cnt]])
        tol_check(rows, ref["rows"][le], f"comb rows expert {le}")
    run.close()


@pytest.mark.parametrize("shape", [
    MoEShape("bfx64", 2, 200, 512, 256, 8, 8, 2, 64, weight_format="bf16", seed=207),
    MoEShape("bfx128", 1, 300, 2048, 256, 4, 4, 2, 128, weight_format="bf16", seed=208),
], ids=lambda s: s.name)
def test_bf16_gemm1_bit_exact(shape):
    """Integer bf16 values: GEMM1's fp32 output equals the int64 product exactly."""
    print(f"[case] bf16 gemm1 exact {shape.name}", flush=True)
    inp = make_inputs(shape, integer_codes=True)
    run = Run(shape, inputs=inp, flags=mm.FLAG_KEEP_GEMM1_OUTPUT)
    n = inputs_np(run)
    rt, off, _ = _check_layout_bf16(run, n)
    px, _, _, _ = oracle.fill_pool(n["x"], None, rt, shape.block_m, shape.topk)
    cap = run.moe.layout["max_pool_blocks"] * run.moe.block_m
    g1 = run.region("gemm1_out", torch.float32, (cap, 2 * shape.intermediate))
    for le in range(shape.num_local_experts):
        base, cnt = int(off[le]) * shape.block_m, int(rt.recv_tot[le])
        if cnt == 0:
            continue
        want = (px[base:base + cnt].astype(np.int64) @ n["w1"][le].astype(np.int64).T).astype(np.float32)
        got = g1[base:base + cnt].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"expert {le}"
    run.close()


@pytest.mark.parametrize("shape", [
    MoEShape("bfx2_64", 2, 150, 768, 384, 8, 4, 2, 64, weight_format="bf16", seed=209),
    MoEShape("bfx2_128", 2, 260, 1024, 1024, 4, 4, 2, 128, weight_format="bf16", seed=210),
], ids=lambda s: s.name)
def test_bf16_gemm2_bit_exact_on_placed_activations(shape):
    """Route + fill + GEMM1, then integer bf16 values placed in the L2 pool and GEMM2 run alone: every
    combine row equals bf16(h W2^T) of the oracle bit for bit."""
    print(f"[case] bf16 gemm2 exact {shape.name}", flush=True)
    inp = make_inputs(shape, integer_codes=True)
    run = Run(shape, inputs=inp)
    n = inputs_np(run)
    rt, off, pm = _check_layout_bf16(run, n)
    P = int(off[-1]) * shape.block_m
    I, bm = shape.intermediate, shape.block_m
    rng = np.random.default_rng(9)
    h = rng.integers(-8, 9, (P, I)).astype(np.float32)
    nb = P // bm
    tiled = h.reshape(nb, bm, I // 64, 4, 16).transpose(0, 2, 3, 1, 4)
    L = run.moe.layout
    dst = run.region("l2_x", torch.bfloat16, (L["max_pool_blocks"] * bm * I,))
    dst[:P * I] = torch.from_numpy(np.ascontiguousarray(tiled).reshape(-1)).to(torch.bfloat16).cuda()
    g = run.inp_gpu
    mm.mega_moe_forward_stages(run.moe.h, mm.STAGE_GEMM2, g["tokens_per_shard"], None, None, None, None,
                               None, None, g["w2_packed"], None, None)
    torch.cuda.synchronize()
    assert run.moe.status() == 0
    for le in range(shape.num_local_experts):
        base, cnt = int(off[le]) * bm, int(rt.recv_tot[le])
        if cnt == 0:
            continue
        want = oracle.bf16_bits(oracle.bf16_round(h[base:base + cnt].astype(np.float64) @
                                                  n["w2"][le].astype(np.float64).T))
        for j in range(cnt):
            s, t, k = (int(v) for v in pm[base + j])
            assert np.array_equal(oracle.bf16_bits(run.comb_row(k, s, t)), want[j]), (le, j)
    run.close()


def test_bf16_repeat_and_poisoned_workspace_identical():
    sh, tps = _CASES["bm64_shared"]
    print("[case] bf16 repeat and poison", flush=True)
    inp = make_inputs(sh, tokens_per_shard=tps)
    clean = Run(sh, inputs=inp, repeat=2)
    pois = Run(sh, inputs=inp, flags=mm.FLAG_DEBUG_POISON, repeat=2)
    # both GEMMs in one launch over a poisoned workspace: a GEMM2 load overtaking GEMM1's stores would show
    pois1 = Run(sh, inputs=inp, flags=mm.FLAG_DEBUG_POISON | mm.FLAG_ONE_GEMM_LAUNCH, repeat=2)
    assert clean.status == 0 and pois.status == 0 and pois1.status == 0
    for y in clean.ys + pois.ys + pois1.ys:
        for i, cnt in enumerate(tps):
            assert torch.equal(y[i, :cnt].view(torch.int16), clean.ys[0][i, :cnt].view(torch.int16))
    clean.close()
    pois.close()
    pois1.close()


def test_bf16_full_size_decode_sampled_tokens():
    """The decode workload's shape with BF16 weights (BLOCK_M 64, 32 experts of H 7168, I 2048): whole
    routing layout, and 12 sampled tokens plus tokens without a local expert against the oracle's
    per-token path."""
    sh = SHAPES["decode"].replace(weight_format="bf16")
    print(f"[case] bf16 full-size {sh.name}", flush=True)
    run = Run(sh, generate_on="cuda")
    assert run.status == 0
    n = inputs_np(run)
    _check_layout_bf16(run, n)
    y = run.y_host()
    for s, t in sample_tokens(n, sh, 12, seed=3):
        want = oracle.direct_token(n, s, t, sh.num_local_experts, sh.local_rank)
        tol_check(y[s, t], want, f"token ({s},{t})")
    run.close()


@pytest.mark.parametrize("case", ["max_hidden", "max_intermediate"])
def test_bf16_maximum_sizes_whole_layer(case):
    """The configuration maxima with bf16 operands: H = 16384 (rows of 32 KB, 256 K steps of 64 values in
    GEMM1, 32 fill chunks per lane) and I = 16384 (256 K steps in GEMM2, 128 GEMM1 n tiles)."""
    print(f"[case] bf16 maximum sizes {case}", flush=True)
    if case == "max_hidden":
        sh = MoEShape("bfmaxh", 2, 24, 16384, 4096, 2, 1, 1, 64, weight_format="bf16", seed=211)
        tps = [24, 19]
    else:
        sh = MoEShape("bfmaxi", 2, 24, 4096, 16384, 2, 1, 1, 64, weight_format="bf16", seed=212)
        tps = [24, 11]
    inp = make_inputs(sh, device="cuda", tokens_per_shard=tps)
    run = Run(sh, inputs=inp)
    assert run.status == 0
    n = inputs_np(run)
    _check_layout_bf16(run, n)
    _whole(run, n)
    run.close()


def _bf16_sweep(n=16, seed=2031):
    """Random small BF16 layers: BLOCK_M 64/128, H 256-1024, I 128-512, 1-16 local experts on 1, 2 or 4
    ranks, top-1..8, 1-4 shards with random (possibly zero) token counts, uniform or Zipf routing, with
    or without a shared expert."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        bm = int(rng.choice([64, 128]))
        H = int(rng.choice([256, 512, 768, 1024]))
        I = int(rng.choice([128, 256, 384, 512]))
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
        out.append((MoEShape(f"bfsweep{i}", S, T, H, I, E, El, K, bm, local_rank=rank, routing=routing,
                             num_shared_experts=nsh, weight_format="bf16", seed=600 + i), tps))
    return out


_BF16_SWEEP = _bf16_sweep()


@pytest.mark.parametrize("case", range(len(_BF16_SWEEP)), ids=[sh.name for sh, _ in _BF16_SWEEP])
def test_bf16_random_configs_whole_layer(case):
    """Each seeded configuration: layout and pool rows bit for bit, the whole output within tolerance,
    a clean status."""
    sh, tps = _BF16_SWEEP[case]
    print(f"[case] bf16 sweep {sh.name} bm={sh.block_m} H={sh.hidden} I={sh.intermediate} "
          f"E={sh.num_experts}/{sh.num_local_experts} K={sh.topk} tps={tps} shared={sh.num_shared_experts}",
          flush=True)
    inp = make_inputs(sh, tokens_per_shard=tps)
    run = Run(sh, inputs=inp)
    assert run.status == 0
    n = inputs_np(run)
    _check_layout_bf16(run, n)
    _whole(run, n)
    run.close()


def _sched_words(moe):
    n = 64 + 2 * moe.layout["max_pool_blocks"]
    return moe.region("sched", torch.int32, (n,)).cpu().numpy()


def _one_launch_matches(sh, tps):
    inp = make_inputs(sh, device="cuda", tokens_per_shard=tps)
    base = mm.MegaMoE.from_shape(sh)
    want = base(inp)
    torch.cuda.synchronize()
    assert base.status() == 0
    nb = int(base.region("status", torch.int32, (2,))[1].item())
    L = base.layout
    l2_want = base.region("l2_x", torch.int16, (L["max_pool_blocks"], sh.intermediate * base.block_m))[:nb].clone()
    moe = mm.MegaMoE.from_shape(sh, flags=mm.FLAG_ONE_GEMM_LAUNCH)
    for _ in range(2):
        got = moe(inp)
        torch.cuda.synchronize()
        assert moe.status() == 0
        assert not _sched_words(moe).any(), "schedule words left non-zero"
        l2 = moe.region("l2_x", torch.int16, (L["max_pool_blocks"], sh.intermediate * moe.block_m))[:nb]
        assert torch.equal(l2, l2_want), "L2 pool"
        for i, n in enumerate(tps):
            assert torch.equal(got[i, :n].view(torch.int16), want[i, :n].view(torch.int16)), i
    moe.close()
    base.close()


@pytest.mark.parametrize("case", ["bm64_ragged", "bm128_waves"])
def test_bf16_one_gemm_launch_matches_stream_order(case):
    """Both BF16 GEMMs in one persistent launch (each GEMM2 tile waits on its block's count of finished
    GEMM1 n tiles, in expert waves per XCD): the L2 pool and the output bit for bit as the stream-ordered
    kernels give them, twice in a row, with a clean status and every schedule word back at zero."""
    print(f"[case] bf16 one GEMM launch {case}", flush=True)
    if case == "bm64_ragged":
        sh = MoEShape("bf1l64", 5, 333, 1024, 256, 64, 16, 6, 64, local_rank=1, weight_format="bf16", seed=211)
        tps = [333, 0, 101, 7, 250]
    else:
        sh = MoEShape("bf1lw", 4, 1024, 512, 1024, 128, 64, 8, 128, local_rank=1, weight_format="bf16", seed=212)
        tps = [1024, 1000, 777, 1024]
    _one_launch_matches(sh, tps)


@pytest.mark.parametrize("case", range(len(_BF16_SWEEP)), ids=[sh.name for sh, _ in _BF16_SWEEP])
def test_bf16_random_configs_one_gemm_launch(case):
    """The seeded BF16 configurations with both GEMMs in one launch: bits equal to stream order."""
    sh, tps = _BF16_SWEEP[case]
    print(f"[case] bf16 one GEMM launch {sh.name} tps={tps}", flush=True)
    _one_launch_matches(sh, tps)


def test_bf16_one_gemm_launch_forced_timeout_latches_and_recovers():
    """BF16 weights with both GEMMs in one launch, its bounded GEMM2 waits forced from the host to give
    up at once: the status word reports TIMEOUT, the launch completes and zeroes its schedule words,
    and a normal handle on the same inputs then matches the oracle."""
    print("[case] bf16 one GEMM launch, forced wait timeout", flush=True)
    sh = MoEShape("bftmo", 2, 80, 256, 128, 8, 4, 2, 64, weight_format="bf16", seed=213)
    inp = make_inputs(sh, device="cuda")
    forced = mm.MegaMoE.from_shape(sh, flags=mm.FLAG_ONE_GEMM_LAUNCH | mm.FLAG_DEBUG_FORCE_TIMEOUT)
    for _ in range(2):
        forced(inp)
        torch.cuda.synchronize()
        assert forced.status() == mm.STATUS_TIMEOUT
        assert not _sched_words(forced).any()
    forced.close()
    run = Run(sh, inputs=inp, flags=mm.FLAG_ONE_GEMM_LAUNCH)
    assert run.status == 0
    n = inputs_np(run)
    _check_layout_bf16(run, n)
    _whole(run, n)
    run.close()
