"""Parity at the full workload sizes on whole outputs (not samples), and the combine stage alone on
hand-set expert rows."""
import numpy as np
import pytest
import torch

import dispatch_fp8_grouped_amd as mm
import oracle
from inputs import SHAPES, MoEShape, make_inputs, to_numpy

from gpu_util import Run, check_layout, inputs_np, tol_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("weight_format", ["fp8", "mxfp4", "bf16"])
def test_decode_whole_output(weight_format):
    """The decode-shaped share (8 x 128 tokens, H 7168, I 2048, 32 of 256 experts, BLOCK_M 64), with each
    weight format: the routing counts bit for bit (and, with FP8 or MXFP4 weights, the whole layout) and
    every output row against the oracle."""
    print(f"[case] decode whole y, {weight_format} weights", flush=True)
    sh = SHAPES["decode"].replace(weight_format=weight_format)
    run = Run(sh)
    assert run.status == 0
    n = inputs_np(run)
    if weight_format == "bf16":
        rt = oracle.route(n["topk_idx"], n["tokens_per_shard"], sh.num_experts, sh.num_local_experts,
                          sh.local_rank)
        got = run.layout_host()
        assert np.array_equal(got["send"], rt.send) and np.array_equal(got["recv"], rt.recv)
    else:
        check_layout(run, n)
    ref = oracle.forward(n, sh.num_experts, sh.num_local_experts, sh.local_rank, sh.block_m)
    y = run.y_host()
    valid = ~np.isnan(ref["y"])
    tol_check(y[valid], ref["y"][valid], "decode y")
    run.close()


def _expert_rows(run, n, experts):
    """Every combine row of the given local experts against the oracle's bf16 expert outputs."""
    sh = run.shape
    ref = oracle.forward(n, sh.num_experts, sh.num_local_experts, sh.local_rank, sh.block_m,
                         experts=experts, keep_rows=True)
    off, pm = ref["off"], ref["pool_meta"]
    S, T = sh.num_shards, sh.max_tokens_per_shard
    comb = run.region("comb", torch.int16, (sh.topk, S * T, sh.hidden))
    for le in experts:
        base, nrows = int(off[le]) * sh.block_m, int(ref["route"].recv_tot[le])
        if nrows == 0:
            continue
        meta = pm[base:base + nrows].astype(np.int64)
        rows = torch.from_numpy(meta[:, 0] * T + meta[:, 1]).cuda()
        planes = torch.from_numpy(meta[:, 2]).cuda()
        got = comb[planes, rows].cpu().view(torch.bfloat16).to(torch.float64).numpy()
        tol_check(got, ref["rows"][le], f"{sh.name} expert {le} ({nrows} rows)")
    return ref


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_full_size_hot_and_last_experts(name):
    """At the full prefill and skewed sizes: every combine row of the hottest local expert (skewed: ~30x
    the mean rows) and of the last one, whose tiles fill the partial last round of both GEMMs."""
    print(f"[case] full-size expert rows {name}", flush=True)
    sh = SHAPES[name]
    run = Run(sh)
    assert run.status == 0
    n = inputs_np(run)
    rt, _ = check_layout(run, n)
    hot = int(np.argmax(rt.recv_tot))
    _expert_rows(run, n, sorted({hot, sh.num_local_experts - 1}))
    run.close()


def test_combine_stage_alone_reproduces_weighted_sum():
    """The combine stage by itself on expert rows placed by hand: a token routed to experts 2 and 7 with
    weights 0.73 and 0.27 gets 0.73*E2 + 0.27*E7 ("Dispatch/Combine: blog theory vs DeepEP vs DeepGEMM
    Mega MoE", section 1); a masked slot (id < 0) and slots of other ranks' experts add nothing; a token
    with no local expert gets zeros; rows t >= T_s are left untouched."""
    print("[case] combine stage alone", flush=True)
    sh = MoEShape("comb", 1, 6, 512, 128, 16, 8, 2, 64, seed=40)        # experts 0..7 local (rank 0)
    moe = mm.MegaMoE.from_shape(sh)
    S, T, H, K = 1, 6, 512, 2
    idx = torch.tensor([[[2, 7], [3, -1], [9, 12], [1, 10], [4, 5], [0, 6]]], dtype=torch.int64)
    wts = torch.tensor([[[0.73, 0.27], [0.6, 0.4], [0.5, 0.5], [0.3, 0.7], [0.25, 0.75], [0.9, 0.1]]],
                       dtype=torch.float32)
    rng = np.random.default_rng(7)
    rows = oracle.bf16_round(rng.normal(size=(K, S * T, H)))          # the hand-set expert outputs
    comb = moe.region("comb", torch.int16, (K, S * T, H))
    comb.copy_(torch.from_numpy(rows).to(torch.bfloat16).view(torch.int16).cuda())
    y = torch.full((S, T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    tps = [5]                                                          # token 5 is past T_s
    mm.mega_moe_forward_stages(moe.h, mm.STAGE_COMBINE, tps, None, None, idx.cuda(), wts.cuda(), None, None,
                               None, None, y)
    torch.cuda.synchronize()
    assert moe.status() == 0
    got = y.to(torch.float64).cpu().numpy()
    w = wts.numpy().astype(np.float64)
    want = np.zeros((S, T, H))
    want[0, 0] = 0.73 * rows[0, 0] + 0.27 * rows[1, 0]                   # 0.73 E2 + 0.27 E7
    want[0, 1] = 0.6 * rows[0, 1]                                        # the masked slot adds nothing
    want[0, 3] = 0.3 * rows[0, 3]                                        # expert 10 belongs to rank 1
    want[0, 4] = w[0, 4, 0] * rows[0, 4] + w[0, 4, 1] * rows[1, 4]
    want = oracle.bf16_round(want)
    tol_check(got[0, :5], want[0, :5], "combine")
    assert np.all(got[0, 2] == 0.0), "token with no local expert"
    assert np.all(np.isnan(got[0, 5])), "row past T_s written"
    # the identity itself, in the combine's fp32 arithmetic: one rounding to bf16 of the fp32 sum
    e2, e7 = rows[0, 0].astype(np.float32), rows[1, 0].astype(np.float32)
    fp32 = np.float32(0.73) * e2 + np.float32(0.27) * e7
    assert np.max(np.abs(got[0, 0] - oracle.bf16_round(fp32.astype(np.float64)))) <= \
        2.0 ** -7 * np.max(np.abs(fp32)), "0.73*E2 + 0.27*E7"
    moe.close()


def test_tile_runs_longer_than_the_lookup_table():
    """A GEMM1 launch with more than 128 tiles per work-group (I = 16384: 128 n tiles per pool block,
    ~264 blocks), so each work-group finds its first 128 tiles in the LDS table and the rest by the
    search over the expert offsets.  The last expert's tiles come last in the tile order, where the
    search takes over: every combine row of it against the oracle, and the layout bit for bit."""
    print("[case] tile runs past the lookup table", flush=True)
    sh = MoEShape("longrun", 8, 2056, 256, 16384, 8, 8, 1, 64, seed=41)
    run = Run(sh)
    assert run.status == 0
    n = inputs_np(run)
    rt, _ = check_layout(run, n)
    nblocks = int(run.layout_host()["nblocks"])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = (cus + 7) // 8 * 8
    tiles = nblocks * (sh.intermediate // 128)
    assert tiles > 128 * grid, (tiles, grid)            # some work-groups run past the table
    _expert_rows(run, n, [sh.num_local_experts - 1])
    run.close()
