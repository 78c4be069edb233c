"""GPU edge cases: degenerate counts, empty and ragged inputs, sentinels, status bits, repeats,
cumulative stats, host validation on a live handle, stage timing."""
import numpy as np
import pytest
import torch

import dispatch_fp8_grouped_amd as mm
import oracle
from inputs import SHAPES, MoEShape, make_inputs, to_numpy

from gpu_util import Run, check_layout, tol_check, on_gpu, inputs_np

pytestmark = pytest.mark.gpu


def _whole(run, inp):
    sh = run.shape
    ref = oracle.forward(inp, sh.num_experts, sh.num_local_experts, sh.local_rank, sh.block_m,
                         num_shared_experts=sh.num_shared_experts)
    y = run.y_host()
    valid = ~np.isnan(ref["y"])
    tol_check(y[valid], ref["y"][valid], sh.name)
    return ref


def test_block_boundary_counts():
    """Experts receiving 0, BM-1, BM, BM+1, 1 and 2*BM rows (BM = 64)."""
    print("[case] block boundary counts", flush=True)
    counts = [0, 63, 64, 65, 1, 128]
    sh = MoEShape("bounds", 2, 161, 256, 256, 6, 6, 1, 64, seed=21)
    inp = make_inputs(sh)
    ids = np.concatenate([np.full(c, e) for e, c in enumerate(counts)])
    np.random.default_rng(0).shuffle(ids)
    flat = np.full(2 * 161, -1, dtype=np.int64)
    flat[:len(ids)] = ids
    inp["topk_idx"] = torch.from_numpy(flat.reshape(2, 161, 1))
    run = Run(sh, inputs=inp)
    n = inputs_np(run)
    rt, off = check_layout(run, n)
    assert rt.recv_tot.tolist() == counts
    assert off.tolist() == [0, 0, 1, 2, 4, 5, 7]
    _whole(run, n)
    run.close()


def test_all_tokens_one_expert_and_sentinels():
    print("[case] one hot expert + -1 entries", flush=True)
    sh = MoEShape("hot", 2, 300, 256, 128, 4, 4, 2, 64, seed=22)
    inp = make_inputs(sh)
    idx = torch.full((2, 300, 2), -1, dtype=torch.int64)
    idx[:, :, 0] = 2
    idx[0, ::7, 1] = 3
    inp["topk_idx"] = idx
    run = Run(sh, inputs=inp)
    n = inputs_np(run)
    rt, off = check_layout(run, n)
    assert rt.recv_tot[2] == 600
    _whole(run, n)
    run.close()


def test_random_negative_entries_and_remote_rank():
    print("[case] sentinel entries, local_rank 3", flush=True)
    sh = MoEShape("neg", 4, 96, 512, 256, 32, 8, 4, 64, local_rank=3, seed=23)
    inp = make_inputs(sh)
    drop = torch.rand(inp["topk_idx"].shape, generator=torch.Generator().manual_seed(1)) < 0.2
    inp["topk_idx"][drop] = -1
    run = Run(sh, inputs=inp, tokens_per_shard=None)
    n = inputs_np(run)
    check_layout(run, n)
    _whole(run, n)
    run.close()


def test_many_local_experts():
    """More than 64 local experts: routing keeps the per-expert slot counters in LDS instead of lanes."""
    print("[case] 128 local experts", flush=True)
    sh = MoEShape("manylocal", 3, 200, 256, 128, 512, 128, 6, 64, local_rank=1, seed=25)
    inp = make_inputs(sh, tokens_per_shard=[200, 57, 131])
    run = Run(sh, inputs=inp)
    n = inputs_np(run)
    rt, _ = check_layout(run, n)
    assert (rt.recv_tot > 0).sum() > 64
    _whole(run, n)
    run.close()


def test_repeat_calls_identical_and_state_clean():
    """Two calls give identical bits; a call on other routing in between does not leak state."""
    print("[case] repeat calls", flush=True)
    sh = SHAPES["mid"].replace(max_tokens_per_shard=256)
    a = make_inputs(sh, device="cuda")
    b = make_inputs(sh, device="cuda", seed=99, tokens_per_shard=[256, 3, 100, 0])
    moe = mm.MegaMoE.from_shape(sh)
    y1 = moe(a)
    moe(b)
    y2 = moe(a)
    moe(a)
    y3 = moe(a)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    assert moe.status() == 0
    moe.close()


def test_cumulative_recv_stats():
    print("[case] cumulative stats", flush=True)
    sh = SHAPES["tiny"]
    cum = torch.full((sh.num_local_experts,), 5, dtype=torch.int32, device="cuda")
    run = Run(sh, cum=cum, repeat=3)
    n = inputs_np(run)
    rt = oracle.route(n["topk_idx"], n["tokens_per_shard"], sh.num_experts, sh.num_local_experts, 0)
    assert cum.cpu().numpy().tolist() == (5 + 3 * rt.recv_tot).tolist()
    run.close()


def test_bad_expert_id_sets_status_and_is_skipped():
    print("[case] bad expert id", flush=True)
    sh = SHAPES["tiny"]
    inp = make_inputs(sh)
    inp["topk_idx"][0, 5, 1] = 8        # E = 8
    inp["topk_idx"][0, 9, 0] = 1000
    run = Run(sh, inputs=inp)
    assert run.status & mm.STATUS_BAD_EXPERT_ID
    assert run.moe.status() == 0        # read-and-clear
    n = inputs_np(run)
    check_layout(run, n)
    _whole(run, n)
    run.close()


@pytest.mark.parametrize("route", ["one_group", "three_launches"])
def test_slot_overflow_status_and_clamped_layout(route):
    print(f"[case] slot overflow, routing {route}", flush=True)
    sh = MoEShape("dup", 1, 4, 256, 128, 2, 2, 2, 64, seed=24)
    inp = make_inputs(sh)
    inp["topk_idx"][:] = 0               # the same expert twice per token: 8 entries, 4 slots
    # poisoned workspace: a combine row the forward never wrote would read as NaN
    flags = mm.FLAG_DEBUG_POISON | (mm.FLAG_DEBUG_ROUTE_LAUNCHES if route == "three_launches" else 0)
    run = Run(sh, inputs=inp, flags=flags)
    assert run.status & mm.STATUS_SLOT_OVERFLOW
    n = inputs_np(run)
    rt, _ = check_layout(run, n)
    assert rt.recv[0, 0] == 4
    # the dropped entries add nothing to y, as in the oracle (their combine rows are never computed)
    ref = oracle.forward(n, sh.num_experts, sh.num_local_experts, sh.local_rank, sh.block_m)
    assert ref["route"].slot_overflow
    _whole(run, n)
    run.close()


def test_host_validation_on_live_handle():
    sh = SHAPES["tiny"]
    inp = on_gpu(make_inputs(sh))
    moe = mm.MegaMoE.from_shape(sh)
    w1p, w2p = moe.pack_weights(inp["w1"], inp["w2"])
    with pytest.raises(mm.MegaMoEError) as ei:
        moe.forward([65], inp["x"], inp["x_sf"], inp["topk_idx"], inp["topk_weights"], w1p,
                    inp["w1_sf"], w2p, inp["w2_sf"])
    assert ei.value.code == mm.ERR_TOO_MANY_TOKENS
    with pytest.raises(mm.MegaMoEError) as ei:
        mm.mega_moe_forward_stages(moe.h, 0x20, [64], inp["x"], inp["x_sf"], inp["topk_idx"],
                                   inp["topk_weights"], inp["w1"], inp["w1_sf"], inp["w2"], inp["w2_sf"],
                                   torch.empty(1, 64, 256, dtype=torch.bfloat16, device="cuda"))
    assert ei.value.code == mm.ERR_INVALID_ARG
    with pytest.raises(mm.MegaMoEError) as ei:     # GEMM1 without weights
        mm.mega_moe_forward_stages(moe.h, mm.STAGE_GEMM1, [64], None, None, None, None, None, None, None,
                                   None, None)
    assert ei.value.code == mm.ERR_INVALID_ARG
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(mm.MegaMoEError) as ei:
        mm.mega_moe_init(moe.cfg, small)
    assert ei.value.code == mm.ERR_WORKSPACE_TOO_SMALL
    moe.close()


def test_pack_weights_layout():
    """The packed weights hold every byte of W1 / W2 at the documented tiled position."""
    print("[case] weight pack layout", flush=True)
    sh = MoEShape("pack", 1, 8, 512, 384, 6, 3, 2, 64, seed=26)
    inp = on_gpu(make_inputs(sh))
    moe = mm.MegaMoE.from_shape(sh)
    w1p, w2p = moe.pack_weights(inp["w1"], inp["w2"])
    torch.cuda.synchronize()
    El, H, I = sh.num_local_experts, sh.hidden, sh.intermediate
    w1 = inp["w1"].cpu().numpy()
    w2 = inp["w2"].cpu().numpy()
    # W1: n tile nt stacks gate rows nt*128.. and up rows I + nt*128..; then K chunks of 128
    rows1 = np.concatenate([np.stack([w1[:, nt * 128:(nt + 1) * 128], w1[:, I + nt * 128:I + (nt + 1) * 128]], 1)
                            .reshape(El, 256, H) for nt in range(I // 128)], 0)      # [NT*El, 256, H]
    rows1 = rows1.reshape(I // 128, El, 256, H).transpose(1, 0, 2, 3)
    want1 = rows1.reshape(El, I // 128, 256, H // 128, 128).transpose(0, 1, 3, 2, 4)
    assert np.array_equal(w1p.cpu().numpy(), want1)
    want2 = w2.reshape(El, H // 256, 256, I // 128, 128).transpose(0, 1, 3, 2, 4)
    assert np.array_equal(w2p.cpu().numpy(), want2)
    # the layer on the packed weights matches the oracle
    run = Run(sh, inputs=inp)
    _whole(run, inputs_np(run))
    run.close()
    moe.close()


def test_pack_scales_layout():
    """The packed MXFP4 exponents hold every byte of the row-major exponents at the documented position:
    chunk (le, nt, kb), row r, byte j = exponent block 4*kb + j of the chunk's weight row r."""
    print("[case] mxfp4 exponent pack layout", flush=True)
    sh = MoEShape("packsf", 1, 8, 512, 384, 6, 3, 2, 64, seed=27, weight_format="mxfp4")
    inp = on_gpu(make_inputs(sh))
    moe = mm.MegaMoE.from_shape(sh)
    s1p, s2p = moe.pack_scales(inp["w1_sf"], inp["w2_sf"])
    torch.cuda.synchronize()
    El, H, I = sh.num_local_experts, sh.hidden, sh.intermediate
    s1 = inp["w1_sf"].cpu().numpy()
    s2 = inp["w2_sf"].cpu().numpy()
    want1 = np.empty((El, I // 128, H // 128, 256, 4), np.uint8)
    for nt in range(I // 128):
        for r in range(256):
            row = nt * 128 + r if r < 128 else I + nt * 128 + r - 128
            want1[:, nt, :, r, :] = s1[:, row, :].reshape(El, H // 128, 4)
    want2 = s2.reshape(El, H // 256, 256, I // 128, 4).transpose(0, 1, 3, 2, 4)
    assert np.array_equal(s1p.cpu().numpy(), want1)
    assert np.array_equal(s2p.cpu().numpy(), want2)
    moe.close()


def test_stage_timing():
    sh = SHAPES["tiny"]
    inp = on_gpu(make_inputs(sh))
    moe = mm.MegaMoE.from_shape(sh)
    mm.mega_moe_set_timing(moe.h, True)
    for _ in range(70):                 # more forwards than the event ring holds
        moe(inp)
    t, n = mm.mega_moe_stage_times(moe.h, with_count=True)
    assert n == 70 and len(t) == 5 and all(v > 0 for v in t)
    mm.mega_moe_set_timing(moe.h, True)  # reset
    moe(inp, stages=mm.STAGE_ROUTE | mm.STAGE_FILL)
    t, n = mm.mega_moe_stage_times(moe.h, with_count=True)
    assert n == 1 and t[0] > 0 and t[1] > 0 and t[2] == t[3] == t[4] == 0
    mm.mega_moe_set_timing(moe.h, False)
    moe(inp)
    assert mm.mega_moe_stage_times(moe.h, with_count=True)[1] == 0     # the reset cleared the count
    moe.close()
    # the fill inside GEMM1's launch is timed with GEMM1
    fused = mm.MegaMoE.from_shape(sh, flags=mm.FLAG_FILL_IN_GEMM1)
    mm.mega_moe_set_timing(fused.h, True)
    fused(inp)
    t, n = mm.mega_moe_stage_times(fused.h, with_count=True)
    assert n == 1 and t[1] == 0 and all(t[i] > 0 for i in (0, 2, 3, 4))
    fused.close()
    # GEMM2 inside GEMM1's launch is timed with GEMM1
    one = mm.MegaMoE.from_shape(sh, flags=mm.FLAG_ONE_GEMM_LAUNCH)
    mm.mega_moe_set_timing(one.h, True)
    one(inp)
    t, n = mm.mega_moe_stage_times(one.h, with_count=True)
    assert n == 1 and t[3] == 0 and all(t[i] > 0 for i in (0, 1, 2, 4))
    one.close()
    # routing, the pull and both GEMMs in one launch: all timed with GEMM1
    alls = mm.MegaMoE.from_shape(sh, flags=mm.FLAG_ROUTE_IN_LAUNCH)
    mm.mega_moe_set_timing(alls.h, True)
    alls(inp)
    t, n = mm.mega_moe_stage_times(alls.h, with_count=True)
    assert n == 1 and t[0] == t[1] == t[3] == 0 and t[2] > 0 and t[4] > 0
    alls.close()


@pytest.mark.parametrize("route", ["default", "three_launches"])
@pytest.mark.parametrize("case", ["zipf_uneven", "many_shards", "zipf_small"])
def test_route_stage_places_pool_rows(case, route):
    """The routing stage alone writes every pool row's metadata and scatter target (the round-robin
    position of each table entry, padding rows all ones), over poisoned workspace contents, with the
    routing the library picks (one work-group for zipf_small; counts and scan in one launch for the
    others, whose shards hold at most 8 chunks) and with the three-launch routing."""
    print(f"[case] route-only pool metadata {case}, routing {route}", flush=True)
    if case == "zipf_uneven":
        sh = MoEShape("rz", 6, 300, 256, 128, 64, 16, 6, 64, local_rank=2, routing="zipf", seed=31)
        tps = [300, 0, 17, 299, 151, 64]
    elif case == "many_shards":
        sh = MoEShape("rs", 64, 40, 256, 128, 32, 8, 4, 64, local_rank=1, seed=32)
        tps = [(7 * i) % 41 for i in range(64)]
    else:                                   # small enough for the one-work-group routing
        sh = MoEShape("rq", 2, 120, 256, 128, 64, 16, 8, 64, local_rank=3, routing="zipf", seed=33)
        tps = [120, 77]
    inp = make_inputs(sh, tokens_per_shard=tps)
    moe = mm.MegaMoE.from_shape(sh, flags=mm.FLAG_DEBUG_ROUTE_LAUNCHES if route == "three_launches" else 0)
    cap = moe.layout["max_pool_blocks"] * moe.block_m
    moe.region("pool_meta", torch.int32, (cap, 3)).fill_(0x5A5A5A5A)
    moe.region("pool_dst", torch.int32, (cap,)).fill_(0x5A5A5A5A)
    g = on_gpu(inp)
    moe(g, stages=mm.STAGE_ROUTE)
    torch.cuda.synchronize()
    n = to_numpy(inp)
    rt = oracle.route(n["topk_idx"], n["tokens_per_shard"], sh.num_experts, sh.num_local_experts, sh.local_rank)
    _, _, pm, _ = oracle.fill_pool(n["x"], n["x_sf"], rt, moe.block_m, sh.topk)
    rows = pm.shape[0]
    gm = moe.region("pool_meta", torch.int32, (cap, 3))[:rows].cpu().numpy().view(np.uint32)
    gd = moe.region("pool_dst", torch.int32, (cap,))[:rows].cpu().numpy().view(np.uint32).astype(np.uint64)
    assert np.array_equal(gm, pm), "pool metadata"
    pad = pm[:, 0] == 0xFFFFFFFF
    want = np.where(pad, np.uint64(0xFFFFFFFF),
                    (pm[:, 2].astype(np.uint64) * sh.num_shards + pm[:, 0]) * sh.max_tokens_per_shard + pm[:, 1])
    assert np.array_equal(gd, want), "pool scatter targets"
    assert pad.any() and (~pad).any()
    moe.close()


def _sched_words(moe):
    n = 64 + 2 * moe.layout["max_pool_blocks"]
    return moe.region("sched", torch.int32, (n,)).cpu().numpy()


_SCHEDULES = {"fill": mm.FLAG_FILL_IN_GEMM1, "one": mm.FLAG_ONE_GEMM_LAUNCH,
              "fill_one": mm.FLAG_FILL_IN_GEMM1 | mm.FLAG_ONE_GEMM_LAUNCH, "route_all": mm.FLAG_ROUTE_IN_LAUNCH}


@pytest.mark.parametrize("sched", list(_SCHEDULES))
@pytest.mark.parametrize("case", ["bm64_ragged", "bm128_zipf", "bm128_mxfp4", "bm128_waves"])
def test_in_launch_schedules_match_stream_order(case, sched):
    """The schedules that hand rows over inside one launch, per XCD: FILL_IN_GEMM1 (GEMM1's work-groups
    pull the pool and wait on per-block arrival counts), ONE_GEMM_LAUNCH (GEMM2 tiles wait on their
    block's count of finished GEMM1 n tiles), both together, and routing in the same launch behind
    device-wide barriers.  Each gives the same pool, L2 pool and output bits as the stream-ordered
    kernels, reports no status bit and leaves every schedule word at zero."""
    print(f"[case] in-launch schedule {sched} vs stream order {case}", flush=True)
    if case == "bm64_ragged":
        sh = MoEShape("fz64", 5, 333, 1024, 256, 64, 16, 6, 64, local_rank=1, seed=41)
        tps = [333, 0, 101, 7, 250]
    elif case == "bm128_zipf":
        sh = MoEShape("fz128", 4, 700, 2048, 512, 64, 16, 8, 128, local_rank=2, routing="zipf", seed=42)
        tps = [700, 513, 1, 650]
    elif case == "bm128_waves":
        # 64 local experts of about two 128-row blocks each and 8 GEMM1 n tiles per block: every XCD's
        # block range splits into several expert waves when GEMM2 shares the launch.
        sh = MoEShape("fzw", 4, 1024, 512, 1024, 128, 64, 8, 128, local_rank=1, seed=44)
        tps = [1024, 1000, 777, 1024]
    else:
        sh = MoEShape("fz4", 4, 500, 1024, 512, 32, 16, 8, 128, local_rank=1, weight_format="mxfp4", seed=43)
        tps = [500, 211, 0, 480]
        if _SCHEDULES[sched] & (mm.FLAG_FILL_IN_GEMM1 | mm.FLAG_ROUTE_IN_LAUNCH):
            pytest.skip("the in-launch fill is built for FP8 weights only (the config check rejects it)")
    inp = make_inputs(sh, tokens_per_shard=tps)
    runs = []
    for flags in (_SCHEDULES[sched], 0):
        run = Run(sh, inputs=inp, flags=flags, repeat=2)
        assert run.status == 0
        assert not _sched_words(run.moe).any(), "schedule words left non-zero"
        runs.append(run)
    a, b = runs
    n = inputs_np(a)
    check_layout(a, n)
    nb = int(a.region("status", torch.int32, (2,))[1].item())
    rows = slice(0, nb * a.moe.block_m)
    qa, sa = a.l2_host(rows)
    qb, sb = b.l2_host(rows)
    assert np.array_equal(qa, qb) and np.array_equal(sa.view(np.uint32), sb.view(np.uint32)), "L2 pool"
    for ya, yb in zip(a.ys, b.ys):
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), "output bits"
    _whole(a, n)
    for r in runs:
        r.close()


@pytest.mark.parametrize("wf", ["fp8", "mxfp4", "bf16", "fp8_one_launch", "bf16_one_launch"])
def test_graph_capture_replays_match_eager(wf):
    """One forward captured in a HIP graph: three replays on changing input contents, with eager
    forwards and synchronisations between them, each bit-identical to the eager forward on the same
    inputs (the forward records no memset and leaves its workspace counters at zero)."""
    print(f"[case] graph capture and replays, {wf} weights", flush=True)
    flags = 0
    if wf.endswith("one_launch"):     # (the in-launch pull is built for FP8 weights)
        flags = mm.FLAG_ONE_GEMM_LAUNCH | (mm.FLAG_FILL_IN_GEMM1 if wf.startswith("fp8") else 0)
    sh = MoEShape("graph", 4, 96, 512, 256, 32, 8, 4, 64, local_rank=1, weight_format=wf.split("_")[0], seed=61)
    tps = [96, 50, 0, 77]
    a = on_gpu(make_inputs(sh, tokens_per_shard=tps))
    b = on_gpu(make_inputs(sh, seed=62, tokens_per_shard=tps))
    for k in ("w1", "w1_sf", "w2", "w2_sf"):
        b[k] = a[k]
    moe = mm.MegaMoE.from_shape(sh, flags=flags)
    moe(a)                                   # packs a's weights (and MXFP4 exponents) into a
    for k in ("w1_packed", "w2_packed", "w1_sf_packed", "w2_sf_packed"):
        if k in a:
            b[k] = a[k]
    ya, yb = moe(a), moe(b)
    torch.cuda.synchronize()
    dyn = tuple(k for k in ("x", "x_sf", "topk_idx", "topk_weights") if a.get(k) is not None)   # (BF16: no x_sf)
    static = dict(a)
    for k in dyn:
        static[k] = a[k].clone()
    y = torch.zeros_like(ya)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe(static, y=y)
    def same(u, v):                          # rows t >= T_s are never written: compare valid rows
        return all(torch.equal(u[i, :n].view(torch.int16), v[i, :n].view(torch.int16)) for i, n in enumerate(tps))
    for src, want in ((a, ya), (b, yb), (a, ya)):
        for k in dyn:
            static[k].copy_(src[k])
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert same(y, want)
        other = moe(b)                       # eager work between replays
        torch.cuda.synchronize()
        assert same(other, yb)
    assert moe.status() == 0
    del g
    moe.close()


def test_forced_timeout_latches_status_and_recovers():
    """The arrival-counted schedule's bounded waits, forced from the host to give up at once: the
    status word reports TIMEOUT, the launch still completes and zeroes its schedule words, and a
    normal handle on the same inputs is unaffected."""
    print("[case] forced wait timeout", flush=True)
    sh = MoEShape("tmo", 2, 80, 256, 128, 8, 4, 2, 64, seed=71)
    inp = on_gpu(make_inputs(sh))
    for flags in (mm.FLAG_FILL_IN_GEMM1, mm.FLAG_ONE_GEMM_LAUNCH, mm.FLAG_FILL_IN_GEMM1 | mm.FLAG_ONE_GEMM_LAUNCH,
                  mm.FLAG_ROUTE_IN_LAUNCH):
        forced = mm.MegaMoE.from_shape(sh, flags=flags | mm.FLAG_DEBUG_FORCE_TIMEOUT)
        for _ in range(2):
            forced(inp)
            assert forced.status() == mm.STATUS_TIMEOUT
            assert not _sched_words(forced).any()
        forced.close()
        run = Run(sh, inputs=inp, flags=flags)
        assert run.status == 0
        _whole(run, inputs_np(run))
        run.close()


@pytest.mark.parametrize("case", ["max_hidden", "max_intermediate", "max_topk", "max_shards"])
def test_maximum_sizes_whole_layer(case):
    """The configuration maxima: H = 16384 (128 K steps in GEMM1, 16 fill and 32 combine chunks per
    lane), I = 16384 (128 K steps in GEMM2, 64 GEMM1 n tiles), K = 64 (every lane of the combine's
    ballot is a top-k slot, 64 local experts), and S = 64 shards through the whole layer."""
    print(f"[case] maximum sizes {case}", flush=True)
    if case == "max_hidden":
        sh = MoEShape("maxh", 2, 24, 16384, 4096, 2, 1, 1, 64, seed=81)
        tps = [24, 19]
    elif case == "max_intermediate":
        sh = MoEShape("maxi", 2, 24, 4096, 16384, 2, 1, 1, 64, seed=84)
        tps = [24, 11]
    elif case == "max_topk":
        sh = MoEShape("maxk", 2, 30, 256, 128, 128, 64, 64, 64, local_rank=1, seed=82)
        tps = [30, 23]
    else:
        sh = MoEShape("maxs", 64, 12, 256, 128, 16, 8, 2, 64, local_rank=1, seed=83)
        tps = [(5 * i) % 13 for i in range(64)]
    inp = make_inputs(sh, device="cuda", tokens_per_shard=tps)
    run = Run(sh, inputs=inp)
    assert run.status == 0
    n = inputs_np(run)
    check_layout(run, n)
    _whole(run, n)
    run.close()


def test_two_handles_on_two_streams():
    """Two handles with their own workspaces run interleaved forwards on two streams (default
    priority) at once; each result equals the same handle's forward run alone (the library keeps no
    state outside a handle's workspace)."""
    print("[case] two handles, two streams", flush=True)
    sa = MoEShape("sa", 3, 120, 512, 256, 32, 8, 4, 64, local_rank=2, seed=91)
    sb = MoEShape("sb", 2, 200, 768, 384, 16, 4, 2, 128, local_rank=1, seed=92)
    a = on_gpu(make_inputs(sa, tokens_per_shard=[120, 77, 5]))
    b = on_gpu(make_inputs(sb, tokens_per_shard=[200, 131]))
    ma, mb = mm.MegaMoE.from_shape(sa), mm.MegaMoE.from_shape(sb)
    ya, yb = ma(a), mb(b)                     # alone, on the current stream (also packs the weights)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a, outs_b = [], []
    for _ in range(4):
        with torch.cuda.stream(s1):
            outs_a.append(ma(a, stream=s1))
        with torch.cuda.stream(s2):
            outs_b.append(mb(b, stream=s2))
    torch.cuda.synchronize()

    def same(u, v, tps):
        return all(torch.equal(u[i, :n].view(torch.int16), v[i, :n].view(torch.int16)) for i, n in enumerate(tps))
    assert all(same(o, ya, a["tokens_per_shard"]) for o in outs_a)
    assert all(same(o, yb, b["tokens_per_shard"]) for o in outs_b)
    assert ma.status() == 0 and mb.status() == 0
    ma.close()
    mb.close()


@pytest.mark.parametrize("case", ["bm64_shared", "bm128_fill_in_gemm1", "bm128_one_launch", "bm64_one_launch",
                                  "bm128_route_in_launch"])
def test_poisoned_workspace_gives_identical_output(case):
    """With the pool, the L2 pool and the combine planes filled with NaN bytes before every forward,
    the output is bit-identical to a clean run: no stage reads a value this forward did not write.
    With the arrival-counted schedule this also shows that no GEMM1 load overtakes the fill."""
    print(f"[case] poisoned workspace {case}", flush=True)
    if case == "bm64_shared":
        sh = MoEShape("poison64", 3, 140, 512, 256, 32, 8, 4, 64, local_rank=1, num_shared_experts=1, seed=95)
        tps, flags = [140, 61, 0], 0
    elif case == "bm64_one_launch":
        sh = MoEShape("poison64o", 3, 140, 512, 256, 32, 8, 4, 64, local_rank=1, num_shared_experts=1, seed=97)
        tps, flags = [140, 61, 0], mm.FLAG_ONE_GEMM_LAUNCH
    else:
        sh = MoEShape("poison128", 4, 300, 1024, 512, 32, 8, 8, 128, local_rank=3, routing="zipf", seed=96)
        tps, flags = [300, 17, 299, 150], mm.FLAG_FILL_IN_GEMM1
        if case == "bm128_one_launch":
            flags |= mm.FLAG_ONE_GEMM_LAUNCH
        elif case == "bm128_route_in_launch":
            flags = mm.FLAG_ROUTE_IN_LAUNCH
    inp = make_inputs(sh, tokens_per_shard=tps)
    clean = Run(sh, inputs=inp, flags=flags)
    pois = Run(sh, inputs=inp, flags=flags | mm.FLAG_DEBUG_POISON, repeat=2)
    assert clean.status == 0 and pois.status == 0
    for y in pois.ys:
        for i, n in enumerate(tps):
            assert torch.isfinite(y[i, :n].float()).all()
            assert torch.equal(y[i, :n].view(torch.int16), clean.y[i, :n].view(torch.int16))
    _whole(clean, inputs_np(clean))
    # the poison is really there: a routing-only forward leaves the pool and combine bytes at 0xFF
    pois.moe(pois.inp_gpu, stages=mm.STAGE_ROUTE)
    torch.cuda.synchronize()
    for name in ("pool_x", "l2_x", "comb"):
        assert (pois.region(name, torch.uint8, (4096,)) == 255).all(), name
    clean.close()
    pois.close()


@pytest.mark.parametrize("case", ["no_tokens", "all_sentinels", "all_remote"])
def test_empty_forward(case):
    """Nothing routed to this GPU: no valid tokens at all (y untouched), valid tokens whose top-k
    entries are all -1, or whose experts all live on other ranks (y rows zero).  No pool block
    exists, every GEMM work-group exits at once, and the next forward on the same handle is exact."""
    print(f"[case] empty forward {case}", flush=True)
    sh = MoEShape("empty", 3, 64, 256, 128, 32, 8, 4, 64, local_rank=1, seed=97)
    inp = on_gpu(make_inputs(sh))
    if case == "no_tokens":
        inp["tokens_per_shard"] = [0, 0, 0]
    elif case == "all_sentinels":
        inp["topk_idx"].fill_(-1)
    else:
        inp["topk_idx"].remainder_(8)            # experts 0..7: rank 0's, none of rank 1's
    moe = mm.MegaMoE.from_shape(sh)
    y = torch.full((3, 64, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe(inp, y=y)
    torch.cuda.synchronize()
    assert moe.status() == 0
    assert int(moe.region("status", torch.int32, (2,))[1].item()) == 0      # no pool block
    if case == "no_tokens":
        assert torch.isnan(y.float()).all()
    else:
        assert (y.float() == 0).all()
    full = on_gpu(make_inputs(sh))
    full["w1_packed"], full["w2_packed"] = inp["w1_packed"], inp["w2_packed"]
    y2 = moe(full)
    torch.cuda.synchronize()
    assert moe.status() == 0
    n = to_numpy(full)
    ref = oracle.forward(n, sh.num_experts, sh.num_local_experts, sh.local_rank, sh.block_m)
    tol_check(y2.to(torch.float64).cpu().numpy(), ref["y"], case)
    moe.close()


def test_poison_flag_refused_under_graph_capture():
    """DEBUG_POISON fills the workspace with memsets, which a captured HIP graph must not hold: a forward
    with the flag on a capturing stream returns UNSUPPORTED before it records anything."""
    print("[case] poison under capture", flush=True)
    sh = SHAPES["tiny"]
    inp = on_gpu(make_inputs(sh))
    moe = mm.MegaMoE.from_shape(sh, flags=mm.FLAG_DEBUG_POISON)
    moe(inp)                                  # eager: allowed (and packs the weights)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    raised = None
    with torch.cuda.graph(g):
        try:
            moe(inp)
        except mm.MegaMoEError as e:
            raised = e
    assert raised is not None and raised.code == mm.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    y = moe(inp)                              # and the handle still works eagerly afterwards
    torch.cuda.synchronize()
    assert moe.status() == 0 and torch.isfinite(y.float()).all()
    moe.close()
