"""Benchmark of the fused FP8 MoE layer on one MI355X: routed tokens/s and GEMM % of FP8 MFMA peak.

    python bench.py [--gpus 1] [--steps 20] [--warmup 20] [--workload prefill] [--no-cpu-baseline]

One step = one mega_moe_forward (routing, pool fill, GEMM1 + SwiGLU + requant, GEMM2 + scatter,
combine) over one resident batch of seeded synthetic inputs.  The timed region brackets exactly
`steps` forwards with a device synchronisation on both sides; inputs and weights are already in HBM.
The per-stage times (and the roofline's kernel time) come from a second timed pass of `steps` forwards
with HIP events the library records around each stage on the forward's stream; the headline pass has no
events inside it.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense BF16 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E

WORKLOAD_TEXT = {
    "prefill": "prefill-shaped EP=8 share: 8 shards x 4096 tokens, H=7168, I=2048, 32 of 256 experts local, "
               "top-8 uniform, FP8 e4m3 (per-128 activation scales, 128x128 weight scales), BLOCK_M=128",
    "decode": "decode-shaped EP=8 share: 8 shards x 128 tokens, H=7168, I=2048, 32 of 256 experts local, "
              "top-8 uniform, BLOCK_M=64",
    "skewed": "skewed EP=8 share: 8 shards x 2048 tokens, H=7168, I=2048, 32 of 256 experts local, "
              "top-8 Zipf(1.2), BLOCK_M=128",
    "mid": "mid-size MoE: 4 shards x 1024 tokens, H=4096, I=1536, 32 of 128 experts local, top-8, BLOCK_M=128",
    "tiny": "tiny: 1 shard x 64 tokens, H=256, I=512, 8 experts all local, top-2, BLOCK_M=64",
}


def algorithmic(shape, R, N, shared_rows=0):
    """Algorithmic work per forward (valid routed rows only, no padding; the GEMMs also count the shared
    expert's rows when there is one)."""
    H, I, K = shape.hidden, shape.intermediate, shape.topk
    El = shape.num_local_experts + shape.num_shared_experts
    return dict(
        gemm1_flop=4.0 * (R + shared_rows) * H * I,
        gemm2_flop=2.0 * (R + shared_rows) * I * H,
        # route: read every (token, k) expert id, write one table entry per routed pair
        route_bytes=N * K * 8 + R * 4,
        # fill: read the row and its scales, write them and 12 B of metadata, read the table entry
        # (BF16 x BF16: rows of 2H bytes and no scales)
        fill_bytes=R * (4 * H + 12 + 4) if shape.weight_format == "bf16" else R * (2 * H + 2 * (H // 128) * 4 + 12 + 4),
        # combine: read each routed pair's bf16 row, read K ids + weights per token, write the bf16 row
        combine_bytes=R * 2 * H + N * (2 * H + K * 12),
        weight_bytes=(El * 3 * H * I // 2 + El * 3 * H * I // 32) if shape.weight_format == "mxfp4" else
                     El * 3 * H * I * 2 if shape.weight_format == "bf16" else
                     El * 3 * H * I + El * (2 * I // 128) * (H // 128) * 4 + El * (H // 128) * (I // 128) * 4,
    )


def measured_traffic(workload: str):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE record, or None
    when that record was taken on other GEMM source than the one built here (or another workload)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm1_prefill_traffic.json")
    if workload != "prefill" or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "dispatch_fp8_grouped_amd", "csrc", "gemm.hip"), "rb").read()
    if hashlib.sha256(src).hexdigest() != rec.get("gemm_source_sha256"):
        return None
    return rec["hbm_read_bytes"] + rec["hbm_write_bytes"]


def cpu_baseline(shape, inp_gpu, n_experts: int):
    """The CPU oracle, as is, on a bounded sample of the same workload: the whole routing and pool
    fill, then the FFN of the first n_experts local experts.  Rate = their routed rows / seconds."""
    import oracle
    import threadpoolctl
    from inputs import to_numpy
    inp = to_numpy(inp_gpu)
    info = threadpoolctl.threadpool_info()
    threads = max([d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"] or [1])
    t0 = time.perf_counter()
    out = oracle.forward(inp, shape.num_experts, shape.num_local_experts, shape.local_rank, shape.block_m,
                         experts=list(range(n_experts)))
    dt = time.perf_counter() - t0
    rows = int(out["route"].recv_tot[:n_experts].sum())
    return {"value": rows / dt, "unit": "routed tokens/s", "cores": threads, "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{shape.name} workload: routing and pool fill of all {int(out['route'].recv_tot.sum())} "
                      f"routed rows, FFN + combine of local experts 0..{n_experts - 1} ({rows} rows), "
                      f"numpy fp64, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--block-m", type=int, default=None, choices=(64, 128),
                    help="override the workload's BLOCK_M")
    ap.add_argument("--weight-format", default="fp8", choices=("fp8", "mxfp4", "bf16"),
                    help="expert weights: FP8 with 128x128 block scales (the workloads' format), MXFP4 "
                         "(e2m1 with UE8M0 exponents per 32 K; the FP8 x FP4 variant) or BF16 (bf16 tokens "
                         "and weights, no scales; the BF16 x BF16 variant, timed against the BF16 MFMA peak)")
    ap.add_argument("--shared-experts", type=int, default=0, choices=(0, 1),
                    help="add a shared expert on the own shard's tokens (pool segment + combine slot K)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one forward in a HIP graph and time its replays (same kernels, fewer "
                         "host launches)")
    ap.add_argument("--fill-in-gemm1", action="store_true",
                    help="pull the pool rows inside GEMM1's launch, GEMM1 waiting on per-block arrival counts "
                         "(default: the fill is its own kernel, stream-ordered before GEMM1)")
    ap.add_argument("--one-launch", action="store_true",
                    help="run GEMM1 and GEMM2 in one persistent launch, each GEMM2 tile waiting on its pool "
                         "block's count of finished GEMM1 n tiles (default: two stream-ordered launches)")
    ap.add_argument("--route-in-launch", action="store_true",
                    help="routing, the pool pull and both GEMMs in one persistent launch, the routing stages "
                         "separated by device-wide barriers (FP8 weights)")
    ap.add_argument("--cpu-experts", type=int, default=8)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MiB",
                    help="instead of the layer, run a plain elementwise copy of this many MiB five times "
                         "(reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy * 2 ** 20 // 4
        src = torch.randint(0, 2 ** 30, (n,), dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(5):
            torch.bitwise_not(src, out=dst)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / 5
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 6,
                          "kernel": "torch.bitwise_not (elementwise int32)", "ms_per_copy": ms,
                          "copy_GB/s": 2 * n * 4 / (ms * 1e-3) / 1e9}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's expert-parallel share; --gpus {args.gpus} is not supported "
              f"(source ranks are emulated as shards on the one GPU)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dispatch_fp8_grouped_amd as mm
    from inputs import SHAPES, make_inputs

    shape = SHAPES[args.workload]
    if args.shared_experts:
        shape = shape.replace(num_shared_experts=args.shared_experts)
    if args.block_m:
        shape = shape.replace(block_m=args.block_m)
    if args.weight_format != "fp8":
        shape = shape.replace(weight_format=args.weight_format)
    # the recorded HBM counters describe the default kernel configuration only
    default_config = (shape == SHAPES[args.workload] and not args.fill_in_gemm1 and not args.one_launch
                      and not args.route_in_launch)
    torch.cuda.set_device(0)
    inp = make_inputs(shape, device="cuda")
    flags = ((mm.FLAG_FILL_IN_GEMM1 if args.fill_in_gemm1 else 0) | (mm.FLAG_ONE_GEMM_LAUNCH if args.one_launch else 0)
             | (mm.FLAG_ROUTE_IN_LAUNCH if args.route_in_launch else 0))
    moe = mm.MegaMoE.from_shape(shape, flags=flags)
    y = torch.empty((shape.num_shards, shape.max_tokens_per_shard, shape.hidden), dtype=torch.bfloat16,
                    device="cuda")
    stream = torch.cuda.current_stream()
    # Warm-up forwards, then the timed ones after nothing but the synchronisation: host-side reads in
    # between (status, routed-row counts) leave the GPU idle for milliseconds, after which its clock
    # takes ~8 forwards to come back (GEMM1 1.35 -> 1.05 ms in the kernel trace).  Those reads follow
    # the timed steps instead.
    for _ in range(args.warmup):
        moe(inp, y=y)
    N = sum(inp["tokens_per_shard"])

    graph = None
    if args.graph:
        # one forward captured (stage timing off: its events would be frozen into the graph)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            moe(inp, y=y)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    # the headline: exactly `steps` forwards between two events, with no per-stage events inside
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            moe(inp, y=y)
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    # per-stage times (and the roofline's kernel time) from a second timed pass of `steps` eager forwards,
    # with HIP events recorded by the library around each stage on the forward's stream
    mm.mega_moe_set_timing(moe.h, True)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        moe(inp, y=y)
    t1.record(stream)
    torch.cuda.synchronize()
    recv_tot = moe.region("recv_tot", torch.int32, (shape.num_local_experts,)).cpu()
    R = int(recv_tot.sum())
    rows_per_expert = {"max": int(recv_tot.max()), "mean": R / shape.num_local_experts, "min": int(recv_tot.min())}
    stage_ms, nt = mm.mega_moe_stage_times(moe.h, with_count=True)
    mm.mega_moe_set_timing(moe.h, False)
    assert nt == args.steps
    ms_staged = t0.elapsed_time(t1) / args.steps
    ms = ms_total / args.steps
    status = moe.status()
    if status:
        raise SystemExit(f"device status {status:#x} after the timed steps")

    shared_rows = inp["tokens_per_shard"][shape.local_rank] if shape.num_shared_experts else 0
    w = algorithmic(shape, R, N, shared_rows)
    st = dict(zip(mm.STAGE_NAMES, stage_ms))
    fused = st["fill"] == 0.0       # the fill ran inside GEMM1's launch and is timed with it
    one = st["gemm2"] == 0.0        # GEMM2 ran inside GEMM1's launch and is timed with it
    routed_in = st["route"] == 0.0  # so did the routing
    # the dominant kernel: GEMM1's launch (with GEMM2's flops when GEMM2 runs inside it)
    g1_flop = w["gemm1_flop"] + (w["gemm2_flop"] if one else 0.0)
    g1_tflops = g1_flop / (st["gemm1"] * 1e-3) / 1e12
    g2_tflops = 0.0 if one else w["gemm2_flop"] / (st["gemm2"] * 1e-3) / 1e12
    gemm_tflops = (w["gemm1_flop"] + w["gemm2_flop"]) / ((st["gemm1"] + st["gemm2"]) * 1e-3) / 1e12
    bf16 = shape.weight_format == "bf16"
    peak = BF16_PEAK_TFLOPS if bf16 else FP8_PEAK_TFLOPS     # the contraction's own dtype
    gbs = lambda b, t: b / (t * 1e-3) / 1e9  # noqa: E731
    fill_stage = ({"schedule": "inside the gemm1 launch (per-block arrival counts); timed with gemm1"} if fused
                  else {"GB/s": gbs(w["fill_bytes"], st["fill"]),
                        "hbm_frac": gbs(w["fill_bytes"], st["fill"]) / HBM_PEAK_GBS})
    out = {
        "metric": "routed tokens/s of fused MoE layer at 1 GPU; GEMM % of FP8 MFMA peak",
        "value": R / (ms * 1e-3),
        "unit": "routed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 x fp4" if shape.weight_format == "mxfp4" else "bf16" if bf16 else "fp8",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload] + (
                       ", weights MXFP4 (e2m1, UE8M0 per 32 K)" if shape.weight_format == "mxfp4" else
                       ", BF16 x BF16 (bf16 tokens and weights, no scales)" if bf16 else "") + (
                       f", plus a shared expert on shard {shape.local_rank}'s {shared_rows} tokens"
                       if shape.num_shared_experts else ""), "routed_rows": R, "tokens": N,
                   "parallelism": "one GPU's EP share, source ranks emulated as shards",
                   "routed_rows_per_local_expert": rows_per_expert},
        ("gemm_pct_bf16_peak" if bf16 else "gemm_pct_fp8_peak"): 100.0 * gemm_tflops / peak,
        "gemm_tflops": gemm_tflops,
        "roofline": {"bound": "mfma",
                     "kernel": "gemm1 (" + ("routing + " if routed_in else "") + ("pool fill + " if fused else "") +
                               ("gate_up + SwiGLU + bf16" if bf16 else "gate_up + SwiGLU + requant") +
                               (" + down GEMM + scatter, one launch" if one else "") + ")",
                     "achieved": g1_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": g1_tflops / peak,
                     "traffic": measured_traffic(args.workload) if default_config else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic": ("6" if one else "4") + "*R*H*I flop per launch, R = routed rows"},
        "schedule": ("routing inside gemm1's launch, " if routed_in else "") +
                    ("fill inside gemm1" if fused else "stream-ordered fill kernel") +
                    (", gemm2 inside gemm1's launch" if one else "") +
                    (", forward replayed from a HIP graph" if graph is not None else ""),
        "stages_ms": st,
        "ms_per_step_with_stage_events": ms_staged,
        "stages": {
            "route": ({"schedule": "inside the gemm1 launch (device-wide barriers); timed with gemm1"} if routed_in
                      else {"GB/s": gbs(w["route_bytes"], st["route"])}),
            "fill": fill_stage,
            "gemm1": {"TFLOP/s": g1_tflops, "frac": g1_tflops / peak},
            "gemm2": ({"schedule": "inside the gemm1 launch (per-block GEMM1 counts); timed with gemm1"} if one
                      else {"TFLOP/s": g2_tflops, "frac": g2_tflops / peak}),
            "combine": {"GB/s": gbs(w["combine_bytes"], st["combine"]),
                        "hbm_frac": gbs(w["combine_bytes"], st["combine"]) / HBM_PEAK_GBS},
            "weights_stream_GB/s": gbs(w["weight_bytes"], st["gemm1"] + st["gemm2"]),
        },
    }
    moe.close()
    if not args.no_cpu_baseline:
        n_exp = min(args.cpu_experts, shape.num_local_experts)
        out["cpu_baseline"] = cpu_baseline(shape, inp, n_exp)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
