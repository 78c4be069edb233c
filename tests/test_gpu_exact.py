"""GEMM exactness on the GPU: integer FP8 codes with power-of-two scales make every product and every
partial sum exact in fp32, so each grouped GEMM must match the oracle bit for bit whatever its
summation order (the SwiGLU path itself cannot be exact: it uses exp)."""
import numpy as np
import pytest
import torch

import dispatch_fp8_grouped_amd as mm
import oracle
from inputs import MoEShape, make_inputs

from gpu_util import Run, check_layout, inputs_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [
    MoEShape("exact64", 2, 200, 512, 256, 8, 8, 2, 64, seed=31),
    MoEShape("exact128", 1, 300, 7168, 256, 4, 4, 2, 128, seed=32),
], ids=lambda s: s.name)
def test_gemm1_bit_exact(shape):
    print(f"[case] gemm1 exact {shape.name}", flush=True)
    inp = make_inputs(shape, integer_codes=True)
    run = Run(shape, inputs=inp, flags=mm.FLAG_KEEP_GEMM1_OUTPUT)
    n = inputs_np(run)
    rt, off = check_layout(run, n)
    px, psf, pm, _ = oracle.fill_pool(n["x"], n["x_sf"], rt, shape.block_m, shape.topk)
    cap = run.moe.layout["max_pool_blocks"] * run.moe.block_m
    g1 = run.region("gemm1_out", torch.float32, (cap, 2 * shape.intermediate))
    for le in range(shape.num_local_experts):
        base, nrows = int(off[le]) * shape.block_m, int(rt.recv_tot[le])
        if nrows == 0:
            continue
        a = oracle.dequant_rows(px[base:base + nrows], psf[base:base + nrows])
        w = oracle.dequant_blocks(n["w1"][le], n["w1_sf"][le])
        want = (a @ w.T).astype(np.float32)
        got = g1[base:base + nrows].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"expert {le}"
    run.close()


@pytest.mark.parametrize("shape", [
    MoEShape("exact2_64", 2, 150, 768, 384, 8, 4, 2, 64, seed=33),
    MoEShape("exact2_128", 2, 260, 1024, 2048, 4, 4, 2, 128, seed=34),
], ids=lambda s: s.name)
def test_gemm2_bit_exact_on_placed_activations(shape):
    """Run route+fill+GEMM1, overwrite the L2 pool with integer codes and 2^-4 scales, run GEMM2 alone."""
    print(f"[case] gemm2 exact {shape.name}", flush=True)
    inp = make_inputs(shape, integer_codes=True)
    run = Run(shape, inputs=inp)
    n = inputs_np(run)
    rt, off = check_layout(run, n)
    _, _, pm, _ = oracle.fill_pool(n["x"], n["x_sf"], rt, shape.block_m, shape.topk)
    P = int(off[-1]) * shape.block_m
    I = shape.intermediate
    rng = np.random.default_rng(5)
    vals = torch.arange(-8, 9, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    l2 = vals[rng.integers(0, 17, (P, I))]
    cap = run.moe.layout["max_pool_blocks"] * run.moe.block_m
    # the L2 pool is tiled: [blocks][I/128][4][BM][32]
    nb = P // shape.block_m
    tiled = l2.reshape(nb, shape.block_m, I // 128, 4, 32).transpose(0, 2, 3, 1, 4)
    run.region("l2_x", torch.uint8, (cap * I,))[:P * I] = torch.from_numpy(np.ascontiguousarray(tiled).reshape(-1)).cuda()
    run.region("l2_sf", torch.float32, (cap, I // 128))[:P] = 2.0 ** -4
    g = run.inp_gpu
    mm.mega_moe_forward_stages(run.moe.h, mm.STAGE_GEMM2, g["tokens_per_shard"], None, None, None, None,
                               None, None, g["w2_packed"], g["w2_sf"], None)
    torch.cuda.synchronize()
    assert run.moe.status() == 0
    for le in range(shape.num_local_experts):
        base, nrows = int(off[le]) * shape.block_m, int(rt.recv_tot[le])
        if nrows == 0:
            continue
        h = oracle.e4m3fn_decode(l2[base:base + nrows]) * 2.0 ** -4
        w = oracle.dequant_blocks(n["w2"][le], n["w2_sf"][le])
        want = oracle.bf16_bits(oracle.bf16_round(h @ w.T))
        for j in range(nrows):
            s, t, k = (int(v) for v in pm[base + j])
            got = oracle.bf16_bits(run.comb_row(k, s, t))
            assert np.array_equal(got, want[j]), (le, j)
    run.close()


@pytest.mark.parametrize("shape", [
    MoEShape("exact_fp4_64", 2, 130, 512, 256, 8, 4, 2, 64, seed=35, weight_format="mxfp4"),
    MoEShape("exact_fp4_128", 1, 300, 7168, 256, 4, 4, 2, 128, seed=36, weight_format="mxfp4"),
], ids=lambda s: s.name)
def test_gemm1_bit_exact_mxfp4_weights(shape):
    """FP8 x FP4: integer FP8 codes times e2m1 values (multiples of 1/2 up to 6) with one power-of-two
    exponent and power-of-two token scales: every product and partial sum is exact in fp32, so GEMM1
    matches the oracle bit for bit whatever the lane order of the scaled MFMA's split K."""
    print(f"[case] gemm1 exact mxfp4 {shape.name}", flush=True)
    inp = make_inputs(shape, integer_codes=True)
    run = Run(shape, inputs=inp, flags=mm.FLAG_KEEP_GEMM1_OUTPUT)
    n = inputs_np(run)
    rt, off = check_layout(run, n)
    px, psf, pm, _ = oracle.fill_pool(n["x"], n["x_sf"], rt, shape.block_m, shape.topk)
    cap = run.moe.layout["max_pool_blocks"] * run.moe.block_m
    g1 = run.region("gemm1_out", torch.float32, (cap, 2 * shape.intermediate))
    for le in range(shape.num_local_experts):
        base, nrows = int(off[le]) * shape.block_m, int(rt.recv_tot[le])
        if nrows == 0:
            continue
        a = oracle.dequant_rows(px[base:base + nrows], psf[base:base + nrows])
        w = oracle.dequant_weight(n["w1"][le], n["w1_sf"][le])
        want = (a @ w.T).astype(np.float32)
        got = g1[base:base + nrows].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"expert {le}"
    run.close()


@pytest.mark.parametrize("shape", [
    MoEShape("exact2_fp4_64", 2, 150, 768, 384, 8, 4, 2, 64, seed=37, weight_format="mxfp4"),
    MoEShape("exact2_fp4_128", 2, 260, 1024, 2048, 4, 4, 2, 128, seed=38, weight_format="mxfp4"),
], ids=lambda s: s.name)
def test_gemm2_bit_exact_mxfp4_weights_on_placed_activations(shape):
    """FP8 x FP4 GEMM2 on integer L2 codes with 2^-4 scales and integer-coded MXFP4 weights: bit-exact bf16
    rows against the oracle."""
    print(f"[case] gemm2 exact mxfp4 {shape.name}", flush=True)
    inp = make_inputs(shape, integer_codes=True)
    run = Run(shape, inputs=inp)
    n = inputs_np(run)
    rt, off = check_layout(run, n)
    _, _, pm, _ = oracle.fill_pool(n["x"], n["x_sf"], rt, shape.block_m, shape.topk)
    P = int(off[-1]) * shape.block_m
    I = shape.intermediate
    rng = np.random.default_rng(6)
    vals = torch.arange(-8, 9, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    l2 = vals[rng.integers(0, 17, (P, I))]
    cap = run.moe.layout["max_pool_blocks"] * run.moe.block_m
    nb = P // shape.block_m
    tiled = l2.reshape(nb, shape.block_m, I // 128, 4, 32).transpose(0, 2, 3, 1, 4)
    run.region("l2_x", torch.uint8, (cap * I,))[:P * I] = torch.from_numpy(np.ascontiguousarray(tiled).reshape(-1)).cuda()
    run.region("l2_sf", torch.float32, (cap, I // 128))[:P] = 2.0 ** -4
    g = run.inp_gpu
    mm.mega_moe_forward_stages(run.moe.h, mm.STAGE_GEMM2, g["tokens_per_shard"], None, None, None, None,
                               None, None, g["w2_packed"], g["w2_sf_packed"], None)
    torch.cuda.synchronize()
    assert run.moe.status() == 0
    for le in range(shape.num_local_experts):
        base, nrows = int(off[le]) * shape.block_m, int(rt.recv_tot[le])
        if nrows == 0:
            continue
        h = oracle.e4m3fn_decode(l2[base:base + nrows]) * 2.0 ** -4
        w = oracle.dequant_weight(n["w2"][le], n["w2_sf"][le])
        want = oracle.bf16_bits(oracle.bf16_round(h @ w.T))
        for j in range(nrows):
            s, t, k = (int(v) for v in pm[base + j])
            got = oracle.bf16_bits(run.comb_row(k, s, t))
            assert np.array_equal(got, want[j]), (le, j)
    run.close()
