"""Pins of the MXFP4 weight decoding (oracle/fp4.py) against what fixes it independently: the e2m1
bit layout written out element by element, torch's own UE8M0 dtype, brute-force nibble packing, and
a block-scaled matrix product through torch routines."""
import numpy as np
import torch

from oracle.fp4 import MX_BLOCK, dequant_mx, e2m1_decode, e8m0_decode, unpack_fp4


def test_e2m1_all_codes():
    # sign, exponent (bias 1) and mantissa fields of every code, evaluated one by one
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        want = (-1.0) ** s * (m / 2 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))
        got = e2m1_decode(np.array([c]))[0]
        assert got == want and np.signbit(got) == bool(s), c
    mags = e2m1_decode(np.arange(8))
    assert mags.tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert e2m1_decode(np.array([0x17]))[0] == 6.0          # bits above the nibble are ignored


def test_e8m0_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = e8m0_decode(codes.numpy())
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and np.isnan(got[255])


def test_unpack_low_nibble_first():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    packed = np.zeros((5, 32), dtype=np.uint8)
    for r in range(5):
        for j in range(32):
            packed[r, j] = codes[r, 2 * j] | (codes[r, 2 * j + 1] << 4)
    assert np.array_equal(unpack_fp4(packed, 64), codes)


def test_dequant_mx_blocks_and_product():
    rng = np.random.default_rng(1)
    N, K = 8, 128
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(120, 131, (N, K // MX_BLOCK)).astype(np.uint8)
    w = dequant_mx(packed, scales)
    # element by element: code value times 2^(scale of its 32-block - 127)
    for n in range(N):
        for k in range(0, K, 7):
            assert w[n, k] == e2m1_decode(codes[n, k]) * 2.0 ** (int(scales[n, k // MX_BLOCK]) - 127)
    # a product with the dequantised weight equals torch's on the same block-scaled operands
    x = rng.standard_normal((3, K))
    tw = torch.tensor(e2m1_decode(codes)) * torch.pow(2.0, torch.tensor(scales, dtype=torch.float64) - 127).repeat_interleave(MX_BLOCK, 1)
    assert np.allclose(x @ w.T, (torch.tensor(x) @ tw.T).numpy(), rtol=1e-12, atol=0)


def _torch_mx(packed, sf):
    """MXFP4 -> float64 with torch ops only: the e2m1 fields of each nibble and 2^(e - 127)."""
    p = torch.from_numpy(packed).to(torch.int64)
    codes = torch.stack([p & 0xF, p >> 4], dim=-1).reshape(p.shape[0], -1)
    s, e, m = (codes >> 3) & 1, (codes >> 1) & 3, (codes & 1).to(torch.float64)
    mag = torch.where(e == 0, 0.5 * m, torch.pow(2.0, (e - 1).to(torch.float64)) * (1 + 0.5 * m))
    val = torch.where(s == 1, -mag, mag)
    return val * torch.pow(2.0, torch.from_numpy(sf).to(torch.float64) - 127).repeat_interleave(32, 1)


def test_layer_with_mxfp4_weights_textbook():
    """S=1, E_l=1, K=1, w=1 with MXFP4 weights: y = bf16(W2 requant(silu(W1g x) * W1u x)) through
    torch routines on independently decoded weights."""
    from inputs import MoEShape, make_inputs, to_numpy
    import oracle
    sh = MoEShape("mx", 1, 40, 256, 128, 1, 1, 1, 64, weight_format="mxfp4", seed=11)
    inp = to_numpy(make_inputs(sh))
    assert inp["w1"].shape == (1, 256, 128) and inp["w1_sf"].shape == (1, 256, 8) and inp["w1_sf"].dtype == np.uint8
    inp["topk_idx"][:] = 0
    inp["topk_weights"][:] = 1.0
    out = oracle.forward(inp, 1, 1, 0, 64)
    f8 = torch.float8_e4m3fn
    x = torch.from_numpy(inp["x"][0]).view(f8).to(torch.float64) * \
        torch.from_numpy(inp["x_sf"][0]).to(torch.float64).repeat_interleave(128, -1)
    W1, W2 = _torch_mx(inp["w1"][0], inp["w1_sf"][0]), _torch_mx(inp["w2"][0], inp["w2_sf"][0])
    g = x @ W1.T
    h = (torch.nn.functional.silu(g[:, :128]) * g[:, 128:]).to(torch.float32)
    hb = h.reshape(40, 1, 128)
    sc = torch.clamp(hb.abs().amax(-1), min=1e-4) / 448.0
    hq = ((hb / sc.unsqueeze(-1)).to(f8).to(torch.float64) * sc.to(torch.float64).unsqueeze(-1)).reshape(40, 128)
    want = (hq @ W2.T).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.all(np.abs(out["y"][0] - want) <= np.abs(want) * 2.0 ** -7 + 1e-30)
    # the generated weights keep the N(0, 0.02) scale of the recipe
    assert 0.017 < float(W1.std()) < 0.023 and 0.017 < float(W2.std()) < 0.023
