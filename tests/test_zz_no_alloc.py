"""The entry point for callers that cannot allocate (mega_moe_forward_noalloc, static per-GPU scratch):
through the C ABI its output must equal mega_moe_forward's bit for bit, on two calls in a row, the second
with a smaller input, with the status reported through the caller's device word."""
import ctypes

import numpy as np
import pytest
import torch

import dispatch_fp8_grouped_amd as mm
from inputs import SHAPES, MoEShape, make_inputs

pytestmark = pytest.mark.gpu


def _noalloc(shape, inp):
    moe = mm.MegaMoE.from_shape(shape)
    y_ref = moe(inp)                                   # packs the weights into inp
    torch.cuda.synchronize()
    assert moe.status() == 0
    moe.close()
    S, T, H = shape.num_shards, shape.max_tokens_per_shard, shape.hidden
    y = torch.full((S, T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    status = torch.full((1,), 0x5A5A, dtype=torch.int32, device="cuda")
    cfg = moe.cfg
    lib = mm.lib()
    tps = (ctypes.c_int32 * S)(*inp["tokens_per_shard"])
    p = lambda t: ctypes.c_void_p(None if t is None else t.data_ptr())   # noqa: E731
    rc = lib.mega_moe_forward_noalloc(ctypes.byref(cfg), tps, p(inp["x"]), p(inp.get("x_sf")), p(inp["topk_idx"]),
                                      p(inp["topk_weights"]), p(inp["w1_packed"]), p(inp.get("w1_sf")),
                                      p(inp["w2_packed"]), p(inp.get("w2_sf")), p(y), None, p(status),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == 0, mm.mega_moe_strerror(rc)
    assert int(status.item()) == 0
    valid = [(s, t) for s in range(S) for t in range(inp["tokens_per_shard"][s])]
    got = y.view(torch.int16).cpu().numpy()
    want = y_ref.view(torch.int16).cpu().numpy()
    for s in range(S):
        n = inp["tokens_per_shard"][s]
        assert np.array_equal(got[s, :n], want[s, :n]), f"shard {s}"
        assert torch.isnan(y[s, n:].float()).all(), f"shard {s}: rows past T_s written"
    return len(valid)


def test_noalloc_forward_matches_forward_on_two_calls():
    print("[case] noalloc decode then a smaller layer", flush=True)
    # first call: the decode-shaped share (205 MiB of workspace, within the 256 MiB scratch)
    dec = SHAPES["decode"]
    n1 = _noalloc(dec, {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
                        for k, v in make_inputs(dec, device="cuda").items()})
    # second call: a smaller layer with ragged shards and a shared expert, on the same scratch
    small = MoEShape("noalloc_small", 3, 96, 512, 256, 16, 8, 4, 64, seed=51, num_shared_experts=1)
    inp = make_inputs(small, device="cuda", tokens_per_shard=[96, 17, 0])
    n2 = _noalloc(small, inp)
    assert n1 > n2 > 0


def test_noalloc_forward_matches_forward_bf16():
    """The same entry point with BF16 x BF16 weights (no scale pointers)."""
    print("[case] noalloc bf16", flush=True)
    sh = MoEShape("noalloc_bf16", 3, 96, 512, 256, 16, 8, 4, 64, seed=52, weight_format="bf16")
    inp = make_inputs(sh, device="cuda", tokens_per_shard=[96, 40, 7])
    assert _noalloc(sh, inp) > 0
