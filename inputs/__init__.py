"""Seeded synthetic inputs for the fused FP8 MoE layer (one GPU's expert-parallel share).

This module is shared by the CPU oracle's tests, the GPU parity tests and the benchmark.
It holds shapes and random draws only: none of the layer's arithmetic (routing, pooling,
GEMMs, SwiGLU, requantisation, combine) lives here.  Inputs are quantised to FP8 e4m3fn
with torch's own dtype cast, which plays the role of the upstream model that hands the
layer FP8 activations and block-scaled FP8 weights.

Input recipe (the workload descriptions the layer is quoted on):
  * x ~ N(0, 1) of shape [S, T, H], quantised per token and per 128 columns:
    scale = amax / 448, codes = e4m3fn(x / scale).
  * W1 ~ N(0, 0.02^2) of shape [E_l + n_shared, 2I, H] (rows 0..I-1 gate, I..2I-1 up) and
    W2 ~ N(0, 0.02^2) of shape [E_l + n_shared, H, I], quantised per 128x128 block the same
    way; with a shared expert (n_shared = 1) its weights are the last expert.
  * topk_idx: K distinct experts per token.  "uniform": a uniformly random K-subset.
    "zipf": expert at rank j of a seeded permutation has weight j^-alpha and K experts are
    drawn without replacement (Gumbel top-k, i.e. successive draws proportional to weight).
  * topk_weights = softmax of N(0, 1) logits over the K chosen experts.
Draw order is fixed: x, W1, W2, routing keys, logits.
"""
from __future__ import annotations

import dataclasses
import hashlib
from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import torch

FP8_MAX = 448.0


@dataclass(frozen=True)
class MoEShape:
    """Shape of one GPU's share of an expert-parallel MoE layer.

    Source ranks are emulated as ``num_shards`` token shards resident on the one GPU.
    This GPU owns global experts [local_rank*E_l, (local_rank+1)*E_l).
    """
    name: str
    num_shards: int            # S
    max_tokens_per_shard: int  # T_max
    hidden: int                # H
    intermediate: int          # I
    num_experts: int           # E (global)
    num_local_experts: int     # E_l
    topk: int                  # K
    block_m: int               # BLOCK_M of the expert pool
    local_rank: int = 0
    routing: str = "uniform"   # "uniform" | "zipf"
    num_shared_experts: int = 0  # 0 or 1: a shared expert on shard local_rank's own tokens
    weight_format: str = "fp8"   # "fp8" (128x128 block scales) | "mxfp4" (e2m1, UE8M0 per 32 along K) | "bf16"
    zipf_alpha: float = 1.2
    seed: int = 0

    def replace(self, **kw) -> "MoEShape":
        return dataclasses.replace(self, **kw)


# The five workloads.  Seeds: tiny 0, decode 1, prefill 2, skewed 3, mid 4.
SHAPES: Dict[str, MoEShape] = {
    "tiny": MoEShape("tiny", 1, 64, 256, 512, 8, 8, 2, 64, seed=0),
    "decode": MoEShape("decode", 8, 128, 7168, 2048, 256, 32, 8, 64, seed=1),
    "prefill": MoEShape("prefill", 8, 4096, 7168, 2048, 256, 32, 8, 128, seed=2),
    "skewed": MoEShape("skewed", 8, 2048, 7168, 2048, 256, 32, 8, 128,
                       routing="zipf", zipf_alpha=1.2, seed=3),
    "mid": MoEShape("mid", 4, 1024, 4096, 1536, 128, 32, 8, 128, seed=4),
}


def _quant_rows_per128(x: torch.Tensor):
    """[..., C] float32 -> (uint8 e4m3fn codes [..., C], float32 scales [..., C/128])."""
    *lead, c = x.shape
    xb = x.reshape(*lead, c // 128, 128)
    amax = xb.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (xb / scale.unsqueeze(-1)).to(torch.float8_e4m3fn)
    return q.reshape(*lead, c).view(torch.uint8), scale.to(torch.float32)


def _quant_block128(w: torch.Tensor):
    """[N, C] float32 -> (uint8 codes [N, C], float32 scales [N/128, C/128])."""
    n, c = w.shape
    wb = w.reshape(n // 128, 128, c // 128, 128)
    amax = wb.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (wb / scale[:, None, :, None]).to(torch.float8_e4m3fn)
    return q.reshape(n, c).view(torch.uint8), scale.to(torch.float32)


_E2M1_MAGS = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _quant_mxfp4(w: torch.Tensor):
    """[N, C] float32 -> (uint8 [N, C/2] two e2m1 codes per byte, low nibble = lower column;
    uint8 [N, C/32] UE8M0 exponents).  Per 32 columns: exponent = floor(log2(amax)) - 2 (6 = 1.5 * 2^2 is
    the largest e2m1 magnitude), clamped to the UE8M0 range; each value goes to the nearest e2m1
    magnitude of w / 2^exponent, saturating at 6.  This plays the upstream model that hands the layer
    MXFP4 weights."""
    n, c = w.shape
    wb = w.reshape(n, c // 32, 32)
    amax = wb.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp_min(2.0 ** -126))) - 2,
                    torch.full_like(amax, -127.0)).clamp(-127, 127)
    v = (wb / torch.pow(2.0, e).unsqueeze(-1)).abs().clamp(max=6.0)
    mags = torch.tensor(_E2M1_MAGS, device=w.device)
    code = (v.unsqueeze(-1) - mags).abs().argmin(dim=-1).to(torch.uint8)
    code = code | torch.where(wb < 0, 8, 0).to(torch.uint8)
    code = code.reshape(n, c)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).to(torch.uint8)
    return packed, (e + 127).to(torch.uint8).reshape(n, c // 32)


def _route(shape: MoEShape, gen: torch.Generator, device) -> torch.Tensor:
    S, T, E, K = shape.num_shards, shape.max_tokens_per_shard, shape.num_experts, shape.topk
    if shape.routing == "uniform":
        keys = torch.rand((S, T, E), generator=gen, device=device)
    elif shape.routing == "zipf":
        perm = torch.randperm(E, generator=gen, device=device)
        rank_w = torch.arange(1, E + 1, device=device, dtype=torch.float64).pow(-shape.zipf_alpha)
        logp = torch.empty(E, dtype=torch.float64, device=device)
        logp[perm] = rank_w.log()
        u = torch.rand((S, T, E), generator=gen, device=device, dtype=torch.float64)
        u = u.clamp_min(1e-300)
        keys = logp - torch.log(-torch.log(u))
    else:
        raise ValueError(f"unknown routing {shape.routing!r}")
    return keys.topk(K, dim=-1).indices.to(torch.int64)


def make_inputs(shape: MoEShape, device="cpu", seed: Optional[int] = None,
                tokens_per_shard: Optional[Sequence[int]] = None,
                integer_codes: bool = False) -> Dict[str, object]:
    """Draw one seeded input set.  Returns a dict of tensors on ``device``:

    x [S,T,H] u8 (e4m3fn codes), x_sf [S,T,H/128] f32, topk_idx [S,T,K] i64,
    topk_weights [S,T,K] f32, w1 [E_w,2I,H] u8, w1_sf [E_w,2I/128,H/128] f32,
    w2 [E_w,H,I] u8, w2_sf [E_w,H/128,I/128] f32 (E_w = E_l + num_shared_experts), and
    tokens_per_shard (list of int).

    weight_format "mxfp4": w1 [E_w,2I,H/2] and w2 [E_w,H,I/2] hold two e2m1 codes per byte, and w1_sf
    [E_w,2I,H/32] / w2_sf [E_w,H,I/32] hold UE8M0 exponents (uint8) of each 32 values along K.

    weight_format "bf16" (BF16 x BF16): x [S,T,H], w1 [E_w,2I,H] and w2 [E_w,H,I] are bfloat16 and there
    are no scales (x_sf, w1_sf and w2_sf are None).

    integer_codes=True draws every FP8 code from the integers -8..8 and every scale as
    one shared power of two (2^-4 for activations, 2^-6 for weights), so that every
    product and every partial sum of the GEMMs is exact in fp32.  With weight_format "mxfp4"
    the weights are then any e2m1 codes with one shared UE8M0 exponent (2^-3): their values are
    multiples of 1/2 up to 6, so the products and sums stay exact too.
    """
    S, T, H, I = shape.num_shards, shape.max_tokens_per_shard, shape.hidden, shape.intermediate
    El, K = shape.num_local_experts + shape.num_shared_experts, shape.topk
    if H % 128 or I % 128:
        raise ValueError("hidden and intermediate must be multiples of 128")
    gen = torch.Generator(device=device)
    gen.manual_seed(shape.seed if seed is None else seed)

    def ints(shape_):
        v = torch.randint(-8, 9, shape_, generator=gen, device=device).to(torch.float32)
        return v.to(torch.float8_e4m3fn).view(torch.uint8)

    def fp4_codes(shape_):
        # any e2m1 codes (values 0, +-0.5, ..., +-6), two per byte, the low nibble first
        lo = torch.randint(0, 16, shape_, generator=gen, device=device)
        hi = torch.randint(0, 16, shape_, generator=gen, device=device)
        return (lo | (hi << 4)).to(torch.uint8)

    def bf16_ints(shape_):
        return torch.randint(-8, 9, shape_, generator=gen, device=device).to(torch.bfloat16)

    if shape.weight_format == "bf16":
        # integer_codes: integers -8..8, exact in bf16, whose GEMM sums stay exact in fp32
        if integer_codes:
            x, w1, w2 = bf16_ints((S, T, H)), bf16_ints((El, 2 * I, H)), bf16_ints((El, H, I))
        else:
            x = torch.randn((S, T, H), generator=gen, device=device).to(torch.bfloat16)
            w1 = (torch.randn((El, 2 * I, H), generator=gen, device=device) * 0.02).to(torch.bfloat16)
            w2 = (torch.randn((El, H, I), generator=gen, device=device) * 0.02).to(torch.bfloat16)
        x_sf = w1_sf = w2_sf = None
    elif integer_codes and shape.weight_format == "mxfp4":
        x = ints((S, T, H))
        x_sf = torch.full((S, T, H // 128), 2.0 ** -4, device=device)
        w1 = fp4_codes((El, 2 * I, H // 2))
        w1_sf = torch.full((El, 2 * I, H // 32), 127 - 3, dtype=torch.uint8, device=device)   # 2^-3
        w2 = fp4_codes((El, H, I // 2))
        w2_sf = torch.full((El, H, I // 32), 127 - 3, dtype=torch.uint8, device=device)
    elif integer_codes:
        x = ints((S, T, H))
        x_sf = torch.full((S, T, H // 128), 2.0 ** -4, device=device)
        w1 = ints((El, 2 * I, H))
        w1_sf = torch.full((El, 2 * I // 128, H // 128), 2.0 ** -6, device=device)
        w2 = ints((El, H, I))
        w2_sf = torch.full((El, H // 128, I // 128), 2.0 ** -6, device=device)
    elif shape.weight_format == "mxfp4":
        x, x_sf = _quant_rows_per128(torch.randn((S, T, H), generator=gen, device=device))
        w1 = torch.empty((El, 2 * I, H // 2), dtype=torch.uint8, device=device)
        w1_sf = torch.empty((El, 2 * I, H // 32), dtype=torch.uint8, device=device)
        for e in range(El):
            w = torch.randn((2 * I, H), generator=gen, device=device) * 0.02
            w1[e], w1_sf[e] = _quant_mxfp4(w)
        w2 = torch.empty((El, H, I // 2), dtype=torch.uint8, device=device)
        w2_sf = torch.empty((El, H, I // 32), dtype=torch.uint8, device=device)
        for e in range(El):
            w = torch.randn((H, I), generator=gen, device=device) * 0.02
            w2[e], w2_sf[e] = _quant_mxfp4(w)
    else:
        x, x_sf = _quant_rows_per128(torch.randn((S, T, H), generator=gen, device=device))
        w1 = torch.empty((El, 2 * I, H), dtype=torch.uint8, device=device)
        w1_sf = torch.empty((El, 2 * I // 128, H // 128), dtype=torch.float32, device=device)
        for e in range(El):
            w = torch.randn((2 * I, H), generator=gen, device=device) * 0.02
            w1[e], w1_sf[e] = _quant_block128(w)
        w2 = torch.empty((El, H, I), dtype=torch.uint8, device=device)
        w2_sf = torch.empty((El, H // 128, I // 128), dtype=torch.float32, device=device)
        for e in range(El):
            w = torch.randn((H, I), generator=gen, device=device) * 0.02
            w2[e], w2_sf[e] = _quant_block128(w)
    topk_idx = _route(shape, gen, device)
    logits = torch.randn((S, T, K), generator=gen, device=device)
    topk_weights = torch.softmax(logits, dim=-1).to(torch.float32)
    if tokens_per_shard is None:
        tokens_per_shard = [T] * S
    tokens_per_shard = [int(t) for t in tokens_per_shard]
    if len(tokens_per_shard) != S or any(t < 0 or t > T for t in tokens_per_shard):
        raise ValueError("tokens_per_shard must hold S values in [0, T_max]")
    return dict(x=x, x_sf=x_sf, topk_idx=topk_idx, topk_weights=topk_weights,
                w1=w1, w1_sf=w1_sf, w2=w2, w2_sf=w2_sf, tokens_per_shard=tokens_per_shard)


def to_numpy(inputs: Dict[str, object]) -> Dict[str, object]:
    """Host (numpy) copies of an input set, for the CPU oracle."""
    out = {}
    for k, v in inputs.items():
        if isinstance(v, torch.Tensor):
            v = v.detach().cpu()
            out[k] = (v.float() if v.dtype == torch.bfloat16 else v).numpy()    # bf16 values exactly
        else:
            out[k] = v
    return out


def digest(inputs: Dict[str, object]) -> str:
    """Short content hash of an input set (recorded next to results)."""
    h = hashlib.sha256()
    for k in sorted(inputs):
        v = inputs[k]
        if isinstance(v, torch.Tensor):
            h.update(k.encode())
            h.update(v.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())
        else:
            h.update(repr((k, v)).encode())
    return h.hexdigest()[:16]
