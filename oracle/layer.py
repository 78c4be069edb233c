"""The layer, step by step, on the CPU.  Test infrastructure only.

Notation: S source shards (emulated ranks), T_max tokens per shard (T_s of them valid in
shard s), E global experts, E_l local experts, r = local rank, K = top-k, H hidden,
I intermediate, BM = BLOCK_M.  This GPU owns global experts [r*E_l, (r+1)*E_l): the rank
of expert e is e // E_l and its local number e % E_l ("Mega-MoE kernel code walkthrough",
section 2).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .fp4 import dequant_mx
from .fp8 import e4m3fn_decode, e4m3fn_encode, bf16_round, E4M3_MAX

META_PAD = 0xFFFFFFFF


# ----------------------------------------------------------------------------- routing
@dataclass
class RouteResult:
    send: np.ndarray        # [S, E] int64: pairs of shard s routed to global expert e
    recv: np.ndarray        # [E_l, S] int64: pairs of shard s for local expert le
    recv_tot: np.ndarray    # [E_l] int64
    table: np.ndarray       # [E_l, S, T_max] int64: t*K+k in slot order, -1 beyond recv
    bad_expert: bool        # some entry had expert id >= E (entry skipped)
    slot_overflow: bool     # some (le, s) needed more than T_max slots (extra entries dropped)


def route(topk_idx: np.ndarray, tokens_per_shard: Sequence[int], num_experts: int,
          num_local_experts: int, local_rank: int) -> RouteResult:
    """Counts and the [local_expert][source_rank][slot] index table.

    Each valid entry (t < T_s, expert id >= 0) of shard s counts once towards send[s][e]
    ("Mega-MoE kernel code walkthrough", 4.1: entries with a negative expert id are
    skipped; 4.2: per-expert send counts).  An entry whose expert is local is written to
    table[le][s][slot] as the flat index t*K+k ("Mega-MoE notes, part 2", 1.1: the slot is
    numbered independently per (source rank, expert); 1.3: the pull reads the same
    coordinates).  Slot order: ascending t*K+k (the pages claim slots with atomics, so
    their order is unspecified; this is the deterministic reading, and it contains the
    walkthrough's "earlier contributor gets the lower slots" rule of 4.2).  The receiving
    side's count is recv[le][s] = send[s][r*E_l + le] (4.4, the count broadcast).
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    S, T_max, K = idx.shape
    E, El, r = num_experts, num_local_experts, local_rank
    lo = r * El
    send = np.zeros((S, E), dtype=np.int64)
    table = np.full((El, S, T_max), -1, dtype=np.int64)
    recv = np.zeros((El, S), dtype=np.int64)
    bad = False
    overflow = False
    for s in range(S):
        n = int(tokens_per_shard[s]) * K
        e = idx[s].reshape(-1)[:n]
        flat = np.arange(n, dtype=np.int64)            # t*K + k
        if np.any(e >= E):
            bad = True
        ok = (e >= 0) & (e < E)
        send[s] = np.bincount(e[ok], minlength=E)
        loc = ok & (e >= lo) & (e < lo + El)
        le = e[loc] - lo
        f = flat[loc]
        # counting sort by local expert, stable in t*K+k
        order = np.argsort(le, kind="stable")
        le_sorted, f_sorted = le[order], f[order]
        counts = np.bincount(le_sorted, minlength=El)
        start = np.concatenate([[0], np.cumsum(counts)[:-1]])
        slot = np.arange(len(le_sorted)) - start[le_sorted]
        keep = slot < T_max
        if not np.all(keep):
            overflow = True
        table[le_sorted[keep], s, slot[keep]] = f_sorted[keep]
        recv[:, s] = np.minimum(counts, T_max)
    # recv[le][s] equals send[s][lo+le] unless slots overflowed
    return RouteResult(send=send, recv=recv, recv_tot=recv.sum(axis=1), table=table,
                       bad_expert=bad, slot_overflow=overflow)


def pool_offsets(recv_tot: Sequence[int], block_m: int) -> np.ndarray:
    """off[le] = sum over earlier experts of ceil(recv_tot / BM) (E_l+1 entries).

    "Mega-MoE notes, part 2", 2.4: the received tokens form one expert-major queue and the
    pool offset of an expert counts the M-blocks taken by the experts before it;
    "Dispatch/Combine ... comparison", 5.3: each expert's rows are padded to BLOCK_M.
    """
    off = [0]
    for c in recv_tot:
        off.append(off[-1] + (int(c) + block_m - 1) // block_m)
    return np.array(off, dtype=np.int64)


# ----------------------------------------------------------------------------- round-robin
def rr_inverse(counts: Sequence[int], j: int) -> Tuple[int, int]:
    """Position j inside one expert's rows -> (source shard, slot), by min-peeling.

    "DeepGEMM Mega MoE symmetric memory deep analysis", 7.5 and "Mega-MoE notes, part 2",
    2.5: each round, L = the smallest remaining count over sources that still have rows;
    every such source contributes L slots, so the round covers L * (number active)
    positions.  If j falls inside the round, the round is read source-interleaved: source
    = the (j mod active)-th active source in ascending order, slot = offset + j div active
    (the pages' walkthrough: index 7 of 3/5/2 lands in round 2 at slot 2 of shard 1).
    Otherwise j drops by the round size, offset grows by L and every count drops by L.
    """
    rem = [int(c) for c in counts]
    if j < 0 or j >= sum(rem):
        raise IndexError("position outside the expert's rows")
    offset = 0
    while True:
        active = [s for s, c in enumerate(rem) if c > 0]
        length = min(rem[s] for s in active)
        n_round = length * len(active)
        if j < n_round:
            return active[j % len(active)], offset + j // len(active)
        j -= n_round
        offset += length
        rem = [c - min(c, length) for c in rem]


def rr_sequence(counts: Sequence[int]) -> List[Tuple[int, int]]:
    """All positions of one expert in order: the same rounds as rr_inverse, enumerated."""
    rem = [int(c) for c in counts]
    out: List[Tuple[int, int]] = []
    offset = 0
    while any(c > 0 for c in rem):
        active = [s for s, c in enumerate(rem) if c > 0]
        length = min(rem[s] for s in active)
        for i in range(length):
            for s in active:
                out.append((s, offset + i))
        offset += length
        rem = [c - min(c, length) for c in rem]
    return out


def rr_position(counts: Sequence[int], s: int, q: int) -> int:
    """Closed form of the inverse: position of slot q of source s.

    Every source with more than q rows places its slots 0..q-1 before the round that
    holds slot q; inside that stretch, sources are interleaved in ascending order.
    pos = sum_s' min(count[s'], q) + #{s' < s : count[s'] > q}.
    """
    c = [int(v) for v in counts]
    if not (0 <= q < c[s]):
        raise IndexError("slot outside the source's rows")
    return sum(min(v, q) for v in c) + sum(1 for sp in range(s) if c[sp] > q)


# ----------------------------------------------------------------------------- pool fill
def fill_pool(x: np.ndarray, x_sf: np.ndarray, rt: RouteResult, block_m: int, topk: int,
              shared_shard: Optional[int] = None, shared_tokens: int = 0):
    """The expert-major L1 pool: rows, per-128 scales and source metadata.

    "Mega-MoE notes, part 2", 2.6 and "DeepGEMM Mega MoE symmetric memory deep analysis",
    7.4: pool row off[le]*BM + j receives the FP8 row and the scale row of the token that
    the table names at (le, source, slot) from the round-robin, plus metadata
    {rank, token, topk} ("Dispatch/Combine ... comparison", 6.2).  Rows past recv_tot in
    an expert's last block are padding: zero codes, zero scales, metadata all ones (the
    pages skip those rows and leave their content open; zeros are the reading taken here).

    shared_shard: with a shared expert, one more segment follows the routed experts: the
    shared expert reads this rank's own input tokens, not pulled ones ("DeepGEMM Mega MoE
    symmetric memory deep analysis", 4.1: the shared expert's L1 tokens reuse the input
    buffer), so its rows are tokens 0..shared_tokens-1 of shard `shared_shard` in order,
    with top-k slot K (the extra combine slot, 8.2), padded to BM like every expert.  The
    returned offsets then have E_l+2 entries, the last one ending the shared segment.
    """
    El = rt.recv.shape[0]
    H = x.shape[2]
    off = pool_offsets(rt.recv_tot, block_m)
    if shared_shard is not None:
        off = np.append(off, off[-1] + (int(shared_tokens) + block_m - 1) // block_m)
    P = int(off[-1]) * block_m
    # FP8 codes (uint8) with scales, or (BF16 x BF16, x_sf None) the bf16 values themselves
    pool_x = np.zeros((P, H), dtype=x.dtype)
    pool_sf = np.zeros((P, H // 128), dtype=np.float32) if x_sf is not None else None
    pool_meta = np.full((P, 3), META_PAD, dtype=np.uint32)
    for le in range(El):
        base = int(off[le]) * block_m
        seq = rr_sequence(rt.recv[le])
        if not seq:
            continue
        s = np.array([p[0] for p in seq], dtype=np.int64)
        q = np.array([p[1] for p in seq], dtype=np.int64)
        v = rt.table[le, s, q]
        t, k = v // topk, v % topk
        rows = base + np.arange(len(seq))
        pool_x[rows] = x[s, t]
        if x_sf is not None:
            pool_sf[rows] = x_sf[s, t]
        pool_meta[rows, 0] = s
        pool_meta[rows, 1] = t
        pool_meta[rows, 2] = k
    if shared_shard is not None and shared_tokens > 0:
        t = np.arange(int(shared_tokens), dtype=np.int64)
        rows = int(off[El]) * block_m + t
        pool_x[rows] = x[shared_shard, t]
        if x_sf is not None:
            pool_sf[rows] = x_sf[shared_shard, t]
        pool_meta[rows, 0] = shared_shard
        pool_meta[rows, 1] = t
        pool_meta[rows, 2] = topk
    return pool_x, pool_sf, pool_meta, off


# ----------------------------------------------------------------------------- expert FFN
def dequant_rows(codes: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """Per-row, per-128-column scaled FP8 -> float64: v[m, c] = dec(q[m, c]) * sf[m, c/128]."""
    v = e4m3fn_decode(codes)
    return v * np.repeat(np.asarray(sf, dtype=np.float64), 128, axis=-1)


def dequant_blocks(codes: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """128x128 block-scaled FP8 weight [N, C] -> float64: W[n, c] = dec(q) * sf[n/128, c/128]."""
    v = e4m3fn_decode(codes)
    s = np.repeat(np.repeat(np.asarray(sf, dtype=np.float64), 128, axis=0), 128, axis=1)
    return v * s


def swiglu(g: np.ndarray, intermediate: int) -> np.ndarray:
    """h = silu(gate) * up with gate = first I columns, up = last I columns, silu(z) = z/(1+e^-z).

    W1 rows 0..I-1 are the gate half and I..2I-1 the up half ("DeepGEMM Mega MoE symmetric
    memory deep analysis", 10.2, which interleaves the two halves of that [gate | up]
    layout); the first layer's epilogue applies SwiGLU ("Mega-MoE kernel code walkthrough",
    section 6).
    """
    gate = g[:, :intermediate]
    up = g[:, intermediate:]
    # e^-z overflows to inf for very negative z, and z/inf = -0 is silu's limit there
    with np.errstate(over="ignore"):
        return gate / (1.0 + np.exp(-gate)) * up


def requant_rows(h: np.ndarray, gran: int = 128):
    """Requantise activations to FP8 with one fp32 scale per row and per `gran` columns.

    The first layer's epilogue writes FP8 activations plus scale factors for the second
    layer ("Mega-MoE kernel code walkthrough", section 6 and 8.2).  The scale rule is this
    build's reading (the pages give none): s = max(amax, 1e-4) / 448, q = e4m3fn(h * (1 / s))
    with ties to even and saturation, where 1 / s is the fp32 reciprocal and the product one fp32
    multiply.  The decision is taken in fp32, as the kernel takes it.
    Returns (codes uint8 [M, C], scales float32 [M, C/gran]).
    """
    h32 = np.asarray(h, dtype=np.float64).astype(np.float32)
    M, C = h32.shape
    hb = h32.reshape(M, C // gran, gran)
    amax = np.abs(hb).max(axis=2)
    s = np.maximum(amax, np.float32(1e-4)).astype(np.float32) / np.float32(E4M3_MAX)
    s = s.astype(np.float32)
    inv = (np.float32(1.0) / s).astype(np.float32)
    v = (hb * inv[:, :, None]).astype(np.float32)
    codes = e4m3fn_encode(v).reshape(M, C)
    return codes, s


def dequant_weight(codes: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """One expert's weight in either format: FP8 codes [N, C] with fp32 128x128 block scales, or MXFP4
    (packed e2m1 [N, C/2] with UE8M0 bytes [N, C/32]; oracle/fp4.py), told apart by the scale dtype."""
    if np.asarray(sf).dtype == np.uint8:
        return dequant_mx(codes, sf)
    return dequant_blocks(codes, sf)


def expert_ffn_rows_bf16(a, w1, w2, intermediate: int, return_parts: bool = False):
    """One expert's FFN with BF16 x BF16 operands: GEMM1 -> SwiGLU -> bf16 -> GEMM2 -> bf16.

    The pages select a separate BF16 kernel by the operand type, and its input buffer takes the
    bf16 tokens without scale factors ("DeepGEMM Mega MoE symmetric memory deep analysis", 5.3 and
    10.1).  Reading taken here (the pages give no detail): the sums are exact (fp64 here, fp32 in
    the kernel), the SwiGLU output is rounded to bf16 where the FP8 path requantises (the second
    GEMM's operands are then bf16 as well), and GEMM2's output is cast to bf16 for the combine buffer
    as in the FP8 path (same page, 8.1-8.2).
    """
    a = np.asarray(a, dtype=np.float64)
    g = a @ np.asarray(w1, dtype=np.float64).T
    h = swiglu(g, intermediate)
    hb = bf16_round(h)
    o = bf16_round(hb @ np.asarray(w2, dtype=np.float64).T)
    if return_parts:
        return o, dict(g=g, h=h, l2=hb)
    return o


def expert_ffn_rows(a_codes, a_sf, w1_codes, w1_sf, w2_codes, w2_sf, intermediate: int,
                    gran: int = 128, return_parts: bool = False):
    """One expert's FFN on pooled rows: GEMM1 -> SwiGLU -> FP8 requant -> GEMM2 -> bf16.

    GEMM1 (gate_up): G = A W1^T with A, W1 dequantised; the per-128-K promotion of the
    pages ("Mega-MoE notes, part 2", 5.2) is the blockwise form of exactly this sum.
    GEMM2 (down): O = requant(h) W2^T.  The second layer's epilogue casts to bf16 before
    the scatter into the combine buffer ("DeepGEMM Mega MoE symmetric memory deep
    analysis", 8.1-8.2).  Rows without scales (a_sf None) are BF16 x BF16: expert_ffn_rows_bf16.
    """
    if a_sf is None:
        return expert_ffn_rows_bf16(a_codes, w1_codes, w2_codes, intermediate, return_parts)
    a = dequant_rows(a_codes, a_sf)
    w1 = dequant_weight(w1_codes, w1_sf)
    g = a @ w1.T
    h = swiglu(g, intermediate)
    q, s = requant_rows(h, gran)
    hq = dequant_rows_gran(q, s, gran)
    w2 = dequant_weight(w2_codes, w2_sf)
    o = bf16_round(hq @ w2.T)
    if return_parts:
        return o, dict(g=g, h=h, l2_codes=q, l2_sf=s)
    return o


def ffn_dequantised(a: np.ndarray, w1: np.ndarray, w2: np.ndarray, intermediate: int,
                    gran: int = 128) -> np.ndarray:
    """The same FFN steps as expert_ffn_rows on already dequantised rows and weights."""
    h = swiglu(a @ w1.T, intermediate)
    q, s = requant_rows(h, gran)
    return bf16_round(dequant_rows_gran(q, s, gran) @ w2.T)


def dequant_rows_gran(codes, sf, gran):
    v = e4m3fn_decode(codes)
    return v * np.repeat(np.asarray(sf, dtype=np.float64), gran, axis=-1)


# ----------------------------------------------------------------------------- full layer
def _intermediate(inp) -> int:
    """I from the down weights: their scales' K extent (FP8: per 128, MXFP4: per 32), or with
    BF16 x BF16 weights (no scales) the weights' own last axis."""
    s2 = inp.get("w2_sf")
    if s2 is None:
        return int(inp["w2"].shape[2])
    return int(s2.shape[2] * (32 if s2.dtype == np.uint8 else 128))


def _scale_of(inp):
    """name, expert -> that expert's scale array, or None without scales (BF16 x BF16)."""
    return lambda name, le: None if inp.get(name) is None else inp[name][le]


def forward(inp: Dict[str, object], num_experts: int, num_local_experts: int, local_rank: int,
            block_m: int, gran: int = 128, experts: Optional[Sequence[int]] = None,
            keep_rows: bool = False, num_shared_experts: int = 0) -> Dict[str, object]:
    """The whole layer on numpy inputs (the dict made by inputs.make_inputs + to_numpy).

    Steps in the pages' order: counts and table, pool layout, round-robin pull, GEMM1,
    SwiGLU, requant, GEMM2 (bf16 into the combine buffer), then the combine
    y[s,t] = bf16(sum over local k of w[s,t,k] * comb[k][s,t]) ("Dispatch/Combine ...
    comparison", section 1: the output is the weight-sum of the chosen experts' outputs;
    "DeepGEMM Mega MoE symmetric memory deep analysis", 9.2: per token, slots with a
    negative index are masked and the rest accumulate in fp32).  Tokens with no local
    expert get a zero row; rows t >= T_s are not part of the output (returned as NaN).

    experts: restrict the FFN to these local experts (the others contribute nothing); used
    to time a bounded sample.  keep_rows: also return per-pool-row outputs and l2 parts.

    num_shared_experts = 1: the shared expert (weights at index E_l of w1/w2) runs on every
    valid token of this rank's own shard (shard local_rank), and its bf16 output is added
    with weight 1 after the routed slots: the pages' combine walks the top-k slots and then
    the extra shared slot K, and the shared expert's epilogue applies no routing weight
    ("DeepGEMM Mega MoE symmetric memory deep analysis", 8.1-8.2 and 9.2).
    """
    x, x_sf = inp["x"], inp.get("x_sf")
    idx, w = inp["topk_idx"], inp["topk_weights"]
    tps = inp["tokens_per_shard"]
    S, T_max, K = idx.shape
    H = x.shape[2]
    I = _intermediate(inp)
    sf = _scale_of(inp)
    rt = route(idx, tps, num_experts, num_local_experts, local_rank)
    shared = num_shared_experts > 0
    pool_x, pool_sf, pool_meta, off = fill_pool(x, x_sf, rt, block_m, K,
                                                shared_shard=local_rank if shared else None,
                                                shared_tokens=int(tps[local_rank]) if shared else 0)
    y = np.zeros((S, T_max, H), dtype=np.float64)
    rows_out = {}
    parts_out = {}
    sel = range(num_local_experts) if experts is None else experts
    for le in sel:
        n = int(rt.recv_tot[le])
        if n == 0:
            continue
        base = int(off[le]) * block_m
        rows = slice(base, base + n)
        o, parts = expert_ffn_rows(pool_x[rows], None if pool_sf is None else pool_sf[rows], inp["w1"][le],
                                   sf("w1_sf", le), inp["w2"][le], sf("w2_sf", le), I, gran, return_parts=True)
        meta = pool_meta[rows]
        s_, t_, k_ = meta[:, 0].astype(np.int64), meta[:, 1].astype(np.int64), meta[:, 2].astype(np.int64)
        # combine: accumulate w * comb row into the token's output (each (s,t,k) occurs once)
        np.add.at(y, (s_, t_), w[s_, t_, k_][:, None].astype(np.float64) * o)
        if keep_rows:
            rows_out[le] = o
            parts_out[le] = parts
    if shared and int(tps[local_rank]) > 0:
        El, n = num_local_experts, int(tps[local_rank])
        rows = slice(int(off[El]) * block_m, int(off[El]) * block_m + n)
        o, parts = expert_ffn_rows(pool_x[rows], None if pool_sf is None else pool_sf[rows], inp["w1"][El],
                                   sf("w1_sf", El), inp["w2"][El], sf("w2_sf", El), I, gran, return_parts=True)
        y[local_rank, :n] += o
        if keep_rows:
            rows_out[El] = o
            parts_out[El] = parts
    y = bf16_round(y)
    for s in range(S):
        y[s, int(tps[s]):] = np.nan
    out = dict(route=rt, off=off, pool_x=pool_x, pool_sf=pool_sf, pool_meta=pool_meta, y=y)
    if keep_rows:
        out["rows"] = rows_out
        out["parts"] = parts_out
    return out


def direct_token(inp: Dict[str, object], s: int, t: int, num_local_experts: int,
                 local_rank: int, gran: int = 128, cache: Optional[dict] = None,
                 num_shared_experts: int = 0) -> np.ndarray:
    """y[s,t] evaluated on its own: no counts, no table, no pool.

    out(T) = sum over the token's local experts of w_k * Expert_k(T) ("Dispatch/Combine ...
    comparison", section 1), with each Expert_k the same FFN steps as the pooled path,
    plus, with a shared expert, Shared(T) with weight 1 for the tokens of shard local_rank.
    Returns a bf16-rounded float64 row of length H.
    """
    K = inp["topk_idx"].shape[2]
    lo = local_rank * num_local_experts
    I = _intermediate(inp)
    sf = _scale_of(inp)
    a_codes = inp["x"][s, t][None, :]
    a_sf = None if inp.get("x_sf") is None else inp["x_sf"][s, t][None, :]
    acc = np.zeros(inp["x"].shape[2], dtype=np.float64)
    slots = []
    for k in range(K):
        e = int(inp["topk_idx"][s, t, k])
        if lo <= e < lo + num_local_experts:
            slots.append((e - lo, float(inp["topk_weights"][s, t, k])))
    if num_shared_experts > 0 and s == local_rank:
        slots.append((num_local_experts, 1.0))
    for le, wk in slots:
        if cache is None or a_sf is None:
            o = expert_ffn_rows(a_codes, a_sf, inp["w1"][le], sf("w1_sf", le), inp["w2"][le],
                                sf("w2_sf", le), I, gran)[0]
        else:
            if le not in cache:
                cache[le] = (dequant_weight(inp["w1"][le], inp["w1_sf"][le]),
                             dequant_weight(inp["w2"][le], inp["w2_sf"][le]))
            o = ffn_dequantised(dequant_rows(a_codes, a_sf), cache[le][0], cache[le][1], I, gran)[0]
        acc += wk * o
    return bf16_round(acc)
