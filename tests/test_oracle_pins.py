"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU)."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from inputs import MoEShape, SHAPES, make_inputs, to_numpy

from conftest import load_golden


# ------------------------------------------------------------------ FP8 / bf16 codecs
def test_e4m3fn_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], got[~nan])
    # closed forms from the format definition
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert got[0x38] == 1.0 and got[0xB8] == -1.0


def test_e4m3fn_encode_matches_torch_in_range_and_ties():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000) * 50,
        rng.standard_normal(20000) * 1e-2,
        rng.uniform(-464, 464, 20000),
        np.ldexp(rng.integers(-16, 16, 5000).astype(np.float64), rng.integers(-12, 6, 5000)),
    ]).astype(np.float32)
    # exact midpoints between neighbouring codes (ties go to the even code)
    finite = oracle.e4m3fn_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = ((finite[:-1] + finite[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    v = v[np.abs(v) <= 464]          # torch's cast does not saturate beyond the last midpoint
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3fn_encode(v)
    zero = oracle.e4m3fn_decode(ref) == 0
    # +-0 are both zero; compare by value there and by code elsewhere
    assert np.array_equal(got[~zero], ref[~zero])
    assert np.all(oracle.e4m3fn_decode(got[zero]) == 0)


def test_e4m3fn_encode_saturates():
    big = np.array([449, 463.9, 464, 1e4, -600, np.inf, -np.inf], dtype=np.float32)
    got = oracle.e4m3fn_encode(big)
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]
    assert oracle.e4m3fn_encode(np.array([np.nan], dtype=np.float32))[0] == 0x7F


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(50000) * 3,
                        rng.standard_normal(5000) * 1e-30,
                        rng.standard_normal(5000) * 1e30]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(v.astype(np.float64))
    assert np.array_equal(ref, got)
    assert np.array_equal(oracle.bf16_bits(got),
                          torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------------ round-robin
def test_round_robin_walkthrough():
    g = load_golden("round_robin_3_5_2.json")
    counts = g["counts"]
    seq = oracle.rr_sequence(counts)
    assert len(seq) == sum(counts)
    for lo, hi, sources in g["position_sources"]:
        assert sorted({seq[j][0] for j in range(lo, hi + 1)}) == sources
        assert [seq[j][0] for j in range(lo, hi + 1)] == \
            [sources[i % len(sources)] for i in range(hi - lo + 1)]
    assert sorted({seq[j][1] for j in range(0, 6)}) == g["position_slots_first_round"]
    assert [seq[8][1], seq[9][1]] == g["last_two_slots_of_rank1"]
    assert oracle.rr_inverse(counts, g["index"]) == (g["index_source"], g["index_slot"])
    assert oracle.rr_position(counts, g["index_source"], g["index_slot"]) == g["index"]


def test_round_robin_exhaustive_small():
    """min-peeling (per position) == enumerated rounds == closed form == (slot, source) sort."""
    for S in range(1, 5):
        for counts in itertools.product(range(0, 5), repeat=S):
            seq = oracle.rr_sequence(counts)
            lex = sorted(((q, s) for s in range(S) for q in range(counts[s])))
            assert seq == [(s, q) for q, s in lex]
            for j, (s, q) in enumerate(seq):
                assert oracle.rr_inverse(counts, j) == (s, q)
                assert oracle.rr_position(counts, s, q) == j


def test_round_robin_random_many_sources():
    rng = np.random.default_rng(2)
    for _ in range(200):
        S = int(rng.integers(1, 65))
        counts = rng.integers(0, 40, S)
        seq = oracle.rr_sequence(counts)
        assert sorted(seq) == sorted((s, q) for s in range(S) for q in range(counts[s]))
        for j in rng.integers(0, max(1, len(seq)), 5):
            if seq:
                assert oracle.rr_inverse(counts, int(j)) == seq[int(j)]


# ------------------------------------------------------------------ pool layout
def test_pool_segmentation_example():
    g = load_golden("pool_segmentation_100_10_30.json")
    recv = g["recv_tot"]
    start = 0
    for c, (lo, hi) in zip(recv, g["flat_ranges"]):
        assert (start, start + c - 1) == (lo, hi)
        start += c
    for bm, want in g["block_offsets"].items():
        assert oracle.pool_offsets(recv, int(bm)).tolist() == want


def test_pool_capacity_bound():
    """sum ceil(recv/BM) <= ceil(R/BM) + E_l (DeepGEMM Mega MoE symmetric memory deep
    analysis, 4.2: pool blocks = ceil_div(max routed, BLOCK_M) + experts per rank)."""
    rng = np.random.default_rng(3)
    for _ in range(2000):
        El = int(rng.integers(1, 64))
        bm = int(rng.choice([64, 128]))
        recv = rng.integers(0, 600, El)
        off = oracle.pool_offsets(recv, bm)
        R = int(recv.sum())
        assert off[-1] <= -(-R // bm) + El
        assert off[-1] >= -(-R // bm)


def test_expert_rank_map():
    g = load_golden("expert_rank_map.json")
    per = g["experts_per_rank"]
    for rank, owned in g["owners"].items():
        # one token per global expert; only the owner's experts land in its table
        idx = np.arange(8, dtype=np.int64).reshape(1, 8, 1)
        rt = oracle.route(idx, [8], 8, per, int(rank))
        assert rt.recv_tot.tolist() == [1] * per
        locals_ = [int(rt.table[le, 0, 0]) for le in range(per)]
        assert locals_ == owned       # flat index t*K+k == t == global expert here


def test_slot_claim_example():
    """The later contributor's rows start at the earlier contributor's count."""
    g = load_golden("slot_claim_3_2.json")
    a, b = g["first_contributor"], g["second_contributor"]
    T = a + b + 3
    idx = np.full((1, T, 1), 5, dtype=np.int64)      # all to some other expert
    idx[0, :a, 0] = 0
    idx[0, a + 3:a + 3 + b, 0] = 0
    rt = oracle.route(idx, [T], 8, 8, 0)
    slots_of = {int(rt.table[0, 0, q]): q for q in range(int(rt.recv[0, 0]))}
    assert [slots_of[t] for t in range(a)] == g["first_slots"]
    assert [slots_of[t] for t in range(a + 3, a + 3 + b)] == g["second_slots"]


def test_route_conservation_and_table():
    for name in ["tiny", "mid"]:
        sh = SHAPES[name].replace(max_tokens_per_shard=64, hidden=128, intermediate=128)
        inp = to_numpy(make_inputs(sh))
        idx = inp["topk_idx"].copy()
        idx[0, 3, 1] = -1
        idx[-1, 10, 0] = -7
        tps = [64 - 5 * s for s in range(sh.num_shards)]
        rt = oracle.route(idx, tps, sh.num_experts, sh.num_local_experts, sh.local_rank)
        valid = sum(t * sh.topk for t in tps)
        neg = sum(int((idx[s, :tps[s]] < 0).sum()) for s in range(sh.num_shards))
        assert rt.send.sum() == valid - neg
        lo = sh.local_rank * sh.num_local_experts
        assert np.array_equal(rt.recv, rt.send[:, lo:lo + sh.num_local_experts].T)
        # every local entry appears exactly once in the table, in ascending order per (le, s)
        for s in range(sh.num_shards):
            for le in range(sh.num_local_experts):
                got = rt.table[le, s, :rt.recv[le, s]]
                flat = idx[s, :tps[s]].reshape(-1)
                want = np.nonzero(flat == lo + le)[0]
                assert np.array_equal(got, want)
    # Tiny: all experts are local, so the received count is T*K exactly
    sh = SHAPES["tiny"]
    inp = to_numpy(make_inputs(sh))
    rt = oracle.route(inp["topk_idx"], inp["tokens_per_shard"], sh.num_experts,
                      sh.num_local_experts, 0)
    assert rt.recv_tot.sum() == sh.max_tokens_per_shard * sh.topk == 128


def test_route_bad_expert_and_overflow_flags():
    idx = np.array([[[0, 9], [1, 2]]], dtype=np.int64)      # 9 >= E=8
    rt = oracle.route(idx, [2], 8, 8, 0)
    assert rt.bad_expert and rt.send.sum() == 3
    dup = np.zeros((1, 2, 2), dtype=np.int64)                 # same expert twice per token
    rt = oracle.route(dup, [2], 8, 8, 0)
    assert rt.slot_overflow and rt.recv[0, 0] == 2


def test_pool_fill_invariants():
    sh = SHAPES["mid"].replace(max_tokens_per_shard=96, hidden=128, intermediate=128)
    inp = to_numpy(make_inputs(sh))
    rt = oracle.route(inp["topk_idx"], inp["tokens_per_shard"], sh.num_experts,
                      sh.num_local_experts, 0)
    px, psf, pm, off = oracle.fill_pool(inp["x"], inp["x_sf"], rt, sh.block_m, sh.topk)
    assert px.shape[0] == off[-1] * sh.block_m
    seen = set()
    for le in range(sh.num_local_experts):
        base = off[le] * sh.block_m
        n = rt.recv_tot[le]
        for j in range(n):
            s, t, k = (int(v) for v in pm[base + j])
            assert sh.topk * t + k in rt.table[le, s, :rt.recv[le, s]]
            assert inp["topk_idx"][s, t, k] == le
            assert np.array_equal(px[base + j], inp["x"][s, t])
            assert np.array_equal(psf[base + j], inp["x_sf"][s, t])
            seen.add((s, t, k))
            # round-robin: position j is rr_inverse's source and the table's slot
            src, q = oracle.rr_inverse(rt.recv[le], j)
            assert src == s and rt.table[le, s, q] == t * sh.topk + k
        pad = slice(base + n, (off[le + 1]) * sh.block_m)
        assert np.all(px[pad] == 0) and np.all(psf[pad] == 0) and np.all(pm[pad] == 0xFFFFFFFF)
    want = {(s, t, k) for s in range(sh.num_shards) for t in range(sh.max_tokens_per_shard)
            for k in range(sh.topk) if inp["topk_idx"][s, t, k] < sh.num_local_experts}
    assert seen == want


# ------------------------------------------------------------------ FFN pieces
def test_silu_sign_and_gate_up_order():
    # silu(z) - silu(-z) = z for every z (catches a sign error in the exponent)
    z = np.linspace(-20, 20, 4001)
    g = np.concatenate([z[:, None], -z[:, None]], axis=1)
    up1 = np.ones_like(g)
    h = oracle.swiglu(np.concatenate([g, up1], axis=1), 2)
    assert np.allclose(h[:, 0] - h[:, 1], z, atol=1e-12)
    # gate first, up second ([gate | up] before the reference's interleaving transform)
    h = oracle.swiglu(np.array([[2.0, 0.5]]), 1)
    assert math.isclose(h[0, 0], 2.0 / (1 + math.exp(-2.0)) * 0.5, rel_tol=1e-15)


def test_requant_closed_forms():
    # a row whose 128-block amax is 448*2^-3 gets scale 2^-3 and codes equal to h/2^-3
    vals = oracle.e4m3fn_decode(np.arange(0, 0x7F, dtype=np.uint8))
    rng = np.random.default_rng(4)
    h = rng.choice(vals, size=(3, 256)) * 2.0 ** -3
    h[:, 0] = 448 * 2.0 ** -3
    h[:, 128] = -448 * 2.0 ** -3
    q, s = oracle.requant_rows(h)
    assert np.all(s == np.float32(2.0 ** -3))
    assert np.array_equal(oracle.e4m3fn_decode(q) * 2.0 ** -3, h)
    # all-zero block: epsilon scale, zero codes
    q, s = oracle.requant_rows(np.zeros((1, 128)))
    assert s[0, 0] == np.float32(np.float32(1e-4) / np.float32(448)) and np.all(q == 0)
    # requant error is within half a code step of the block scale
    h = rng.standard_normal((8, 512))
    q, s = oracle.requant_rows(h)
    back = oracle.e4m3fn_decode(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    rel = np.abs(back - h) / np.repeat(np.abs(h).reshape(8, 4, 128).max(2), 128, axis=1)
    assert rel.max() < 2.0 ** -4 * 1.01


def test_requant_uses_the_fp32_reciprocal_of_the_scale():
    """The code is decided on h * fp32(1/s), not on h / s.  For this block amax and value the two fp32
    results are 400.0 exactly (a tie between the e4m3 codes for 384 and 416, so to even: 384) and
    400.00003 (416); the value was found by search over random h."""
    h = np.zeros((1, 128), dtype=np.float32)
    h[0, 0] = np.float32(3.5609652996063232)      # the block's amax
    h[0, 1] = np.float32(3.1794333457946777)
    q, s = oracle.requant_rows(h)
    assert s[0, 0] == np.float32(np.float32(3.5609652996063232) / np.float32(448))
    assert oracle.e4m3fn_decode(q[0, 1:2])[0] == 384.0
    # division would have rounded up
    assert (h[0, 1] / s[0, 0]).astype(np.float32) > np.float32(400.0)
    assert oracle.e4m3fn_decode(oracle.e4m3fn_encode(np.float32(h[0, 1] / s[0, 0])[None]))[0] == 416.0


def test_requant_scale_granularity():
    """The scale covers `gran` columns: a row of two 64-column halves holding 1.0 and 4.0 gets, with
    gran = 64, scales 1/448 and 4/448 and every code 448 (e4m3fn 0x7E); with gran = 128, the one scale
    4/448, codes 448 for the second half and 448/4 = 112 (0x6E: 2^6 * 1.75) for the first."""
    h = np.concatenate([np.full((1, 64), 1.0), np.full((1, 64), 4.0)], axis=1)
    q, s = oracle.requant_rows(h, gran=64)
    assert s.shape == (1, 2)
    assert s[0, 0] == np.float32(np.float32(1.0) / np.float32(448))
    assert s[0, 1] == np.float32(np.float32(4.0) / np.float32(448))
    assert np.all(q == 0x7E)
    q, s = oracle.requant_rows(h)
    assert s.shape == (1, 1) and s[0, 0] == np.float32(np.float32(4.0) / np.float32(448))
    assert np.all(q[0, :64] == 0x6E) and np.all(q[0, 64:] == 0x7E)
    # each half comes back from its own code and scale
    q, s = oracle.requant_rows(h, gran=64)
    back = oracle.e4m3fn_decode(q) * np.repeat(s.astype(np.float64), 64, axis=1)
    assert np.allclose(back, h, rtol=1e-6, atol=0)


def test_gemm1_exact_on_integer_codes():
    """Integer codes with power-of-two scales: G equals an int64 matmul times the scales."""
    sh = MoEShape("t", 1, 32, 256, 128, 2, 2, 1, 64)
    inp = to_numpy(make_inputs(sh, integer_codes=True))
    a = oracle.e4m3fn_decode(inp["x"][0]).astype(np.int64)
    w = oracle.e4m3fn_decode(inp["w1"][1]).astype(np.int64)
    want = (a @ w.T).astype(np.float64) * 2.0 ** -4 * 2.0 ** -6
    got = oracle.dequant_rows(inp["x"][0], inp["x_sf"][0]) @ \
        oracle.dequant_blocks(inp["w1"][1], inp["w1_sf"][1]).T
    assert np.array_equal(got, want)


def _torch_textbook(x_codes, x_sf, w1, w1_sf, w2, w2_sf, I):
    """The same layer for one row through torch CPU library routines only."""
    f8 = torch.float8_e4m3fn
    x = torch.from_numpy(x_codes).view(f8).to(torch.float64) * \
        torch.from_numpy(x_sf).to(torch.float64).repeat_interleave(128, -1)

    def wdeq(c, s):
        return torch.from_numpy(c).view(f8).to(torch.float64) * torch.from_numpy(s).to(
            torch.float64).repeat_interleave(128, 0).repeat_interleave(128, 1)
    W1, W2 = wdeq(w1, w1_sf), wdeq(w2, w2_sf)
    g = torch.matmul(x, W1.T)
    h = (torch.nn.functional.silu(g[..., :I]) * g[..., I:]).to(torch.float32)
    hb = h.reshape(*h.shape[:-1], -1, 128)
    s = torch.clamp(hb.abs().amax(-1), min=1e-4) / 448.0
    q = (hb / s.unsqueeze(-1)).to(f8)
    hq = (q.to(torch.float64) * s.to(torch.float64).unsqueeze(-1)).reshape(h.shape)
    o = torch.matmul(hq, W2.T)
    return o, q.view(torch.uint8).reshape(h.shape).numpy()


def test_textbook_reduction_single_expert():
    """S=1, E_l=1, K=1, w=1: y = bf16(W2 requant(silu(W1g x) * W1u x)) -- torch routines."""
    sh = MoEShape("t", 1, 48, 384, 256, 1, 1, 1, 64)
    inp = to_numpy(make_inputs(sh))
    inp["topk_idx"][:] = 0
    inp["topk_weights"][:] = 1.0
    out = oracle.forward(inp, 1, 1, 0, sh.block_m, keep_rows=True)
    o, q = _torch_textbook(inp["x"][0], inp["x_sf"][0], inp["w1"][0], inp["w1_sf"][0],
                           inp["w2"][0], inp["w2_sf"][0], sh.intermediate)
    want = o.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    y = out["y"][0]
    # order pool rows back to tokens through the metadata
    assert np.array_equal(out["pool_meta"][:48, 1], np.arange(48))
    assert np.mean(out["parts"][0]["l2_codes"] == q) > 0.999
    ulp = np.abs(want) * 2.0 ** -7
    assert np.all(np.abs(y - want) <= ulp + 1e-30)


def test_combine_identity_example():
    g = load_golden("combine_identity.json")
    sh = MoEShape("t", 1, 16, 256, 128, 8, 8, 2, 64)
    inp = to_numpy(make_inputs(sh))
    inp["topk_idx"][0, 0] = g["experts"]
    inp["topk_weights"][0, 0] = g["weights"]
    out = oracle.forward(inp, 8, 8, 0, sh.block_m)
    e2, _ = _torch_textbook(inp["x"][0, :1], inp["x_sf"][0, :1], inp["w1"][2], inp["w1_sf"][2],
                            inp["w2"][2], inp["w2_sf"][2], 128)
    e7, _ = _torch_textbook(inp["x"][0, :1], inp["x_sf"][0, :1], inp["w1"][7], inp["w1_sf"][7],
                            inp["w2"][7], inp["w2_sf"][7], 128)
    bf = lambda t: t.to(torch.float32).to(torch.bfloat16).to(torch.float64)  # noqa: E731
    want = (np.float32(g["weights"][0]) * bf(e2) + np.float32(g["weights"][1]) * bf(e7))
    want = bf(want)[0].numpy()
    assert np.all(np.abs(out["y"][0, 0] - want) <= np.abs(want) * 2.0 ** -7 + 1e-30)
    # and the direct per-token path gives the same row
    d = oracle.direct_token(inp, 0, 0, 8, 0)
    assert np.array_equal(d, out["y"][0, 0])


def test_gate_up_halves_closed_form():
    """Constant gate half gives G_gate = 2, constant up half G_up = 0.5: h = silu(2) * 0.5."""
    H = I = 128
    sh = MoEShape("t", 1, 4, H, I, 1, 1, 1, 64)
    inp = to_numpy(make_inputs(sh))
    inp["x"][:] = 0x38                                   # 1.0
    inp["x_sf"][:] = 1.0 / 128
    inp["w1"][0, :I] = 0x40                              # 2.0  (gate rows)
    inp["w1"][0, I:] = 0x30                              # 0.5  (up rows)
    inp["w1_sf"][:] = 1.0
    inp["w2"][:] = 0x38
    inp["w2_sf"][:] = 1.0
    inp["topk_idx"][:] = 0
    inp["topk_weights"][:] = 1.0
    out = oracle.forward(inp, 1, 1, 0, 64)
    h = 2.0 / (1 + math.exp(-2.0)) * 0.5
    assert np.allclose(out["y"][0], 128 * h, rtol=2.0 ** -7)


# ------------------------------------------------------------------ whole layer
def _brute_inputs(S, T, E, El, r, K, idx_choice):
    sh = MoEShape("b", S, T, 128, 128, E, El, K, 64, local_rank=r)
    inp = to_numpy(make_inputs(sh, seed=11))
    return sh, inp


def test_brute_force_pooled_equals_direct():
    """Every routing of tiny shapes through the pooled path and the direct per-token path."""
    K = 2
    choices = [(a, b) for a in (-1, 0, 1, 2) for b in (-1, 0, 1, 2) if a < 0 or b < 0 or a != b]
    for S, T in [(1, 3), (3, 1)]:
        sh, base = _brute_inputs(S, T, 3, 2, 0, K, None)
        # per-(expert, token) FFN rows memoised through the direct path of single entries
        memo = {}
        for s in range(S):
            for t in range(T):
                for e in range(2):
                    one = dict(base)
                    one["topk_idx"] = np.full_like(base["topk_idx"], -1)
                    one["topk_idx"][s, t, 0] = e
                    one["topk_weights"] = np.ones_like(base["topk_weights"])
                    memo[(e, s, t)] = oracle.direct_token(one, s, t, 2, 0)
        for combo in itertools.product(choices, repeat=S * T):
            inp = dict(base)
            inp["topk_idx"] = np.array(combo, dtype=np.int64).reshape(S, T, K)
            out = oracle.forward(inp, 3, 2, 0, 64)
            for s in range(S):
                for t in range(T):
                    acc = np.zeros(128)
                    for k in range(K):
                        e = int(inp["topk_idx"][s, t, k])
                        if 0 <= e < 2:
                            acc += float(np.float32(inp["topk_weights"][s, t, k])) * memo[(e, s, t)]
                    assert np.array_equal(out["y"][s, t], oracle.bf16_round(acc)), (combo, s, t)


def test_tokens_beyond_valid_and_no_local_expert():
    sh = MoEShape("t", 2, 8, 128, 128, 8, 4, 2, 64, local_rank=1)
    inp = to_numpy(make_inputs(sh))
    inp["topk_idx"][0, 0] = [0, 1]           # remote experts only -> zero row
    inp["tokens_per_shard"] = [8, 5]
    out = oracle.forward(inp, 8, 4, 1, 64)
    assert np.all(out["y"][0, 0] == 0)
    assert np.all(np.isnan(out["y"][1, 5:]))
    assert not np.any(np.isnan(out["y"][1, :5]))


# ----------------------------------------------------------------------------- shared expert
def test_shared_expert_textbook():
    """One routed expert with weight w plus the shared expert on the rank's own shard:
    y = bf16(w * bf16(E0(x)) + bf16(Shared(x))), each FFN through torch routines only; tokens of
    the other shard get no shared contribution."""
    sh = MoEShape("t", 2, 24, 256, 128, 2, 1, 1, 64, local_rank=1, num_shared_experts=1, seed=5)
    inp = to_numpy(make_inputs(sh))
    assert inp["w1"].shape[0] == 2           # routed expert 0, shared expert at index E_l = 1
    inp["topk_idx"][:] = 1                   # global expert 1 = local expert 0 of rank 1
    inp["topk_weights"][:] = 0.625
    inp["tokens_per_shard"] = [24, 17]
    out = oracle.forward(inp, 2, 1, 1, 64, num_shared_experts=1)
    bf = lambda t: t.to(torch.float32).to(torch.bfloat16).to(torch.float64)  # noqa: E731
    for s in (0, 1):
        n = inp["tokens_per_shard"][s]
        e0, _ = _torch_textbook(inp["x"][s, :n], inp["x_sf"][s, :n], inp["w1"][0], inp["w1_sf"][0],
                                inp["w2"][0], inp["w2_sf"][0], 128)
        want = 0.625 * bf(e0)
        if s == 1:
            sx, _ = _torch_textbook(inp["x"][s, :n], inp["x_sf"][s, :n], inp["w1"][1], inp["w1_sf"][1],
                                    inp["w2"][1], inp["w2_sf"][1], 128)
            want = want + bf(sx)
        want = bf(want).numpy()
        assert np.all(np.abs(out["y"][s, :n] - want) <= np.abs(want) * 2.0 ** -7 + 1e-30), s
    # the shared segment follows the routed one: own shard's 17 tokens in order, slot K = 1
    off = out["off"]
    assert len(off) == 3 and off[2] - off[1] == 1      # E_l + 2 entries; ceil(17 / 64) blocks
    seg = out["pool_meta"][off[1] * 64: off[1] * 64 + 64]
    assert np.array_equal(seg[:17, 0], np.full(17, 1)) and np.array_equal(seg[:17, 1], np.arange(17))
    assert np.array_equal(seg[:17, 2], np.full(17, 1)) and np.all(seg[17:] == 0xFFFFFFFF)
    assert np.array_equal(out["pool_x"][off[1] * 64: off[1] * 64 + 17], inp["x"][1, :17])


def test_shared_expert_zero_weights_reduce_to_routed_only():
    """A shared expert with all-zero weight codes contributes exactly zero (silu(0) * 0 = 0, requant
    of a zero row gives zero codes), so the output equals the layer without one, bit for bit."""
    sh = MoEShape("t", 3, 40, 256, 256, 16, 4, 2, 64, local_rank=2, num_shared_experts=1, seed=6)
    inp = to_numpy(make_inputs(sh))
    inp["tokens_per_shard"] = [40, 13, 29]
    inp["w1"][4] = 0
    inp["w2"][4] = 0
    with_sh = oracle.forward(inp, 16, 4, 2, 64, num_shared_experts=1)
    plain = dict(inp)
    for k in ("w1", "w1_sf", "w2", "w2_sf"):
        plain[k] = inp[k][:4]
    without = oracle.forward(plain, 16, 4, 2, 64)
    assert np.array_equal(with_sh["y"], without["y"], equal_nan=True)


def test_shared_expert_brute_force_pooled_equals_direct():
    """Every routing of a tiny shape with a shared expert: pooled path == direct per-token path."""
    K = 2
    choices = [(a, b) for a in (-1, 0, 1) for b in (-1, 0, 1) if a < 0 or b < 0 or a != b]
    sh = MoEShape("b", 2, 2, 128, 128, 2, 2, K, 64, local_rank=0, num_shared_experts=1, seed=7)
    base = to_numpy(make_inputs(sh))
    cache = {}
    for combo in itertools.product(choices, repeat=4):
        inp = dict(base)
        inp["topk_idx"] = np.array(combo, dtype=np.int64).reshape(2, 2, K)
        out = oracle.forward(inp, 2, 2, 0, 64, num_shared_experts=1)
        for s in range(2):
            for t in range(2):
                d = oracle.direct_token(inp, s, t, 2, 0, cache=cache, num_shared_experts=1)
                assert np.allclose(out["y"][s, t], d, rtol=2.0 ** -7, atol=1e-30), (combo, s, t)
