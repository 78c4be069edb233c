"""Helpers for the GPU parity tests: run the HIP layer through the C ABI and read its workspace."""
import numpy as np
import torch

import dispatch_fp8_grouped_amd as mm
import oracle
from inputs import make_inputs, to_numpy


def on_gpu(inputs):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inputs.items()}


class Run:
    """One forward of the HIP layer plus host copies of what the tests compare."""

    def __init__(self, shape, inputs=None, flags=0, cum=None, seed=None, tokens_per_shard=None, repeat=1,
                 generate_on="cuda"):
        if inputs is None:
            inputs = make_inputs(shape, device=generate_on, seed=seed, tokens_per_shard=tokens_per_shard)
        self.shape = shape
        self.inp_gpu = on_gpu(inputs)
        self.moe = mm.MegaMoE.from_shape(shape, flags=flags)
        self.cum = cum
        self.ys = []
        for _ in range(repeat):
            y = torch.full((shape.num_shards, shape.max_tokens_per_shard, shape.hidden), float("nan"),
                           dtype=torch.bfloat16, device="cuda")
            self.moe(self.inp_gpu, y=y, cum_recv_stats=cum)
            self.ys.append(y)
        self.status = self.moe.status()
        torch.cuda.synchronize()
        self.y = self.ys[-1]

    # ---- workspace reads
    def region(self, name, dtype, shape):
        return self.moe.region(name, dtype, shape)

    def layout_host(self):
        sh, L = self.shape, self.moe.layout
        S, T, E, El = sh.num_shards, sh.max_tokens_per_shard, sh.num_experts, sh.num_local_experts
        nsh = getattr(sh, "num_shared_experts", 0)
        status = self.region("status", torch.int32, (2,)).cpu().numpy()
        nb = int(status[1])
        out = dict(
            nblocks=nb,
            send=self.region("send", torch.int32, (S, E)).cpu().numpy(),
            recv=self.region("recv", torch.int32, (El, S)).cpu().numpy(),
            recv_tot=self.region("recv_tot", torch.int32, (El,)).cpu().numpy(),
            pool_off=self.region("pool_off", torch.int32, (El + 2,)).cpu().numpy()[:El + 1 + nsh],
            block_expert=self.region("block_expert", torch.int32, (L["max_pool_blocks"],)).cpu().numpy()[:nb],
            block_index=self.region("block_index", torch.int32, (L["max_pool_blocks"],)).cpu().numpy()[:nb],
            table=self.region("table", torch.int32, (El, S, T)).cpu().numpy(),
        )
        return out

    def pool_host(self, rows=None):
        sh = self.shape
        nb = int(self.region("status", torch.int32, (2,))[1].item())
        P = nb * self.moe.block_m
        sel = slice(0, P) if rows is None else rows
        H = sh.hidden
        cap = self.moe.layout["max_pool_blocks"] * self.moe.block_m
        px = self.tiled_rows("pool_x", H)[sel]
        psf = self.scales_rows("pool_sf", H // 128)[sel]
        pm = self.region("pool_meta", torch.int32, (cap, 3))[sel].cpu().numpy().view(np.uint32)
        return px, psf, pm

    def pool_dst_host(self):
        nb = int(self.region("status", torch.int32, (2,))[1].item())
        cap = self.moe.layout["max_pool_blocks"] * self.moe.block_m
        return self.region("pool_dst", torch.int32, (cap,))[:nb * self.moe.block_m].cpu().numpy().view(np.uint32)

    def l2_host(self, rows):
        sh = self.shape
        cap = self.moe.layout["max_pool_blocks"] * self.moe.block_m
        q = self.l2_rows(sh.intermediate)[rows]
        s = self.scales_rows("l2_sf", sh.intermediate // 128)[rows]
        return q, s

    def tiled_rows(self, name, width):
        """A tiled code region ([blocks][width/128][BM][128]) as [rows][width]."""
        nblk, bm = self.moe.layout["max_pool_blocks"], self.moe.block_m
        q = self.region(name, torch.uint8, (nblk, width // 128, bm, 128)).cpu().numpy()
        return np.ascontiguousarray(q.transpose(0, 2, 1, 3)).reshape(nblk * bm, width)

    def l2_rows(self, width):
        """The L2 pool ([blocks][width/128][4][BM][32]) as [rows][width]."""
        nblk, bm = self.moe.layout["max_pool_blocks"], self.moe.block_m
        q = self.region("l2_x", torch.uint8, (nblk, width // 128, 4, bm, 32)).cpu().numpy()
        return np.ascontiguousarray(q.transpose(0, 3, 1, 2, 4)).reshape(nblk * bm, width)

    def scales_rows(self, name, kb):
        """A block-major scale region ([blocks][kb][BM]) as [rows][kb]."""
        nblk, bm = self.moe.layout["max_pool_blocks"], self.moe.block_m
        s = self.region(name, torch.float32, (nblk, kb, bm)).cpu().numpy()
        return np.ascontiguousarray(s.transpose(0, 2, 1)).reshape(nblk * bm, kb)

    def comb_row(self, k, s, t):
        sh = self.shape
        plane = sh.num_shards * sh.max_tokens_per_shard
        c = self.region("comb", torch.int16, (sh.topk, plane, sh.hidden))
        return c[k, s * sh.max_tokens_per_shard + t].cpu().view(torch.bfloat16).to(torch.float64).numpy()

    def y_host(self, y=None):
        y = self.y if y is None else y
        return y.to(torch.float64).cpu().numpy()

    def close(self):
        self.moe.close()


def check_layout(run, inp_np, ref=None):
    """Counts, table, offsets, block list and the whole pool: bit-exact against the oracle.
    With a shared expert the offsets, block list and pool include its segment."""
    sh = run.shape
    nsh = getattr(sh, "num_shared_experts", 0)
    rt = oracle.route(inp_np["topk_idx"], inp_np["tokens_per_shard"], sh.num_experts,
                      sh.num_local_experts, sh.local_rank)
    got = run.layout_host()
    assert np.array_equal(got["send"], rt.send), "send counts"
    assert np.array_equal(got["recv"], rt.recv), "recv counts"
    assert np.array_equal(got["recv_tot"], rt.recv_tot), "recv_tot"
    px, psf, pm, off = oracle.fill_pool(inp_np["x"], inp_np["x_sf"], rt, run.moe.block_m, sh.topk,
                                        shared_shard=sh.local_rank if nsh else None,
                                        shared_tokens=inp_np["tokens_per_shard"][sh.local_rank] if nsh else 0)
    assert np.array_equal(off[:sh.num_local_experts + 1], oracle.pool_offsets(rt.recv_tot, run.moe.block_m))
    assert np.array_equal(got["pool_off"], off), "pool offsets"
    assert got["nblocks"] == off[-1]
    want_be = np.repeat(np.arange(len(off) - 1), np.diff(off))
    want_bi = np.concatenate([np.arange(n) for n in np.diff(off)]) if off[-1] else np.zeros(0, np.int64)
    assert np.array_equal(got["block_expert"], want_be), "block -> expert"
    assert np.array_equal(got["block_index"], want_bi), "block index in expert"
    for le in range(sh.num_local_experts):
        for s in range(sh.num_shards):
            n = rt.recv[le, s]
            assert np.array_equal(got["table"][le, s, :n], rt.table[le, s, :n]), ("table", le, s)
    gx, gsf, gm = run.pool_host()
    assert gx.shape == px.shape
    assert np.array_equal(gm, pm), "pool metadata"
    # scatter target of each pool row: comb row k*S*T_max + shard*T_max + token, padding all ones
    pad = pm[:, 0] == 0xFFFFFFFF
    want_dst = np.where(pad, np.uint64(0xFFFFFFFF),
                        (pm[:, 2].astype(np.uint64) * sh.num_shards + pm[:, 0]) * sh.max_tokens_per_shard + pm[:, 1])
    assert np.array_equal(run.pool_dst_host().astype(np.uint64), want_dst), "pool scatter targets"
    assert np.array_equal(gx, px), "pool rows"
    assert np.array_equal(gsf.view(np.uint32), psf.view(np.uint32)), "pool scales"
    return rt, off


def tol_check(got, want, what=""):
    """max|d| <= 2e-2 * max|ref| + 1e-3 over the compared elements."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - want).max() if got.size else 0.0
    bound = 2e-2 * np.abs(want).max() + 1e-3 if want.size else 1e-3
    assert d <= bound, f"{what}: max|d| {d:.4g} > {bound:.4g}"
    return d, bound


def sample_tokens(inp_np, shape, n, seed=0):
    """n valid (s, t) tokens with at least one local expert, plus a few with none."""
    rng = np.random.default_rng(seed)
    lo = shape.local_rank * shape.num_local_experts
    idx = inp_np["topk_idx"]
    cand = []
    for s in range(shape.num_shards):
        T = inp_np["tokens_per_shard"][s]
        loc = ((idx[s, :T] >= lo) & (idx[s, :T] < lo + shape.num_local_experts)).any(-1)
        cand += [(s, t, bool(loc[t])) for t in range(T)]
    with_local = [c for c in cand if c[2]]
    without = [c for c in cand if not c[2]]
    pick = [with_local[i] for i in rng.choice(len(with_local), min(n, len(with_local)), replace=False)]
    if without:
        pick += [without[i] for i in rng.choice(len(without), min(2, len(without)), replace=False)]
    return [(s, t) for s, t, _ in pick]


def inputs_np(run):
    return to_numpy(run.inp_gpu)
