// Routing work as device functions, shared by the routing kernels (route.hip) and the launch that routes,
// pulls and runs both GEMMs (gemm.hip).  The algorithm and its sources are described in route.hip.
#pragma once

#include "mm_internal.h"

namespace mm {

constexpr int kPerLane = kRouteChunk / 64;      // entries per lane of a routing wave
constexpr int kStageInts = 4096;                // recv counts a routing wave stages in LDS

// LDS written by some lanes of a wave is visible to all of them after this.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// The histogram over all E experts of chunk c of shard s, by all nthreads (>= 256) threads of a work-group
// (hist: E ints of LDS), written to chunk_hist.
__device__ __forceinline__ void route_count_chunk(const Params& p, int c, int s, int* hist, int tid, int nthreads) {
    for (int e = tid; e < p.E; e += nthreads) hist[e] = 0;
    __syncthreads();
    const long n = (long)p.tps[s] * p.K;
    const long f0 = (long)c * kRouteChunk;
    const int64_t* idx = p.topk_idx + (size_t)s * p.T_max * p.K;
    const long f = f0 + tid;
    const int64_t e = (tid < kRouteChunk && f < n) ? idx[f] : -1;
    bool bad = false;
    if (e >= p.E) bad = true;
    else if (e >= 0) atomicAdd(&hist[(int)e], 1);
    if (bad) atomicOr(p.status, MEGA_MOE_STATUS_BAD_EXPERT_ID);
    __syncthreads();
    int* out = p.chunk_hist + ((size_t)s * p.chunks + c) * p.E;
    for (int i = tid; i < p.E; i += nthreads) out[i] = hist[i];
    __syncthreads();     // hist is reused
}

// The nthreads threads of a work-group, for shard s: send[s][e] = sum over chunks; per local expert, the exclusive scan over
// chunks (first slot of each chunk) and recv[le][s].
__device__ __forceinline__ void route_scan_shard(const Params& p, int s, int tid, int nthreads) {
    const int lane = tid & 63, wave = tid >> 6;
    const int* hs = p.chunk_hist + (size_t)s * p.chunks * p.E;
    // send[s][e]: independent loads, summed in chunk order
    for (int e = tid; e < p.E; e += nthreads) {
        const int* h = hs + e;
        int sum = 0;
#pragma unroll 16
        for (int c = 0; c < p.chunks; ++c) sum += h[(size_t)c * p.E];
        p.send[(size_t)s * p.E + e] = sum;
    }
    // one wave per local expert: scan over chunks, lane = chunk, 64 at a time
    bool overflow = false;
    for (int le = wave; le < p.El; le += nthreads / 64) {
        const int* h = hs + p.lo + le;
        int* base = p.chunk_base + (size_t)s * p.chunks * p.El + le;
        int run = 0;
        for (int c0 = 0; c0 < p.chunks; c0 += 64) {
            const int c = c0 + lane;
            const int v = c < p.chunks ? h[(size_t)c * p.E] : 0;
            int incl = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int u = __shfl_up(incl, o);
                if (lane >= o) incl += u;
            }
            if (c < p.chunks) base[(size_t)c * p.El] = run + incl - v;
            run += __shfl(incl, 63);
        }
        if (lane == 0) {
            if (run > p.T_max) { overflow = true; run = p.T_max; }
            p.recv[(size_t)le * p.S + s] = run;
        }
    }
    if (overflow) atomicOr(p.status, MEGA_MOE_STATUS_SLOT_OVERFLOW);
}

// Pool layout from the counts ("Mega-MoE notes, part 2: index table and pull", 2.4: expert-major
// segments of ceil(recv_tot / BLOCK_M) blocks).  Every routing work-group (one wave) computes the
// offsets for itself in LDS with a wave prefix sum, so no launch sits between the scan and the table.
// offs[le] = first block of local expert le, offs[El] = end of the routed segments, offs[El + 1] = end
// of the shared expert's segment (the own shard's valid tokens; equal to offs[El] without one).
__device__ __forceinline__ void pool_layout(const Params& p, const int* recv_v, int* offs, int lane) {
    int carry = 0;
    for (int le0 = 0; le0 < p.El; le0 += 64) {
        const int le = le0 + lane;
        int nb = 0;
        if (le < p.El) {
            int tot = 0;
            for (int sp = 0; sp < p.S; ++sp) tot += recv_v[le * p.S + sp];
            nb = (tot + p.BM - 1) / p.BM;
        }
        int x = nb;                                  // inclusive prefix sum over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        if (le < p.El) offs[le] = carry + x - nb;
        carry += __shfl(x, 63);
    }
    if (lane == 0) {
        const int n_own = p.nsh ? p.tps[p.own] : 0;
        offs[p.El] = carry;
        offs[p.El + 1] = carry + (n_own + p.BM - 1) / p.BM;
    }
}

// Written once per forward (by the first routing work-group): recv_tot, the cumulative statistics, the
// offsets, the block count and the block list.  With a shared expert, its segment follows the routed
// ones: the valid tokens of the own shard in order, with top-k slot K ("DeepGEMM Mega MoE symmetric
// memory deep analysis", 4.1: the shared expert reads the rank's own input buffer; 8.2: its output
// takes the extra combine slot K); its metadata and scatter targets are written here too.
__device__ __forceinline__ void pool_publish(const Params& p, const int* recv_v, const int* offs, int lane) {
    for (int le = lane; le < p.El; le += 64) {
        int tot = 0;
        for (int sp = 0; sp < p.S; ++sp) tot += recv_v[le * p.S + sp];
        p.recv_tot[le] = tot;
        if (p.cum) p.cum[le] += tot;
    }
    for (int i = lane; i <= p.El + 1; i += 64) p.pool_off[i] = offs[i];
    if (lane == 0) p.status[1] = (uint32_t)offs[p.El + 1];
    const int nseg = p.El + p.nsh;                   // pool segments: routed experts, then the shared one
    const int nb = min(offs[nseg], p.max_blocks);    // never below offs[nseg]: the pool holds every row
    for (int b = lane; b < nb; b += 64) {
        int lo = 0, hi = nseg;            // last segment with offs[le] <= b: the non-empty owner of b
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (offs[mid] <= b) lo = mid; else hi = mid;
        }
        p.block_expert[b] = lo;
        p.block_index[b] = b - offs[lo];
    }
    if (p.nsh) {
        // row off*BM + t holds token t of the own shard, k = K; the rest of the last block is padding
        const int n_own = p.tps[p.own];
        const size_t r0 = (size_t)offs[p.El] * p.BM;
        const size_t r1 = min((size_t)offs[p.El + 1] * p.BM, (size_t)p.max_blocks * p.BM);
        for (size_t r = r0 + lane; r < r1; r += 64) {
            const int t = (int)(r - r0);
            const bool ok = t < n_own;
            p.pool_meta[r * 3] = ok ? (uint32_t)p.own : kMetaPad;
            p.pool_meta[r * 3 + 1] = ok ? (uint32_t)t : kMetaPad;
            p.pool_meta[r * 3 + 2] = ok ? (uint32_t)p.K : kMetaPad;
            p.pool_dst[r] = ok ? (uint32_t)(((size_t)p.K * p.S + p.own) * p.T_max + t) : kMetaPad;
        }
    }
}

// kRegRun: with at most 64 local experts the running slot of expert L lives in lane L's register (read
// with a uniform readlane), otherwise in LDS.
//
// Every table entry is also placed straight into its pool row, so the fill needs no table walk.  The
// round-robin order ("Mega-MoE notes, part 2: index table and pull", 2.5) puts slot q of shard s of
// expert le after every slot below q of every shard, and after the shards s' < s that still hold a slot
// at q: with c[s'] = recv[le][s'],
//     j(s, q) = sum over s' of min(c[s'], q)  +  #{s' < s : c[s'] > q}.
// (Round r of the min-peeling covers the slots between two consecutive distinct counts, and the shards
// active in it are exactly those whose count exceeds the slot.)  The row gets the metadata {s, t, k} and
// the GEMM2 scatter target k*S*T_max + s*T_max + t; the padding rows of each expert get all ones from
// one work-group.  recv is staged in LDS when it fits (kStageInts), else read from global memory
// through the same generic pointer; the pool offsets are computed from it (pool_layout).

// One wave's share: chunk c of shard s.  run, stage and offs are LDS of the wave's own (run: E_l ints
// unless kRegRun, stage: stage_ints ints, offs: E_l + 2 ints); recv is staged there when it fits.
template <bool kRegRun>
__device__ __forceinline__ void route_table_chunk(const Params& p, int c, int s, int lane, int* run, int* stage,
                                                  int* offs, int stage_ints = kStageInts) {
    const int* base = p.chunk_base + ((size_t)s * p.chunks + c) * p.El;
    const long n = (long)p.tps[s] * p.K;
    const long f0 = (long)c * kRouteChunk;
    const int64_t* idx = p.topk_idx + (size_t)s * p.T_max * p.K;
    // the chunk's expert ids first, so that their loads overlap the staging below
    int64_t e_of[kPerLane];
#pragma unroll
    for (int r = 0; r < kPerLane; ++r) {
        const long f = f0 + r * 64 + lane;
        e_of[r] = f < n ? idx[f] : -1;
    }
    // (E_l <= 64) the chunk's slot bases, one per lane: issued with the ids, so their latency overlaps
    int run_reg = 0;
    if (kRegRun) run_reg = lane < p.El ? base[lane] : 0;
    const bool staged = p.El * p.S <= stage_ints;
    const int* recv_v = p.recv;
    if (staged) {
        // up to 8 loads per lane in flight per round (one round for the usual El*S)
        const int nr = p.El * p.S;
        for (int i0 = 0; i0 < nr; i0 += 64 * 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * 64 + lane;
                v[u] = i < nr ? p.recv[i] : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * 64 + lane;
                if (i < nr) stage[i] = v[u];
            }
        }
        recv_v = stage;
        wave_lds_sync();
    }
    pool_layout(p, recv_v, offs, lane);
    const int* off_v = offs;
    if (!kRegRun) {
        for (int le = lane; le < p.El; le += 64) run[le] = base[le];
    }
    wave_lds_sync();
    if (c == 0 && s == 0) pool_publish(p, recv_v, offs, lane);
    // padding rows of the experts this work-group owns (le = its index, then every chunks*S further):
    // metadata and scatter target all ones
    const size_t cap_rows = (size_t)p.max_blocks * p.BM;
    for (int le = s * p.chunks + c; le < p.El; le += p.chunks * p.S) {
        int tot = 0;
        for (int sp = 0; sp < p.S; ++sp) tot += recv_v[le * p.S + sp];
        const size_t r1 = min((size_t)off_v[le + 1] * p.BM, cap_rows);
        for (size_t r = (size_t)off_v[le] * p.BM + tot + lane; r < r1; r += 64) {
            p.pool_meta[r * 3] = kMetaPad;
            p.pool_meta[r * 3 + 1] = kMetaPad;
            p.pool_meta[r * 3 + 2] = kMetaPad;
            p.pool_dst[r] = kMetaPad;
        }
    }
    int le_of[kPerLane];
#pragma unroll
    for (int r = 0; r < kPerLane; ++r)
        le_of[r] = (e_of[r] >= p.lo && e_of[r] < p.lo + p.El) ? (int)(e_of[r] - p.lo) : -1;
    const size_t plane = (size_t)p.S * p.T_max;      // table stride between local experts
    int* tab = p.table + (size_t)s * p.T_max;
    bool overflow = false;
    int slot_of[kPerLane];
#pragma unroll
    for (int r = 0; r < kPerLane; ++r) {
        const int le = le_of[r];
        const int f = (int)(f0 + r * 64 + lane);
        slot_of[r] = p.T_max;
        uint64_t pending = __ballot(le >= 0);
        while (pending) {                                 // one pass per distinct expert in the wave
            const int leader = __ffsll((unsigned long long)pending) - 1;
            const int L = __builtin_amdgcn_readlane(le, leader);
            const uint64_t m = __ballot(le == L);
            const int b0 = kRegRun ? __builtin_amdgcn_readlane(run_reg, L) : run[L];
            if (le == L) {
                const int slot = b0 + __popcll(m & lanemask_lt());
                if (slot < p.T_max) {
                    tab[(size_t)L * plane + slot] = f;
                    slot_of[r] = slot;
                } else {
                    overflow = true;
                }
            }
            if (kRegRun) {
                if (lane == L) run_reg = b0 + __popcll(m);
            } else if (lane == leader) {
                run[L] = b0 + __popcll(m);
            }
            pending &= ~m;
        }
    }
    bool bad = false;
#pragma unroll
    for (int r = 0; r < kPerLane; ++r) {
        const int le = le_of[r], q = slot_of[r];
        if (le < 0 || q >= p.T_max) continue;
        const int* cnt = recv_v + le * p.S;
        int j = 0;
        int sp = 0;
        for (; sp + 4 <= p.S; sp += 4) {               // four independent reads at a time
            const int c0 = cnt[sp], c1 = cnt[sp + 1], c2 = cnt[sp + 2], c3 = cnt[sp + 3];
            j += min(c0, q) + min(c1, q) + min(c2, q) + min(c3, q);
            j += (sp < s && c0 > q) + (sp + 1 < s && c1 > q) + (sp + 2 < s && c2 > q) + (sp + 3 < s && c3 > q);
        }
        for (; sp < p.S; ++sp) {
            const int cs = cnt[sp];
            j += min(cs, q) + (sp < s && cs > q ? 1 : 0);
        }
        const size_t row = (size_t)off_v[le] * p.BM + j;
        if (row >= cap_rows) { bad = true; continue; }   // unreachable: the pool holds every routed row
        const int f = (int)(f0 + r * 64 + lane);
        const int t = f / p.K, k = f - t * p.K;
        uint32_t* meta = p.pool_meta + row * 3;
        meta[0] = (uint32_t)s;
        meta[1] = (uint32_t)t;
        meta[2] = (uint32_t)k;
        p.pool_dst[row] = (uint32_t)(((size_t)k * p.S + s) * p.T_max + t);
    }
    // An entry that found no slot is dropped, as the oracle drops it: GEMM2 never writes its combine row,
    // so that row is zeroed here and the combine adds nothing for the entry.
    if (overflow) {
#pragma unroll
        for (int r = 0; r < kPerLane; ++r) {
            if (le_of[r] < 0 || slot_of[r] < p.T_max) continue;
            const int f = (int)(f0 + r * 64 + lane);
            const int t = f / p.K, k = f - t * p.K;
            uint4* row = reinterpret_cast<uint4*>(p.comb + (((size_t)k * p.S + s) * p.T_max + t) * p.H);
            for (int c = 0; c < (p.H >> 3); ++c) row[c] = uint4{0u, 0u, 0u, 0u};
        }
        atomicOr(p.status, MEGA_MOE_STATUS_SLOT_OVERFLOW);
    }
    if (bad) atomicOr(p.status, MEGA_MOE_STATUS_BAD_LAYOUT);
}

}  // namespace mm
