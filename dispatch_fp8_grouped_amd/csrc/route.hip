// Routing metadata: per-expert send counts, the [local_expert][source_shard][slot] index table, the
// expert-major pool offsets and the pool block list.
//
// The pages count with shared-memory atomics and claim slots with a global 64-bit atomic per SM
// ("Mega-MoE kernel code walkthrough: from Dispatch to WGMMA", 4.2), which makes the slot order
// depend on timing.  Here the same counting sort ("Dispatch/Combine: blog theory vs DeepEP vs DeepGEMM
// Mega MoE", 4.4: count, prefix sum, scatter) is done deterministically: slots of one (expert, shard)
// follow ascending t*K+k.  Three launches (one, route_small, for inputs whose counts fit in LDS):
//   route_count  grid (chunks, S): LDS histogram of one chunk of 256 (token, k) entries over all E
//   route_scan   grid S:           send[s][e], per-chunk slot bases, recv
//   route_table  grid (chunks, S), one wave each: the pool offsets from recv ("Mega-MoE notes, part 2:
//                index table and pull", 2.4; the first work-group also writes recv_tot, the offsets,
//                the block count and the block list), then a stable in-wave ranking by
//                ballot/popcount that writes table[le][s][slot] = t*K+k (same page, 1.1-1.3) and the
//                entry's pool row metadata and GEMM2 scatter target (its round-robin position, 2.5),
//                padding rows
#include "mm_internal.h"

namespace mm {
namespace {

constexpr int kCountThreads = 256;
constexpr int kPerThread = kRouteChunk / kCountThreads;   // 1
constexpr int kPerLane = kRouteChunk / 64;                // 4

__global__ __launch_bounds__(kCountThreads) void route_count_kernel(Params p) {
    extern __shared__ int hist[];   // [E]
    const int c = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
    for (int e = tid; e < p.E; e += kCountThreads) hist[e] = 0;
    __syncthreads();
    const long n = (long)p.tps[s] * p.K;
    const long f0 = (long)c * kRouteChunk;
    const int64_t* idx = p.topk_idx + (size_t)s * p.T_max * p.K;
    int64_t e[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const long f = f0 + tid + i * kCountThreads;
        e[i] = f < n ? idx[f] : -1;
    }
    bool bad = false;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        if (e[i] >= p.E) bad = true;
        else if (e[i] >= 0) atomicAdd(&hist[(int)e[i]], 1);
    }
    if (bad) atomicOr(p.status, MEGA_MOE_STATUS_BAD_EXPERT_ID);
    __syncthreads();
    int* out = p.chunk_hist + ((size_t)s * p.chunks + c) * p.E;
    for (int i = tid; i < p.E; i += kCountThreads) out[i] = hist[i];
}

// One work-group per shard s: send[s][e] = sum over chunks; per local expert, the exclusive scan over
// chunks (first slot of each chunk) and recv[le][s].
__global__ __launch_bounds__(1024) void route_scan_kernel(Params p) {
    const int s = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int* hs = p.chunk_hist + (size_t)s * p.chunks * p.E;
    // send[s][e]: independent loads, summed in chunk order
    for (int e = tid; e < p.E; e += 1024) {
        const int* h = hs + e;
        int sum = 0;
#pragma unroll 16
        for (int c = 0; c < p.chunks; ++c) sum += h[(size_t)c * p.E];
        p.send[(size_t)s * p.E + e] = sum;
    }
    // one wave per local expert: scan over chunks, lane = chunk, 64 at a time
    bool overflow = false;
    for (int le = wave; le < p.El; le += 1024 / 64) {
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
constexpr int kStageInts = 4096;

template <bool kRegRun>
__global__ __launch_bounds__(64) void route_table_kernel(Params p) {
    __shared__ int run[kRegRun ? 1 : MEGA_MOE_MAX_LOCAL_EXPERTS];
    __shared__ int stage[kStageInts];
    __shared__ int offs[MEGA_MOE_MAX_LOCAL_EXPERTS + 2];
    const int c = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
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
    const bool staged = p.El * p.S <= kStageInts;
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
        __syncthreads();
    }
    pool_layout(p, recv_v, offs, lane);
    const int* off_v = offs;
    int run_reg = 0;
    if (kRegRun) {
        run_reg = lane < p.El ? base[lane] : 0;
    } else {
        for (int le = lane; le < p.El; le += 64) run[le] = base[le];
    }
    __syncthreads();
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

// ---------------------------------------------------------------- small inputs: one work-group
// The same outputs for inputs small enough that every count fits in LDS (decode-sized batches), in one
// launch of 16 waves instead of three launches: the three stages above are latency-bound there.
// Entries are taken in groups of 64 consecutive (token, k) entries of one shard; group g of shard s
// covers entries [64g, 64g + 64) of that shard.  Slots of one (expert, shard) still follow ascending
// t*K+k: a group's entries of expert le start at the sum of the earlier groups' counts of le.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int kSmallSend = 8192;     // S*E counters
constexpr int kSmallGroupCnt = 8192; // groups * El counters
constexpr int kSmallRecv = 4096;     // El*S counts
constexpr int kBatch = 8;            // groups whose loads a wave issues together

__global__ __launch_bounds__(kSmallThreads) void route_small_kernel(Params p) {
    __shared__ int send_l[kSmallSend];          // [s][e]
    __shared__ int grp_l[kSmallGroupCnt];       // [s][g][le]: count, then the group's first slot
    __shared__ int recv_l[kSmallRecv];          // [le][s]
    __shared__ int offs[MEGA_MOE_MAX_LOCAL_EXPERTS + 2];
    __shared__ int flags;                       // bit 0 bad expert id, bit 1 slot overflow
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = p.S, E = p.E, El = p.El, K = p.K;
    const int G = (p.T_max * K + 63) >> 6;      // groups per shard
    for (int i = tid; i < S * E; i += kSmallThreads) send_l[i] = 0;
    for (int i = tid; i < S * G * El; i += kSmallThreads) grp_l[i] = 0;
    if (tid == 0) flags = 0;
    __syncthreads();
    // A wave takes groups q = wave + 16i, kBatch of them per batch with all their loads issued first.
    const int NQ = S * G;
    auto load_batch = [&](int q0, int64_t (&ev)[kBatch]) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int q = q0 + i * kSmallWaves;
            ev[i] = -1;
            if (q < NQ) {
                const int s = q / G, g = q - s * G;
                const long f = (long)g * 64 + lane;
                if (f < (long)p.tps[s] * K) ev[i] = p.topk_idx[(size_t)s * p.T_max * K + f];
            }
        }
    };
    // count: the global expert histogram of each shard, and each group's count per local expert
    for (int q0 = wave; q0 < NQ; q0 += kBatch * kSmallWaves) {
      int64_t ev[kBatch];
      load_batch(q0, ev);
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int q = q0 + i * kSmallWaves;
        if (q >= NQ) break;
        const int s = q / G;
        const int64_t e = ev[i];
        if (e >= E) atomicOr(&flags, 1);
        else if (e >= 0) atomicAdd(&send_l[s * E + (int)e], 1);
        const int le = (e >= p.lo && e < p.lo + El) ? (int)(e - p.lo) : -1;
        uint64_t pending = __ballot(le >= 0);
        while (pending) {
            const int L = __builtin_amdgcn_readlane(le, __ffsll((unsigned long long)pending) - 1);
            const uint64_t m = __ballot(le == L);
            if (lane == 0) grp_l[q * El + L] = __popcll(m);
            pending &= ~m;
        }
      }
    }
    __syncthreads();
    // per (shard, local expert): exclusive scan over the shard's groups, and recv[le][s] (at most T_max)
    for (int i = tid; i < S * El; i += kSmallThreads) {
        const int s = i / El, le = i - s * El;
        int run = 0;
        for (int g = 0; g < G; ++g) {
            int* c = &grp_l[(s * G + g) * El + le];
            const int v = *c;
            *c = run;
            run += v;
        }
        if (run > p.T_max) { atomicOr(&flags, 2); run = p.T_max; }
        recv_l[le * S + s] = run;
        p.recv[(size_t)le * S + s] = run;
    }
    for (int i = tid; i < S * E; i += kSmallThreads) p.send[i] = send_l[i];
    __syncthreads();
    if (wave == 0) {
        pool_layout(p, recv_l, offs, lane);
        pool_publish(p, recv_l, offs, lane);
    }
    __syncthreads();
    // padding rows of every expert: metadata and scatter target all ones
    const size_t cap_rows = (size_t)p.max_blocks * p.BM;
    for (int le = wave; le < El; le += kSmallWaves) {
        int tot = 0;
        for (int sp = 0; sp < S; ++sp) tot += recv_l[le * S + sp];
        const size_t r1 = min((size_t)offs[le + 1] * p.BM, cap_rows);
        for (size_t r = (size_t)offs[le] * p.BM + tot + lane; r < r1; r += 64) {
            p.pool_meta[r * 3] = kMetaPad;
            p.pool_meta[r * 3 + 1] = kMetaPad;
            p.pool_meta[r * 3 + 2] = kMetaPad;
            p.pool_dst[r] = kMetaPad;
        }
    }
    // ranking, table and pool rows, one group per wave at a time
    const size_t plane = (size_t)S * p.T_max;
    bool overflow = false, bad = false;
    for (int q0 = wave; q0 < NQ; q0 += kBatch * kSmallWaves) {
      int64_t ev[kBatch];
      load_batch(q0, ev);
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int q = q0 + i * kSmallWaves;
        if (q >= NQ) break;
        const int s = q / G, g = q - s * G;
        const int f = g * 64 + lane;
        const int64_t e = ev[i];
        const int le = (e >= p.lo && e < p.lo + El) ? (int)(e - p.lo) : -1;
        int slot = p.T_max;
        uint64_t pending = __ballot(le >= 0);
        while (pending) {
            const int L = __builtin_amdgcn_readlane(le, __ffsll((unsigned long long)pending) - 1);
            const uint64_t m = __ballot(le == L);
            if (le == L) slot = grp_l[q * El + L] + __popcll(m & lanemask_lt());
            pending &= ~m;
        }
        if (le < 0) continue;
        const int t = f / K, k = f - t * K;
        if (slot >= p.T_max) {
            // dropped, as the oracle drops it: its combine row is zeroed so the combine adds nothing
            overflow = true;
            uint4* row = reinterpret_cast<uint4*>(p.comb + (((size_t)k * S + s) * p.T_max + t) * p.H);
            for (int c = 0; c < (p.H >> 3); ++c) row[c] = uint4{0u, 0u, 0u, 0u};
            continue;
        }
        p.table[(size_t)le * plane + (size_t)s * p.T_max + slot] = f;
        // round-robin position (see route_table_kernel)
        const int* cnt = recv_l + le * S;
        int j = 0;
        for (int sp = 0; sp < S; ++sp) {
            const int cs = cnt[sp];
            j += min(cs, slot) + (sp < s && cs > slot ? 1 : 0);
        }
        const size_t row = (size_t)offs[le] * p.BM + j;
        if (row >= cap_rows) { bad = true; continue; }
        uint32_t* meta = p.pool_meta + row * 3;
        meta[0] = (uint32_t)s;
        meta[1] = (uint32_t)t;
        meta[2] = (uint32_t)k;
        p.pool_dst[row] = (uint32_t)(((size_t)k * S + s) * p.T_max + t);
      }
    }
    if (overflow) atomicOr(&flags, 2);
    if (bad) atomicOr(p.status, MEGA_MOE_STATUS_BAD_LAYOUT);
    __syncthreads();
    if (tid == 0) {
        if (flags & 1) atomicOr(p.status, MEGA_MOE_STATUS_BAD_EXPERT_ID);
        if (flags & 2) atomicOr(p.status, MEGA_MOE_STATUS_SLOT_OVERFLOW);
    }
}

// The one-work-group path takes inputs whose counts fit its LDS arrays and that give each wave at most
// two groups: there it beats three launches (tiny layer, 128 entries: 39 -> 33 us per forward).  At the
// decode size (8192 entries, 8 groups per wave) its serial steps cost more than the launches save
// (route 33 us against 20 us), so decode keeps the three-launch routing.
bool route_small_fits(const Params& p) {
    const long G = ((long)p.T_max * p.K + 63) / 64;
    return (long)p.S * G <= 2 * kSmallWaves && (long)p.S * p.E <= kSmallSend &&
           (long)p.S * G * p.El <= kSmallGroupCnt && (long)p.El * p.S <= kSmallRecv;
}

}  // namespace

hipError_t launch_route(const Params& p, hipStream_t stream) {
    if (route_small_fits(p) && !(p.flags & MEGA_MOE_FLAG_DEBUG_ROUTE_LAUNCHES)) {
        hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(kSmallThreads), 0, stream, p);
        return hipGetLastError();
    }
    dim3 grid(p.chunks, p.S);
    hipLaunchKernelGGL(route_count_kernel, grid, dim3(kCountThreads), p.E * sizeof(int), stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_scan_kernel, dim3(p.S), dim3(1024), 0, stream, p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (p.El <= 64) hipLaunchKernelGGL(route_table_kernel<true>, grid, dim3(64), 0, stream, p);
    else hipLaunchKernelGGL(route_table_kernel<false>, grid, dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mm
