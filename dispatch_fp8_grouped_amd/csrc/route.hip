// Routing metadata: per-expert send counts, the [local_expert][source_shard][slot] index table, the
// expert-major pool offsets and the pool block list.
//
// The pages count with shared-memory atomics and claim slots with a global 64-bit atomic per SM
// ("Mega-MoE kernel code walkthrough: from Dispatch to WGMMA", 4.2), which makes the slot order
// depend on timing.  Here the same counting sort ("Dispatch/Combine: blog theory vs DeepEP vs DeepGEMM
// Mega MoE", 4.4: count, prefix sum, scatter) is done deterministically: slots of one (expert, shard)
// follow ascending t*K+k.  Three launches (one, route_small, for inputs whose counts fit in LDS; two,
// with route_count_scan in place of the first two, for shards of at most 8 chunks):
//   route_count  grid (chunks, S): LDS histogram of one chunk of 256 (token, k) entries over all E
//   route_scan   grid S:           send[s][e], per-chunk slot bases, recv
//   route_table  grid (chunks, S), one wave each: the pool offsets from recv ("Mega-MoE notes, part 2:
//                index table and pull", 2.4; the first work-group also writes recv_tot, the offsets,
//                the block count and the block list), then a stable in-wave ranking by
//                ballot/popcount that writes table[le][s][slot] = t*K+k (same page, 1.1-1.3) and the
//                entry's pool row metadata and GEMM2 scatter target (its round-robin position, 2.5),
//                padding rows
#include "route_impl.h"

namespace mm {
namespace {

constexpr int kCountThreads = 256;

__global__ __launch_bounds__(kCountThreads) void route_count_kernel(Params p) {
    extern __shared__ int hist[];   // [E]
    route_count_chunk(p, blockIdx.x, blockIdx.y, hist, threadIdx.x, kCountThreads);
}

// One work-group per shard.
__global__ __launch_bounds__(1024) void route_scan_kernel(Params p) { route_scan_shard(p, blockIdx.x, threadIdx.x, 1024); }

// Counts and scan in one launch, for shards of at most a few chunks (decode): one work-group per shard
// histograms kFusedChunks chunks at a time (256 threads per chunk, one LDS histogram each), writes them
// to chunk_hist, and after a barrier (the same work-group reads them back) runs the scan.  Saves the
// count launch where its 4 us and the launch gap are a tenth of the routing.
constexpr int kFusedChunks = 4;
constexpr int kFusedMaxChunks = 8;
__global__ __launch_bounds__(1024) void route_count_scan_kernel(Params p) {
    extern __shared__ int hist[];   // [kFusedChunks][E]
    const int s = blockIdx.x, tid = threadIdx.x;
    const long n = (long)p.tps[s] * p.K;
    const int64_t* idx = p.topk_idx + (size_t)s * p.T_max * p.K;
    bool bad = false;
    for (int c0 = 0; c0 < p.chunks; c0 += kFusedChunks) {
        for (int i = tid; i < kFusedChunks * p.E; i += 1024) hist[i] = 0;
        __syncthreads();
        const int j = tid / kRouteChunk, c = c0 + j;
        const long f = (long)c * kRouteChunk + (tid % kRouteChunk);
        const int64_t e = (c < p.chunks && f < n) ? idx[f] : -1;
        if (e >= p.E) bad = true;
        else if (e >= 0) atomicAdd(&hist[j * p.E + (int)e], 1);
        __syncthreads();
        for (int i = tid; i < kFusedChunks * p.E; i += 1024) {
            const int cc = c0 + i / p.E;
            if (cc < p.chunks) p.chunk_hist[((size_t)s * p.chunks + cc) * p.E + i % p.E] = hist[i];
        }
        __syncthreads();
    }
    if (bad) atomicOr(p.status, MEGA_MOE_STATUS_BAD_EXPERT_ID);
    route_scan_shard(p, s, tid, 1024);
}
static_assert(kFusedChunks * kRouteChunk == 1024, "one thread per entry of kFusedChunks chunks");

// One wave per (chunk, shard).
template <bool kRegRun>
__global__ __launch_bounds__(64) void route_table_kernel(Params p) {
    __shared__ int run[kRegRun ? 1 : MEGA_MOE_MAX_LOCAL_EXPERTS];
    __shared__ int stage[kStageInts];
    __shared__ int offs[MEGA_MOE_MAX_LOCAL_EXPERTS + 2];
    route_table_chunk<kRegRun>(p, blockIdx.x, blockIdx.y, threadIdx.x, run, stage, offs);
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
    hipError_t err;
    if (p.chunks <= kFusedMaxChunks && !(p.flags & MEGA_MOE_FLAG_DEBUG_ROUTE_LAUNCHES)) {
        hipLaunchKernelGGL(route_count_scan_kernel, dim3(p.S), dim3(1024), kFusedChunks * p.E * sizeof(int), stream, p);
    } else {
        hipLaunchKernelGGL(route_count_kernel, grid, dim3(kCountThreads), p.E * sizeof(int), stream, p);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(route_scan_kernel, dim3(p.S), dim3(1024), 0, stream, p);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (p.El <= 64) hipLaunchKernelGGL(route_table_kernel<true>, grid, dim3(64), 0, stream, p);
    else hipLaunchKernelGGL(route_table_kernel<false>, grid, dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mm
