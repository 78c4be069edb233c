// Routing metadata: per-expert send counts, the [local_expert][source_shard][slot] index table, the
// expert-major pool offsets and the pool block list.
//
// The pages count with shared-memory atomics and claim slots with a global 64-bit atomic per SM
// ("Mega-MoE kernel code walkthrough: from Dispatch to WGMMA", 4.2), which makes the slot order
// depend on timing.  Here the same counting sort ("Dispatch/Combine: blog theory vs DeepEP vs DeepGEMM
// Mega MoE", 4.4: count, prefix sum, scatter) is done deterministically: slots of one (expert, shard)
// follow ascending t*K+k.  Three launches:
//   route_count  grid (chunks, S): LDS histogram of one chunk of 2048 (token, k) entries over all E
//   route_scan   one work-group:   send[s][e], per-chunk slot bases, recv, recv_tot, pool offsets
//                                  ("Mega-MoE notes, part 2: index table and pull", 2.4), block list
//   route_table  grid (chunks, S), one wave each: stable in-wave ranking by ballot/popcount, writes
//                table[le][s][slot] = t*K+k ("Mega-MoE notes, part 2", 1.1-1.3)
#include "mm_internal.h"

namespace mm {
namespace {

constexpr int kCountThreads = 256;
constexpr int kPerThread = kRouteChunk / kCountThreads;   // 8
constexpr int kPerLane = kRouteChunk / 64;                // 32

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

__global__ __launch_bounds__(1024) void route_scan_kernel(Params p) {
    __shared__ int s_tot[MEGA_MOE_MAX_LOCAL_EXPERTS];
    __shared__ int s_off[MEGA_MOE_MAX_LOCAL_EXPERTS + 1];
    const int tid = threadIdx.x;
    // send[s][e] = sum over chunks
    for (int i = tid; i < p.S * p.E; i += 1024) {
        const int s = i / p.E, e = i - s * p.E;
        const int* h = p.chunk_hist + (size_t)s * p.chunks * p.E + e;
        int sum = 0;
        for (int c = 0; c < p.chunks; ++c) sum += h[(size_t)c * p.E];
        p.send[i] = sum;
    }
    // per (local expert, shard): exclusive scan over chunks -> first slot of each chunk; recv
    bool overflow = false;
    for (int i = tid; i < p.El * p.S; i += 1024) {
        const int le = i / p.S, s = i - le * p.S;
        const int* h = p.chunk_hist + (size_t)s * p.chunks * p.E + p.lo + le;
        int* base = p.chunk_base + (size_t)s * p.chunks * p.El + le;
        int run = 0;
        for (int c = 0; c < p.chunks; ++c) {
            base[(size_t)c * p.El] = run;
            run += h[(size_t)c * p.E];
        }
        if (run > p.T_max) { overflow = true; run = p.T_max; }
        p.recv[i] = run;   // recv[le][s]
    }
    if (overflow) atomicOr(p.status, MEGA_MOE_STATUS_SLOT_OVERFLOW);
    __syncthreads();
    for (int le = tid; le < p.El; le += 1024) {
        int t = 0;
        for (int s = 0; s < p.S; ++s) t += p.recv[le * p.S + s];
        s_tot[le] = t;
        p.recv_tot[le] = t;
        if (p.cum) p.cum[le] += t;
    }
    __syncthreads();
    if (tid == 0) {
        int o = 0;
        for (int le = 0; le < p.El; ++le) {
            s_off[le] = o;
            p.pool_off[le] = o;
            o += (s_tot[le] + p.BM - 1) / p.BM;
        }
        s_off[p.El] = o;
        p.pool_off[p.El] = o;
        p.status[1] = (uint32_t)o;
    }
    __syncthreads();
    const int nb = s_off[p.El];
    for (int b = tid; b < nb; b += 1024) {
        int lo = 0, hi = p.El;            // last le with s_off[le] <= b: the non-empty owner of b
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_off[mid] <= b) lo = mid; else hi = mid;
        }
        p.block_expert[b] = lo;
        p.block_index[b] = b - s_off[lo];
    }
}

__global__ __launch_bounds__(64) void route_table_kernel(Params p) {
    __shared__ int run[MEGA_MOE_MAX_LOCAL_EXPERTS];
    const int c = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
    const int* base = p.chunk_base + ((size_t)s * p.chunks + c) * p.El;
    for (int le = lane; le < p.El; le += 64) run[le] = base[le];
    __syncthreads();
    const long n = (long)p.tps[s] * p.K;
    const long f0 = (long)c * kRouteChunk;
    const int64_t* idx = p.topk_idx + (size_t)s * p.T_max * p.K;
    // load the whole chunk first so that the 32 loads are in flight together
    int le_of[kPerLane];
#pragma unroll
    for (int r = 0; r < kPerLane; ++r) {
        const long f = f0 + r * 64 + lane;
        const int64_t e = f < n ? idx[f] : -1;
        le_of[r] = (e >= p.lo && e < p.lo + p.El) ? (int)(e - p.lo) : -1;
    }
    const size_t plane = (size_t)p.S * p.T_max;      // table stride between local experts
    int* tab = p.table + (size_t)s * p.T_max;
    bool overflow = false;
#pragma unroll
    for (int r = 0; r < kPerLane; ++r) {
        const int le = le_of[r];
        const int f = (int)(f0 + r * 64 + lane);
        uint64_t pending = __ballot(le >= 0);
        while (pending) {                                 // one pass per distinct expert in the wave
            const int leader = __ffsll((unsigned long long)pending) - 1;
            const int L = __shfl(le, leader);
            const uint64_t m = __ballot(le == L);
            const int b0 = run[L];
            if (le == L) {
                const int slot = b0 + __popcll(m & lanemask_lt());
                if (slot < p.T_max) tab[(size_t)L * plane + slot] = f;
                else overflow = true;
            }
            if (lane == leader) run[L] = b0 + __popcll(m);
            pending &= ~m;
        }
    }
    if (overflow) atomicOr(p.status, MEGA_MOE_STATUS_SLOT_OVERFLOW);
}

}  // namespace

hipError_t launch_route(const Params& p, hipStream_t stream) {
    dim3 grid(p.chunks, p.S);
    hipLaunchKernelGGL(route_count_kernel, grid, dim3(kCountThreads), p.E * sizeof(int), stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_table_kernel, grid, dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mm
