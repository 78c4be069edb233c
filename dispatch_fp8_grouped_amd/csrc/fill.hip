// Pool fill: the receiver-side pull of routed FP8 rows into the expert-major L1 pool.
//
// Pool row off[le]*BM + j (j = position inside local expert le) is resolved to a source shard and slot
// by the min-peeling round-robin ("DeepGEMM Mega MoE symmetric memory deep analysis", 7.5; "Mega-MoE
// notes, part 2: index table and pull", 2.5): every round takes L = the smallest remaining count over
// the sources that still have rows, each such source gives L slots, and positions inside a round
// alternate between the active sources in ascending order.  One lane per source runs the rounds with
// wave ballots and a wave-wide minimum.  The table entry t*K+k at (le, source, slot) names the token;
// its H-byte row (into the tiled pool), its H/128 scales and the metadata {shard, token, k} are copied
// ("Mega-MoE notes, part 2", 2.6; "Dispatch/Combine ... comparison", 6.2), with the row's GEMM2
// scatter target k*S*T_max + shard*T_max + token beside them.  Rows past the expert's count are
// padding: zero codes, zero scales, metadata and target all ones.
//
// One wave per pool row, 16-byte loads and stores, all loads of a pass issued before its stores; the
// kernel stays within 64 VGPRs so 8 waves per SIMD keep many rows in flight.
#include "mm_internal.h"

namespace mm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kFillThreads = 256;
constexpr int kUnroll = 2;   // 16-byte chunks per lane per pass: the kernel fits 8 waves per SIMD

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

__global__ __launch_bounds__(kFillThreads, 8) void fill_kernel(Params p) {
    const int lane = threadIdx.x & 63;
    const long wave0 = (long)blockIdx.x * (kFillThreads / 64) + (threadIdx.x >> 6);
    const long nwaves = (long)gridDim.x * (kFillThreads / 64);
    const long rows = (long)min((int)p.status[1], p.max_blocks) * p.BM;
    const int H16 = p.H >> 4;
    const int SF = p.H >> 7;
    for (long row = wave0; row < rows; row += nwaves) {
        const int b = (int)(row / p.BM);
        const int le = min(max(p.block_expert[b], 0), p.El - 1);
        const int j = p.block_index[b] * p.BM + (int)(row - (long)b * p.BM);
        const int n = p.recv_tot[le];
        // the pool is tiled: 16-byte chunk i of the row (K block i/8) at dst[(i/8)*BM*8 + i%8]
        v4i* dst = reinterpret_cast<v4i*>(p.pool_x + (size_t)b * SF * p.BM * 128) + (row - (long)b * p.BM) * 8;
        const int kstride = p.BM * 8;
        // scales are block-major: K block i of this row at dsf[i * BM]
        float* dsf = p.pool_sf + (size_t)b * SF * p.BM + (row - (long)b * p.BM);
        uint32_t* meta = p.pool_meta + (size_t)row * 3;
        if (j >= n) {
            const v4i z = {0, 0, 0, 0};
            for (int i = lane; i < H16; i += 64) dst[(i >> 3) * kstride + (i & 7)] = z;
            for (int i = lane; i < SF; i += 64) dsf[(size_t)i * p.BM] = 0.f;
            if (lane < 3) meta[lane] = kMetaPad;
            if (lane == 3) p.pool_dst[row] = kMetaPad;
            continue;
        }
        // min-peeling round-robin over the sources (lane = source shard).  Every round retires at
        // least one source, so S rounds always suffice.
        int rem = lane < p.S ? p.recv[le * p.S + lane] : 0;
        int jj = j, offset = 0, src = 0, slot = 0;
        for (int round = 0; round < p.S; ++round) {
            const bool act = rem > 0;
            const uint64_t am = __ballot(act);
            const int nact = __popcll(am);
            if (nact == 0) break;
            const int len = wave_min(act ? rem : 0x7FFFFFFF);
            const long nround = (long)len * nact;
            if (jj < nround) {
                const int target = jj % nact;
                const uint64_t sel = __ballot(act && __popcll(am & lanemask_lt()) == target);
                src = __ffsll((unsigned long long)sel) - 1;
                slot = offset + jj / nact;
                break;
            }
            jj -= (int)nround;
            offset += len;
            rem -= min(rem, len);
        }
        const int v = slot < p.T_max ? p.table[((size_t)le * p.S + src) * p.T_max + slot] : -1;
        if (v < 0 || v >= p.tps[src] * p.K) {              // never for metadata the routing stage made
            if (lane == 0) atomicOr(p.status, MEGA_MOE_STATUS_BAD_LAYOUT);
            for (int i = lane; i < H16; i += 64) dst[(i >> 3) * kstride + (i & 7)] = v4i{0, 0, 0, 0};
            for (int i = lane; i < SF; i += 64) dsf[(size_t)i * p.BM] = 0.f;
            if (lane < 3) meta[lane] = kMetaPad;
            if (lane == 3) p.pool_dst[row] = kMetaPad;
            continue;
        }
        const int t = v / p.K, k = v - t * p.K;
        const size_t srow = (size_t)src * p.T_max + t;
        const v4i* sp = reinterpret_cast<const v4i*>(p.x + srow * p.H);
        for (int base = 0; base < H16; base += 64 * kUnroll) {
            v4i r[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = base + u * 64 + lane;
                if (i < H16) r[u] = sp[i];
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = base + u * 64 + lane;
                if (i < H16) dst[(i >> 3) * kstride + (i & 7)] = r[u];
            }
        }
        const float* ssf = p.x_sf + srow * SF;
        for (int i = lane; i < SF; i += 64) dsf[(size_t)i * p.BM] = ssf[i];
        if (lane < 3) meta[lane] = lane == 0 ? (uint32_t)src : (lane == 1 ? (uint32_t)t : (uint32_t)k);
        if (lane == 3) p.pool_dst[row] = (uint32_t)(((size_t)k * p.S + src) * p.T_max + t);
    }
}

}  // namespace

hipError_t launch_fill(const Params& p, int num_cus, hipStream_t stream) {
    // Enough waves to cover HBM latency; rows beyond the routed count make the waves exit at once.
    const long cap_rows = (long)p.max_blocks * p.BM;
    long grid = (cap_rows + 3) / 4;
    const long max_grid = (long)num_cus * 8;
    if (grid > max_grid) grid = max_grid;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)grid), dim3(kFillThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mm
