// Top-k weighted combine back to token-major order.
//
// y[s,t] = bf16( sum over k with a local expert of w[s,t,k] * comb[k][s*T_max+t] ), accumulated in fp32
// in ascending k ("Dispatch/Combine: blog theory vs DeepEP vs DeepGEMM Mega MoE", section 1: the output
// is the weight-sum of the chosen experts' outputs; "DeepGEMM Mega MoE symmetric memory deep analysis",
// 9.2: per token the top-k slots with a negative index are masked, the rest are accumulated in fp32 and
// cast to bf16).  With a shared expert, tokens of the own shard also add combine slot K with weight 1,
// after the routed slots (same page, 8.2 and 9.2: the lane after the top-k lanes stands for the shared
// slot).  A token with nothing to add gets a zero row; rows t >= T_s are left untouched.
//
// One wave per token: lanes 0..K-1 read the token's expert ids and weights and a ballot gives the
// local slots.  Lane l owns the 16-byte chunks l, l+64, ... of the row; a batch of kBatch chunks is
// loaded for one slot (all loads in flight together), accumulated in fp32, and after the last slot
// converted and stored.  The code is branch-free per lane: chunk indices past the row's end are clamped
// to its last chunk (the same bytes are read and written again), so the compiler's memory-counter waits
// stay exact.
#include "mm_internal.h"

namespace mm {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void acc8(float* acc, const uint4& v, float w) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w * bf16_to_f32(u[i] & 0xFFFFu);
        acc[2 * i + 1] += w * bf16_to_f32(u[i] >> 16);
    }
}

// Two fp32 -> two bf16 (round to nearest even) in one word, the first value in the low half.
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}

template <int kBatch>
__global__ __launch_bounds__(kThreads) void combine_kernel(Params p) {
    const int lane = threadIdx.x & 63;
    const long tok = (long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const long ntok = (long)p.S * p.T_max;
    if (tok >= ntok) return;
    const int s = (int)(tok / p.T_max), t = (int)(tok - (long)s * p.T_max);
    if (t >= p.tps[s]) return;
    float w = 0.f;
    bool is_local = false;
    if (lane < p.K) {
        const int64_t e = p.topk_idx[tok * p.K + lane];
        is_local = e >= p.lo && e < p.lo + p.El;
        if (is_local) w = p.topk_w[tok * p.K + lane];
    } else if (lane == p.K && p.nsh && s == p.own) {
        is_local = true;
        w = 1.0f;
    }
    const uint64_t mask = __ballot(is_local);
    const int H8 = p.H >> 3;                        // 16-byte chunks per row
    const int J = (H8 + 63) >> 6;                   // chunks per lane
    const size_t plane = (size_t)ntok * p.H;        // elements per k plane of comb
    uint4* yrow = reinterpret_cast<uint4*>(p.y + (size_t)tok * p.H);
    auto chunk = [&](int j) { return min(min(j, J - 1) * 64 + lane, H8 - 1); };
    for (int j0 = 0; j0 < J; j0 += kBatch) {
        float a[kBatch][8];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) a[u][i] = 0.f;
        for (uint64_t m = mask; m; m &= m - 1) {          // ascending k
            const int k = __ffsll((unsigned long long)m) - 1;
            const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
            const uint4* src = reinterpret_cast<const uint4*>(p.comb + (size_t)k * plane + (size_t)tok * p.H);
            uint4 v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) v[u] = src[chunk(j0 + u)];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) acc8(a[u], v[u], wk);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            yrow[chunk(j0 + u)] = uint4{bf16x2(a[u][0], a[u][1]), bf16x2(a[u][2], a[u][3]),
                                        bf16x2(a[u][4], a[u][5]), bf16x2(a[u][6], a[u][7])};
    }
}

}  // namespace

hipError_t launch_combine(const Params& p, hipStream_t stream) {
    const long ntok = (long)p.S * p.T_max;
    const long grid = (ntok + (kThreads / 64) - 1) / (kThreads / 64);
    // a batch that divides the chunks per lane (H/512) when it can.  A whole row per batch (14 chunks at
    // H = 7168: one load round per slot) measured faster than two batches of 7 at the 2 waves per SIMD its
    // 203 VGPRs leave (prefill 172 -> 168 us, decode 11.4 -> 10.9 us, same box)
    const int J = ((p.H >> 3) + 63) >> 6;
    if (J % 14 == 0) hipLaunchKernelGGL(combine_kernel<14>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    else if (J % 7 == 0) hipLaunchKernelGGL(combine_kernel<7>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    else if (J % 8 == 0) hipLaunchKernelGGL(combine_kernel<8>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL(combine_kernel<4>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mm
