// Top-k weighted combine back to token-major order.
//
// y[s,t] = bf16( sum over k with a local expert of w[s,t,k] * comb[k][s*T_max+t] ), accumulated in fp32
// in ascending k ("Dispatch/Combine: blog theory vs DeepEP vs DeepGEMM Mega MoE", section 1: the output
// is the weight-sum of the chosen experts' outputs; "DeepGEMM Mega MoE symmetric memory deep analysis",
// 9.2: per token the top-k slots with a negative index are masked, the rest are accumulated in fp32 and
// cast to bf16).  A token with no local expert gets a zero row; rows t >= T_s are left untouched.
//
// One wave per token: lanes 0..K-1 read the token's expert ids and weights, a ballot gives the local
// slots, then each lane reduces 8 bf16 (16 bytes) per slot and chunk, two chunks in flight per lane.
#include "mm_internal.h"

namespace mm {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLocal = 8;    // slots loaded together; more are handled in further passes

__device__ __forceinline__ void acc8(float* acc, const uint4& v, float w) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w * bf16_to_f32(u[i] & 0xFFFFu);
        acc[2 * i + 1] += w * bf16_to_f32(u[i] >> 16);
    }
}

__global__ __launch_bounds__(kThreads) void combine_kernel(Params p) {
    const int lane = threadIdx.x & 63;
    const long tok = (long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const long ntok = (long)p.S * p.T_max;
    if (tok >= ntok) return;
    const int s = (int)(tok / p.T_max), t = (int)(tok - (long)s * p.T_max);
    if (t >= p.tps[s]) return;
    int k_local = 0;
    float w = 0.f;
    bool is_local = false;
    if (lane < p.K) {
        const int64_t e = p.topk_idx[tok * p.K + lane];
        is_local = e >= p.lo && e < p.lo + p.El;
        if (is_local) w = p.topk_w[tok * p.K + lane];
    }
    (void)k_local;
    const uint64_t mask = __ballot(is_local);
    const int H8 = p.H >> 3;                        // 16-byte chunks per row
    const size_t plane = (size_t)ntok * p.H;        // elements per k plane of comb
    uint4* yrow = reinterpret_cast<uint4*>(p.y + (size_t)tok * p.H);
    for (int c0 = lane; c0 < H8; c0 += 128) {
        const int c1 = c0 + 64;
        float a0[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float a1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        uint64_t m = mask;
        while (m) {
            int ks[kMaxLocal];
            int n = 0;
#pragma unroll
            for (int u = 0; u < kMaxLocal; ++u) {
                ks[u] = 0;
                if (m) { ks[u] = __ffsll((unsigned long long)m) - 1; m &= m - 1; n = u + 1; }
            }
            uint4 v0[kMaxLocal], v1[kMaxLocal];
#pragma unroll
            for (int u = 0; u < kMaxLocal; ++u) {
                if (u < n) {
                    const uint4* src = reinterpret_cast<const uint4*>(p.comb + (size_t)ks[u] * plane +
                                                                      (size_t)tok * p.H);
                    v0[u] = src[c0];
                    if (c1 < H8) v1[u] = src[c1];
                }
            }
#pragma unroll
            for (int u = 0; u < kMaxLocal; ++u) {
                if (u < n) {
                    const float wk = __shfl(w, ks[u]);
                    acc8(a0, v0[u], wk);
                    if (c1 < H8) acc8(a1, v1[u], wk);
                }
            }
        }
        uint4 o;
        o.x = (uint32_t)f32_to_bf16(a0[0]) | ((uint32_t)f32_to_bf16(a0[1]) << 16);
        o.y = (uint32_t)f32_to_bf16(a0[2]) | ((uint32_t)f32_to_bf16(a0[3]) << 16);
        o.z = (uint32_t)f32_to_bf16(a0[4]) | ((uint32_t)f32_to_bf16(a0[5]) << 16);
        o.w = (uint32_t)f32_to_bf16(a0[6]) | ((uint32_t)f32_to_bf16(a0[7]) << 16);
        yrow[c0] = o;
        if (c1 < H8) {
            o.x = (uint32_t)f32_to_bf16(a1[0]) | ((uint32_t)f32_to_bf16(a1[1]) << 16);
            o.y = (uint32_t)f32_to_bf16(a1[2]) | ((uint32_t)f32_to_bf16(a1[3]) << 16);
            o.z = (uint32_t)f32_to_bf16(a1[4]) | ((uint32_t)f32_to_bf16(a1[5]) << 16);
            o.w = (uint32_t)f32_to_bf16(a1[6]) | ((uint32_t)f32_to_bf16(a1[7]) << 16);
            yrow[c1] = o;
        }
    }
}

}  // namespace

hipError_t launch_combine(const Params& p, hipStream_t stream) {
    const long ntok = (long)p.S * p.T_max;
    const long grid = (ntok + (kThreads / 64) - 1) / (kThreads / 64);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mm
