// Internal definitions shared by the HIP translation units of libmegamoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mega_moe.h"

namespace mm {

constexpr int kRouteChunk = 256;       // flat (token, k) entries per routing work-group
constexpr int kBK = 128;               // GEMM K step = one scale block
constexpr int kBN = 256;               // GEMM weight rows per tile
constexpr uint32_t kMetaPad = 0xFFFFFFFFu;
// Schedule words of the launches that hand rows over inside (workspace region `sched`, zero between
// forwards)
constexpr int kSchedExit = 2;          // work-groups that have finished
constexpr int kSchedXcdClaim = 8;      // [8 + x]: next fill unit of XCD x to claim
constexpr int kSchedXcdSlots = 16;     // [16 + x]: bit r = the work-group in slot r of XCD x has started
constexpr int kSchedGridBar = 40;      // [40 + i]: work-groups past device-wide barrier i of the routing
constexpr int kSchedArrival = 64;      // [64 + b]: completed fill units of pool block b, then
                                       // [64 + max_blocks + b]: completed GEMM1 n tiles of pool block b

// Everything a kernel needs, passed by value (kernel arguments).
struct Params {
    // shapes
    int S, T_max, H, I, E, El, lo, K, BM;
    int nsh;              // shared experts (0 or 1): pool segment El, weights index El, combine slot K
    int own;              // the shard the shared expert reads (local_rank)
    int wfmt;             // MEGA_MOE_WEIGHTS_FP8 or MEGA_MOE_WEIGHTS_MXFP4
    int chunks;           // routing chunks per shard
    int max_blocks;       // pool capacity in BM blocks
    int wave_tiles;       // one-launch GEMMs: GEMM1 tiles an expert wave holds at least (0: one wave)
    uint32_t flags;
    int tps[MEGA_MOE_MAX_SHARDS];
    // workspace
    uint32_t* status;     // [0] status bits, [1] number of pool blocks
    int* chunk_hist;      // [S][chunks][E]
    int* chunk_base;      // [S][chunks][El]
    int* send;            // [S][E]
    int* recv;            // [El][S]
    int* recv_tot;        // [El]
    int* pool_off;        // [El+1]
    int* block_expert;    // [max_blocks]
    int* block_index;     // [max_blocks]
    int* table;           // [El][S][T_max]
    uint8_t* pool_x;      // [rows][H]
    float* pool_sf;       // [blocks][H/128][BM]: scale of row b*BM+i, K block kb at (b*(H/128)+kb)*BM+i
    uint32_t* pool_meta;  // [rows][3]
    uint32_t* pool_dst;   // [rows]: comb row k*S*T_max + shard*T_max + token, padding ~0
    uint8_t* l2_x;        // [blocks][I/128][4][BM][32]: row b*BM+m, columns kb*128 + 32q .. +31 at
                          // ((b*(I/128) + kb)*4 + q)*BM*32 + m*32
    float* l2_sf;         // [blocks][I/128][BM], the same block-major order
    uint16_t* comb;       // [K][S*T_max][H]
    float* gemm1_out;     // [rows][2I] or null
    uint32_t* sched;      // kSched* words, then the per-block fill and GEMM1 counts
    // caller tensors
    const uint8_t* x;
    const float* x_sf;
    const int64_t* topk_idx;
    const float* topk_w;
    const uint8_t* w1;
    const float* w1_sf;
    const uint8_t* w2;
    const float* w2_sf;
    uint16_t* y;
    int* cum;
};

// Launchers (one per translation unit), all on `stream`.  Return hipSuccess or the launch error.
hipError_t launch_route(const Params& p, hipStream_t stream);
hipError_t launch_fill(const Params& p, int num_cus, hipStream_t stream);
// fuse_fill: GEMM1's work-groups also pull the pool rows, and each tile waits for its block's arrival
hipError_t launch_gemm1(const Params& p, bool fuse_fill, int num_cus, hipStream_t stream);
hipError_t launch_gemm2(const Params& p, int num_cus, hipStream_t stream);
// GEMM1 and GEMM2 in one launch (fuse_fill: the pool rows are pulled in it as well)
hipError_t launch_gemms(const Params& p, bool fuse_fill, int num_cus, hipStream_t stream);
// Routing, the pull and both GEMMs in one launch (FP8 weights; needs every work-group resident at once)
hipError_t launch_route_fill_gemms(const Params& p, int num_cus, hipStream_t stream);
hipError_t launch_combine(const Params& p, hipStream_t stream);
hipError_t launch_pack(const void* w1, const void* w2, void* w1p, void* w2p, int El, int Hk, int Ik, int I, bool fp4,
                       int num_cus, hipStream_t stream);
// MXFP4 exponent transform: [E_w][2I][H/32] / [E_w][H][I/32] bytes -> [E_w][NT][K/128][256] words.
hipError_t launch_pack_scales(const void* s1, const void* s2, void* s1p, void* s2p, int El, int H, int I,
                              int num_cus, hipStream_t stream);

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = __lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

}  // namespace mm
