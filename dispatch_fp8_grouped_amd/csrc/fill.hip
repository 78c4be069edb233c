// Pool fill: the receiver-side pull of routed FP8 (or BF16) rows into the expert-major L1 pool.
//
// The routing stage already resolved every pool row to its source: the round-robin position of each
// index-table entry ("Mega-MoE notes, part 2: index table and pull", 2.5) gave the row's metadata
// {shard, token, k}, and padding rows carry all ones.  The fill copies each row's H FP8 codes into the
// tiled pool and its H/128 scales into the block-major scale array ("Mega-MoE notes, part 2", 2.6;
// "Dispatch/Combine ... comparison", 6.2); padding rows get zero codes and zero scales.
//
// One wave per pool row, 16-byte loads and stores.  A wave reads the metadata of its next 64 rows in
// one vector load (lane l: row l), so each row waits only on its own data.
#include "mm_internal.h"

namespace mm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kFillThreads = 256;

// Lane l copies chunks l, l+64, ... of a row.  A batch issues kUnroll loads, then kUnroll stores, with
// no branch between them: indices past the row's end are clamped to its last chunk, so those lanes
// copy a chunk again (the same bytes to the same place).  Straight-line code keeps the compiler's
// memory-counter waits exact; a per-lane branch around a load or store makes it wait for every
// outstanding access, stores included, before each store.
// kFull: H is a multiple of 1024, so every lane has the same chunk count and no index is clamped.
// kUnroll: 16-byte chunks per lane per batch.  Seven when a row is seven chunks per lane (H = 7168: one
// load round per row, 48 VGPRs, still 8 waves per SIMD; prefill fill 96.5-97.1 -> 93.2-93.5 us in a
// same-box A/B), else four.
template <bool kFull, int kUnroll>
__global__ __launch_bounds__(kFillThreads, 8) void fill_kernel(Params p) {
    const int lane = threadIdx.x & 63;
    const int wave0 = __builtin_amdgcn_readfirstlane(blockIdx.x * (kFillThreads / 64) + (threadIdx.x >> 6));
    const int nwaves = gridDim.x * (kFillThreads / 64);
    const int rows = min((int)p.status[1], p.max_blocks) * p.BM;
    // bytes per row: H e4m3fn codes, or (BF16 x BF16) H bf16 values, in 128-byte K chunks either way
    const bool bf16 = p.wfmt == MEGA_MOE_WEIGHTS_BF16;
    const int Hb = bf16 ? 2 * p.H : p.H;
    const int H16 = Hb >> 4;
    const int CH = Hb >> 7;                   // 128-byte chunks per row
    const int J = (H16 + 63) >> 6;            // chunks per lane
    const uint32_t kstride16 = (uint32_t)p.BM * 128;   // bytes between K blocks of the tiled pool
    // chunk c of a row: source byte c*16; tiled destination byte (c/8)*BM*128 + (c%8)*16
    auto src_off = [&](int j) -> uint32_t {
        return kFull ? (uint32_t)j * 1024 + (uint32_t)lane * 16 : (uint32_t)min(j * 64 + lane, H16 - 1) * 16;
    };
    auto dst_off = [&](int j) -> uint32_t {
        if (kFull) return (uint32_t)j * 8 * kstride16 + (uint32_t)(lane >> 3) * kstride16 + (uint32_t)(lane & 7) * 16;
        const int c = min(j * 64 + lane, H16 - 1);
        return (uint32_t)(c >> 3) * kstride16 + (uint32_t)(c & 7) * 16;
    };
    // metadata of this wave's rows wave0, wave0 + nwaves, ...: lane l holds row l of each batch of 64,
    // read back with a uniform readlane, so a row waits only on its own data
    const int nmine = wave0 < rows ? (rows - wave0 + nwaves - 1) / nwaves : 0;
    for (int it0 = 0; it0 < nmine; it0 += 64) {
        uint32_t ms = kMetaPad, mt = 0;
        if (it0 + lane < nmine) {
            const size_t r = (size_t)wave0 + (size_t)(it0 + lane) * nwaves;
            ms = p.pool_meta[r * 3];
            mt = p.pool_meta[r * 3 + 1];
        }
        // consume the metadata here, so the compiler's wait for it is not repeated (as a wait for every
        // outstanding store) at the top of each row
        asm volatile("" ::"v"(ms), "v"(mt));
        const int cnt = min(64, nmine - it0);
        for (int it = 0; it < cnt; ++it) {
            const int row = wave0 + (it0 + it) * nwaves;
            const uint32_t src = __builtin_amdgcn_readlane(ms, it), tok = __builtin_amdgcn_readlane(mt, it);
            const int b = row / p.BM, i_in = row - b * p.BM;
            char* dbase = reinterpret_cast<char*>(p.pool_x + (size_t)b * CH * p.BM * 128 + (size_t)i_in * 128);
            const bool pad = src == kMetaPad;
            if (pad || src >= (uint32_t)p.S || tok >= (uint32_t)p.T_max) {
                // a non-padding row outside the shards never comes from the routing stage
                if (!pad && lane == 0) atomicOr(p.status, MEGA_MOE_STATUS_BAD_LAYOUT);
                const v4i z = {0, 0, 0, 0};
                for (int j = 0; j < J; ++j) *reinterpret_cast<v4i*>(dbase + dst_off(j)) = z;
                continue;
            }
            const size_t srow = (size_t)src * p.T_max + tok;
            const char* sbase = reinterpret_cast<const char*>(p.x + srow * Hb);
            for (int j0 = 0; j0 < J; j0 += kUnroll) {
                v4i r[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    r[u] = *reinterpret_cast<const v4i*>(sbase + src_off(min(j0 + u, J - 1)));
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    *reinterpret_cast<v4i*>(dbase + dst_off(min(j0 + u, J - 1))) = r[u];
            }
        }
    }
    // Scales, block-major (K block k of block b's row m at pool_sf[(b*SF + k)*BM + m]): a wave takes 64
    // consecutive pool rows, lane = row, reads up to 32 of its row's scales at once and writes each K
    // block's 64 values as one coalesced 256-byte store (a row-per-wave store would scatter its SF
    // values over SF lines).  Padding rows and rows the copy above rejected get zeros.
    // When there are fewer rows than waves (decode) the groups go to the first waves that copy no rows,
    // so the scale pass does not queue behind a row copy.
    if (bf16) return;                       // no scales
    const int SF = p.H >> 7;
    const int ngroups = rows >> 6;          // BM is a multiple of 64
    const int first = rows < nwaves ? rows : 0;
    for (int grp = (wave0 - first + nwaves) % nwaves; grp < ngroups; grp += nwaves) {
        const int row = grp * 64 + lane;
        const uint32_t src = p.pool_meta[(size_t)row * 3], tok = p.pool_meta[(size_t)row * 3 + 1];
        const bool ok = src < (uint32_t)p.S && tok < (uint32_t)p.T_max;
        const float2* ssf = reinterpret_cast<const float2*>(p.x_sf + (ok ? ((size_t)src * p.T_max + tok) * SF : 0));
        const int b = row / p.BM, i_in = row - b * p.BM;
        float* dsf = p.pool_sf + (size_t)b * SF * p.BM + i_in;
        for (int k0 = 0; k0 < SF; k0 += 32) {     // SF is even (H is a multiple of 256)
            float2 v[16];                          // up to 32 scales in flight per lane
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = ssf[min(k0 / 2 + u, SF / 2 - 1)];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int k = min(k0 + 2 * u, SF - 2);
                dsf[(size_t)k * p.BM] = ok ? v[u].x : 0.f;
                dsf[(size_t)(k + 1) * p.BM] = ok ? v[u].y : 0.f;
            }
        }
    }
}

}  // namespace

hipError_t launch_fill(const Params& p, int num_cus, hipStream_t stream) {
    // Enough waves to cover HBM latency; rows beyond the routed count make the waves exit at once.  The
    // grid follows the rows expected under uniform routing (each local expert's share padded to BM) with
    // a 2x margin, not the pool's capacity: at decode that halves the work-groups launched (the layer
    // 0.302 -> 0.299 ms); the waves loop, so any row count is covered.
    const long cap_rows = (long)p.max_blocks * p.BM;
    const long per_e = ((long)p.S * p.T_max * p.K / p.E + p.BM - 1) / p.BM * p.BM;
    const long exp_rows = 2 * per_e * (p.El + p.nsh);
    long grid = ((exp_rows < cap_rows ? exp_rows : cap_rows) + 3) / 4;
    if (grid < num_cus) grid = num_cus;
    const long max_grid = (long)num_cus * 8;
    if (grid > max_grid) grid = max_grid;
    if (grid < 1) grid = 1;
    const int Hb = p.wfmt == MEGA_MOE_WEIGHTS_BF16 ? 2 * p.H : p.H;    // bytes per row
    const int J = ((Hb >> 4) + 63) >> 6;                                // 16-byte chunks per lane and row
    if (Hb % 1024 == 0 && J % 7 == 0)
        hipLaunchKernelGGL((fill_kernel<true, 7>), dim3((unsigned)grid), dim3(kFillThreads), 0, stream, p);
    else if (Hb % 1024 == 0)
        hipLaunchKernelGGL((fill_kernel<true, 4>), dim3((unsigned)grid), dim3(kFillThreads), 0, stream, p);
    else hipLaunchKernelGGL((fill_kernel<false, 4>), dim3((unsigned)grid), dim3(kFillThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mm
