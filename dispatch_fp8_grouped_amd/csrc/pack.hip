// One-time weight transform into the tiled order the grouped GEMMs stream: every (local expert, n tile,
// K step) chunk of 256 weight rows x 128 bytes becomes contiguous, so one GEMM step's weight DMA reads
// 32 KB of consecutive lines.  The pages' kernels also take their weights in a transformed layout
// ("DeepGEMM Mega MoE symmetric memory deep analysis", 10.2: gate/up interleaving and a scale-factor
// transpose for the SM100 tensor memory); this transform is the MI355X counterpart.
//
//   W1 [E_l][2I][H] -> [E_l][I/128][H/128][256][128]: row r < 128 is gate row nt*128 + r, row r >= 128 is
//                     up row I + nt*128 + (r - 128)
//   W2 [E_l][H][I]  -> [E_l][H/256][I/128][256][128]: row r is W2 row nt*256 + r
// MXFP4 weights (two e2m1 codes per byte) pack the same way with 64-byte rows per 128-value K step:
//   W1 [E_l][2I][H/2] -> [E_l][I/128][H/128][256][64], W2 [E_l][H][I/2] -> [E_l][H/256][I/128][256][64].
// Their UE8M0 exponents (one byte per 32 values along K) follow the same chunking, four bytes per row and
// K step, so that one GEMM step reads a chunk's exponents as 1 KB of consecutive words:
//   W1 exponents [E_l][2I][H/32] -> [E_l][I/128][H/128][256] words, W2 [E_l][H][I/32] -> [E_l][H/256][I/128][256].
//
// One thread per 16-byte piece of the packed tensor (contiguous stores); one per word for the exponents.
#include "mm_internal.h"

namespace mm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kPackThreads = 256;

// gate_up: W1 (rows of an n tile are 128 gate rows then 128 up rows); otherwise W2 (256 consecutive rows).
// P: 16-byte pieces per row and K step (8 for FP8, 4 for two FP4 codes per byte).
template <bool kGateUp, int P>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const v4i* __restrict__ src, v4i* __restrict__ dst,
                                                            int rows, int K, int I, long pieces) {
    const int KB = K >> 7;
    const long row_pieces = (long)KB * P;           // 16-byte pieces of one source row
    for (long o = (long)blockIdx.x * kPackThreads + threadIdx.x; o < pieces; o += (long)gridDim.x * kPackThreads) {
        // o = ((((le * NT + nt) * KB + kb) * 256 + r) * P + j)
        const int j = (int)(o % P);
        long q = o / P;
        const int r = (int)(q & 255);
        q >>= 8;
        const int kb = (int)(q % KB);
        q /= KB;                               // le * NT + nt
        const int NT = kGateUp ? (I >> 7) : (rows >> 8);
        const int nt = (int)(q % NT);
        const long le = q / NT;
        const int row = kGateUp ? (r < 128 ? nt * 128 + r : I + nt * 128 + r - 128) : nt * 256 + r;
        dst[o] = src[(le * rows + row) * row_pieces + (long)kb * P + j];
    }
}

// MXFP4 exponents: word (le, nt, kb, r) = the four bytes of packed row r for K step kb.
template <bool kGateUp>
__global__ __launch_bounds__(kPackThreads) void pack_scales_kernel(const uint32_t* __restrict__ src,
                                                                   uint32_t* __restrict__ dst, int rows, int K,
                                                                   int I, long words) {
    const int KB = K >> 7;                          // source row: K/32 bytes = KB words
    const int NT = kGateUp ? (I >> 7) : (rows >> 8);
    for (long o = (long)blockIdx.x * kPackThreads + threadIdx.x; o < words; o += (long)gridDim.x * kPackThreads) {
        const int r = (int)(o & 255);
        long q = o >> 8;
        const int kb = (int)(q % KB);
        q /= KB;
        const int nt = (int)(q % NT);
        const long le = q / NT;
        const int row = kGateUp ? (r < 128 ? nt * 128 + r : I + nt * 128 + r - 128) : nt * 256 + r;
        dst[o] = src[(le * rows + row) * KB + kb];
    }
}

long pack_grid(long items, int num_cus) {
    long g = (items + kPackThreads - 1) / kPackThreads;
    const long cap = (long)num_cus * 8;
    return g < cap ? (g < 1 ? 1 : g) : cap;
}

}  // namespace

hipError_t launch_pack_scales(const void* s1, const void* s2, void* s1p, void* s2p, int El, int H, int I,
                              int num_cus, hipStream_t stream) {
    const long n1 = (long)El * 2 * I * H / 128, n2 = (long)El * H * I / 128;   // words
    hipLaunchKernelGGL((pack_scales_kernel<true>), dim3((unsigned)pack_grid(n1, num_cus)), dim3(kPackThreads), 0,
                       stream, static_cast<const uint32_t*>(s1), static_cast<uint32_t*>(s1p), 2 * I, H, I, n1);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((pack_scales_kernel<false>), dim3((unsigned)pack_grid(n2, num_cus)), dim3(kPackThreads), 0,
                       stream, static_cast<const uint32_t*>(s2), static_cast<uint32_t*>(s2p), H, I, I, n2);
    return hipGetLastError();
}

// Hk / Ik: the K extents of W1 and W2 rows in bytes-per-value units (H and I for FP8 and MXFP4, 2H and
// 2I for BF16, whose 128-byte K chunks then hold 64 values); I: the intermediate size (W1's gate / up
// split and W2's row count H = its N extent are in values).  With BF16, W2 has Hk/2 rows.
hipError_t launch_pack(const void* w1, const void* w2, void* w1p, void* w2p, int El, int Hk, int Ik, int I, bool fp4,
                       int num_cus, hipStream_t stream) {
    const int div = fp4 ? 32 : 16;                  // bytes per weight value: 1/2 or 1
    const int H = Hk / (Ik / I);                    // W2 rows
    const long p1 = (long)El * 2 * I * Hk / div, p2 = (long)El * H * Ik / div;
    auto grid = [&](long pieces) { return (unsigned)pack_grid(pieces, num_cus); };
    if (fp4) {
        hipLaunchKernelGGL((pack_kernel<true, 4>), dim3(grid(p1)), dim3(kPackThreads), 0, stream,
                           static_cast<const v4i*>(w1), static_cast<v4i*>(w1p), 2 * I, H, I, p1);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((pack_kernel<false, 4>), dim3(grid(p2)), dim3(kPackThreads), 0, stream,
                           static_cast<const v4i*>(w2), static_cast<v4i*>(w2p), H, I, I, p2);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((pack_kernel<true, 8>), dim3(grid(p1)), dim3(kPackThreads), 0, stream,
                       static_cast<const v4i*>(w1), static_cast<v4i*>(w1p), 2 * I, Hk, I, p1);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((pack_kernel<false, 8>), dim3(grid(p2)), dim3(kPackThreads), 0, stream,
                       static_cast<const v4i*>(w2), static_cast<v4i*>(w2p), H, Ik, I, p2);
    return hipGetLastError();
}

}  // namespace mm
