// Grouped FP8 GEMMs over the expert-major pool, on gfx950 MFMA (v_mfma_f32_16x16x128_f8f6f4).
//
//   GEMM1 (gate_up): for pool block b of local expert le, G = A W1[le]^T over K = H, with A the pooled
//     FP8 rows.  Epilogue: h = silu(gate) * up, then per row and 128 columns s = max(amax, 1e-4)/448 and
//     q = e4m3fn(h / s) into the L2 pool ("Mega-MoE kernel code walkthrough: from Dispatch to WGMMA",
//     section 6: the L1 epilogue is SwiGLU then FP8; "MoE fused operators", DeepGEMM part, section 5).
//   GEMM2 (down): O = L2 W2[le]^T over K = I; epilogue casts to bf16 and scatters row m to
//     comb[k][shard*T_max + token] from the pool metadata ("DeepGEMM Mega MoE symmetric memory deep
//     analysis", 8.1-8.2).
//
// Scale promotion ("Mega-MoE notes, part 2: index table and pull", 5.2): every 128-deep K step is one
// MFMA into a fresh accumulator P, then final += (sa[m, kb] * sw[n_block, kb]) * P in fp32.
//
// Tiling: one work-group of 8 waves computes a BM x 256 tile (BM tokens = one pool block, 256 weight
// rows), K step 128, A and B staged through a double-buffered LDS (global -> registers -> LDS, XOR
// swizzle of 16-byte chunks).  The MFMA's A operand is the weight tile and its B operand the token tile,
// so each lane's four outputs share one token and one weight block: the promotion needs one scale per
// token subtile.  Wave (wm, wn) owns tokens [wm*BM/2, +BM/2) and 64 weight rows:
//   GEMM1: gate rows nt*128 + wn*32 + [0,32) and the matching up rows I + nt*128 + wn*32 + [0,32),
//          so gate and up of one output column sit in the same lane;
//   GEMM2: hidden rows nt*256 + wn*64 + [0,64).
// The kernel is persistent: one work-group per CU walks the (block, n-tile) space; consecutive
// work-groups of one XCD take neighbouring tiles (8 pool blocks x 4 n-tiles share A and B in L2).
#include "mm_internal.h"

namespace mm {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kGroupBlocks = 8;   // pool blocks per tile group

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
    // scale operands 0 select the unscaled v_mfma_f32_16x16x128_f8f6f4; format 0 = FP8 e4m3
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16-byte chunk c of a 128-byte LDS row r sits at position c ^ (r & 7).
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

// Fragment of 16 rows x 128 K bytes for one MFMA operand: lane l takes row (l & 15) and the 32 bytes
// [32*(l>>4), +32).  A and B use the same lane -> K mapping, so the product sums every K exactly once.
__device__ __forceinline__ v8i load_frag(const uint8_t* lds, int row0, int lane) {
    const int r = row0 + (lane & 15);
    const int g = lane >> 4;
    const uint4 lo = *reinterpret_cast<const uint4*>(lds + swz(r, 2 * g));
    const uint4 hi = *reinterpret_cast<const uint4*>(lds + swz(r, 2 * g + 1));
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
}

// Four fp32 -> four e4m3fn codes (round to nearest even, saturating), byte i from value i.  The
// hardware conversion rounds to nearest even but turns magnitudes that round past 448 into NaN, so
// values are clamped to +-448 first (a no-op for h/s, which is within 448 up to one rounding).
__device__ __forceinline__ float sat448(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }
__device__ __forceinline__ uint32_t cvt_fp8x4(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), v, true);
    return (uint32_t)v;
}

template <int BM, bool kGemm1>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(Params p) {
    constexpr int TM = BM / 32;                 // 16-token subtiles per wave
    constexpr int WN = 4;                       // 16-row weight subtiles per wave
    constexpr int A_CH = BM * 8 / kThreads;     // 16-byte A chunks per thread per K step
    constexpr int B_CH = 256 * 8 / kThreads;    // 16-byte B chunks per thread per K step
    static_assert(A_CH >= 1 && B_CH == 4, "tile shape");

    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * 128];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][256 * 128];
    __shared__ float sSA[2][BM];
    __shared__ float sRed[BM][4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int rr = lane & 15, g = lane >> 4;
    const int Kdim = kGemm1 ? p.H : p.I;
    const int KB = Kdim >> 7;
    const int NT = kGemm1 ? (p.I >> 7) : (p.H >> 8);
    const int nblocks = min((int)p.status[1], p.max_blocks);
    const long ngroups = (nblocks + kGroupBlocks - 1) / kGroupBlocks;
    const long ntiles = ngroups * kGroupBlocks * NT;
    const int G = gridDim.x;                    // a multiple of 8
    const int logical = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

    for (long tile = logical; tile < ntiles; tile += G) {
        const long grp = tile / (kGroupBlocks * NT);
        const int rem = (int)(tile - grp * (kGroupBlocks * NT));
        const int nt = rem / kGroupBlocks;
        const int b = (int)(grp * kGroupBlocks) + (rem - nt * kGroupBlocks);
        if (b >= nblocks) continue;
        const int le = p.block_expert[b];
        if (le < 0 || le >= p.El) continue;
        const size_t row0 = (size_t)b * BM;
        const uint8_t* A = (kGemm1 ? p.pool_x : p.l2_x) + row0 * Kdim;
        const float* Asf = (kGemm1 ? p.pool_sf : p.l2_sf) + row0 * KB;
        const uint8_t* W = kGemm1 ? p.w1 + (size_t)le * (2 * p.I) * p.H : p.w2 + (size_t)le * p.H * p.I;
        const float* Wsf = kGemm1 ? p.w1_sf + (size_t)le * ((2 * p.I) >> 7) * KB
                                  : p.w2_sf + (size_t)le * (p.H >> 7) * KB;

        // global source / LDS destination of this thread's chunks
        const uint8_t* a_src[A_CH];
        int a_dst[A_CH];
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int ci = tid + i * kThreads, r = ci >> 3, c = ci & 7;
            a_src[i] = A + (size_t)r * Kdim + c * 16;
            a_dst[i] = swz(r, c);
        }
        const uint8_t* b_src[B_CH];
        int b_dst[B_CH];
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int ci = tid + i * kThreads, r = ci >> 3, c = ci & 7;
            int wrow;
            if (kGemm1) wrow = r < 128 ? nt * 128 + r : p.I + nt * 128 + (r - 128);
            else wrow = nt * 256 + r;
            b_src[i] = W + (size_t)wrow * Kdim + c * 16;
            b_dst[i] = swz(r, c);
        }
        // LDS row of this wave's weight subtile a
        int wrow0[WN];
#pragma unroll
        for (int a = 0; a < WN; ++a) {
            if (kGemm1) wrow0[a] = (a < 2 ? 0 : 128) + wn * 32 + (a & 1) * 16;
            else wrow0[a] = wn * 64 + a * 16;
        }
        // scale rows of the weight blocks this wave touches
        const float* swp0;
        const float* swp1;
        if (kGemm1) {
            swp0 = Wsf + (size_t)nt * KB;                          // gate block
            swp1 = Wsf + (size_t)((p.I >> 7) + nt) * KB;           // up block
        } else {
            swp0 = Wsf + (size_t)(nt * 2 + (wn >> 1)) * KB;
            swp1 = swp0;
        }

        v4f acc[WN][TM];
#pragma unroll
        for (int a = 0; a < WN; ++a)
#pragma unroll
            for (int t = 0; t < TM; ++t) acc[a][t] = v4f{0.f, 0.f, 0.f, 0.f};

        uint4 ra[A_CH], rb[B_CH];
        float rsa = 0.f;
        // prologue: K step 0 into buffer 0
#pragma unroll
        for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i]);
#pragma unroll
        for (int i = 0; i < B_CH; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i]);
        if (tid < BM) rsa = Asf[(size_t)tid * KB];
#pragma unroll
        for (int i = 0; i < A_CH; ++i) *reinterpret_cast<uint4*>(&sA[0][a_dst[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_CH; ++i) *reinterpret_cast<uint4*>(&sB[0][b_dst[i]]) = rb[i];
        if (tid < BM) sSA[0][tid] = rsa;
        __syncthreads();

        for (int kb = 0; kb < KB; ++kb) {
            const int cur = kb & 1;
            const bool more = kb + 1 < KB;
            if (more) {
                const int off = (kb + 1) * 128;
#pragma unroll
                for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + off);
#pragma unroll
                for (int i = 0; i < B_CH; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + off);
                if (tid < BM) rsa = Asf[(size_t)tid * KB + kb + 1];
            }
            const float sw0 = swp0[kb], sw1 = swp1[kb];
            float sa[TM];
            v8i xf[TM];
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const int r0 = wm * (BM / 2) + t * 16;
                sa[t] = sSA[cur][r0 + rr];
                xf[t] = load_frag(sA[cur], r0, lane);
            }
#pragma unroll
            for (int a = 0; a < WN; ++a) {
                const v8i wf = load_frag(sB[cur], wrow0[a], lane);
                const float swa = (kGemm1 && a >= 2) ? sw1 : sw0;
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    const v4f pr = mfma_fp8(wf, xf[t], v4f{0.f, 0.f, 0.f, 0.f});
                    const float sc = sa[t] * swa;
                    acc[a][t] += sc * pr;
                }
            }
            if (more) {
#pragma unroll
                for (int i = 0; i < A_CH; ++i) *reinterpret_cast<uint4*>(&sA[cur ^ 1][a_dst[i]]) = ra[i];
#pragma unroll
                for (int i = 0; i < B_CH; ++i) *reinterpret_cast<uint4*>(&sB[cur ^ 1][b_dst[i]]) = rb[i];
                if (tid < BM) sSA[cur ^ 1][tid] = rsa;
            }
            __syncthreads();
        }

        // ------------------------------------------------------------------ epilogues
        // lane holds acc[a][t][i]: weight row wrow0[a] + 4g + i, token wm*BM/2 + 16t + rr
        if (kGemm1) {
            float h[2][TM][4];
            float amax[TM];
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                float m = 0.f;
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float gt = acc[a][t][i], up = acc[a + 2][t][i];
                        const float v = gt / (1.0f + __expf(-gt)) * up;
                        h[a][t][i] = v;
                        m = fmaxf(m, fabsf(v));
                    }
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                amax[t] = m;
                if (g == 0) sRed[wm * (BM / 2) + t * 16 + rr][wn] = m;
            }
            __syncthreads();
            const int I = p.I;
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const int tok = wm * (BM / 2) + t * 16 + rr;
                const float* red = sRed[tok];
                const float am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
                const float s = fmaxf(am, 1e-4f) / 448.0f;
                const size_t row = row0 + tok;
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const int col = nt * 128 + wn * 32 + a * 16 + 4 * g;
                    const uint32_t q = cvt_fp8x4(h[a][t][0] / s, h[a][t][1] / s, h[a][t][2] / s,
                                                 h[a][t][3] / s);
                    *reinterpret_cast<uint32_t*>(p.l2_x + row * I + col) = q;
                    if (p.gemm1_out) {
                        float* go = p.gemm1_out + row * (size_t)(2 * I);
                        *reinterpret_cast<float4*>(go + col) =
                            make_float4(acc[a][t][0], acc[a][t][1], acc[a][t][2], acc[a][t][3]);
                        *reinterpret_cast<float4*>(go + I + col) =
                            make_float4(acc[a + 2][t][0], acc[a + 2][t][1], acc[a + 2][t][2], acc[a + 2][t][3]);
                    }
                }
                if (wn == 0 && g == 0) p.l2_sf[row * (size_t)(I >> 7) + nt] = s;
            }
            (void)amax;
            __syncthreads();   // sRed is rewritten by the next tile
        } else {
            const size_t plane = (size_t)p.S * p.T_max;
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const int tok = wm * (BM / 2) + t * 16 + rr;
                const uint32_t* meta = p.pool_meta + (row0 + tok) * 3;
                const uint32_t ms = meta[0], mt = meta[1], mk = meta[2];
                if (ms >= (uint32_t)p.S || mt >= (uint32_t)p.T_max || mk >= (uint32_t)p.K) continue;  // padding
                uint16_t* dst = p.comb + ((size_t)mk * plane + (size_t)ms * p.T_max + mt) * p.H;
#pragma unroll
                for (int a = 0; a < WN; ++a) {
                    const int col = nt * 256 + wn * 64 + a * 16 + 4 * g;
                    uint2 v;
                    v.x = (uint32_t)f32_to_bf16(acc[a][t][0]) | ((uint32_t)f32_to_bf16(acc[a][t][1]) << 16);
                    v.y = (uint32_t)f32_to_bf16(acc[a][t][2]) | ((uint32_t)f32_to_bf16(acc[a][t][3]) << 16);
                    *reinterpret_cast<uint2*>(dst + col) = v;
                }
            }
        }
    }
}

template <int BM, bool kGemm1>
hipError_t launch(const Params& p, int num_cus, hipStream_t stream) {
    int grid = (num_cus + 7) / 8 * 8;
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, kGemm1>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm1(const Params& p, int num_cus, hipStream_t stream) {
    return p.BM == 64 ? launch<64, true>(p, num_cus, stream) : launch<128, true>(p, num_cus, stream);
}

hipError_t launch_gemm2(const Params& p, int num_cus, hipStream_t stream) {
    return p.BM == 64 ? launch<64, false>(p, num_cus, stream) : launch<128, false>(p, num_cus, stream);
}

}  // namespace mm
