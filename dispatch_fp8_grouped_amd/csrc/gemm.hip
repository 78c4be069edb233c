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
// rows) in K steps of 128.  The MFMA's A operand is the weight tile and its B operand the token tile, so
// each lane's four outputs share one token and one weight block and the promotion needs one scale per
// token subtile.  Wave (wm, wn) owns tokens [wm*BM/2, +BM/2) and 64 weight rows:
//   GEMM1: gate rows nt*128 + wn*32 + [0,32) and the matching up rows I + nt*128 + wn*32 + [0,32),
//          so gate and up of one output column sit in the same lane;
//   GEMM2: hidden rows nt*256 + wn*64 + [0,64).
//
// Pipeline: a K step's operands (A and B tiles, the token scales, the two weight-block scales and, for
// GEMM2, the tile's pool metadata) arrive by LDS DMA (global_load_lds) into one of three LDS stages.
// The persistent work-group walks its (tile, K step) sequence as one stream: step s waits until stage s
// has landed (vmcnt counts only the one younger stage), barriers, issues the DMA of step s+2 into the
// stage freed by step s-1, then runs its MFMAs; the next tile's first steps load during the current
// tile's last ones.  Every step issues the same number of DMA instructions (past the end the last step
// is loaded again), so the wait count is a constant.  LDS rows are 128 bytes with the 16-byte chunks
// XOR-swizzled by row; the DMA lanes fetch the global chunk that belongs at their LDS position.
// Tiles map XCD-aware: consecutive work-groups of one XCD take neighbouring tiles of a group of eight
// pool blocks, which share A and B through that XCD's L2.
#include <type_traits>

#include "mm_internal.h"

namespace mm {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kWaves = 8;         // waves per work-group, 2 per SIMD
constexpr int kStages = 3;
constexpr int kGroupBlocks = 8;   // pool blocks per tile group

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
    // scale operands 0 select the unscaled v_mfma_f32_16x16x128_f8f6f4; format 0 = FP8 e4m3
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16-byte chunk c of a 128-byte LDS row r sits at position c ^ (r & 7) ^ ((r >> 3) & 1): the 16 rows
// of one fragment read land in 16 different 16-byte bank slots whether the LDS serves 8 or 16 lanes of a
// 128-bit read per cycle.
__device__ __forceinline__ int swz_chunk(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + (swz_chunk(r, c) << 4); }

// Fragment of 16 rows x 128 K bytes for one MFMA operand: lane l takes row (l & 15) and the 32 bytes
// [32*(l>>4), +32).  A and B use the same lane -> K mapping, so the product sums every K exactly once.
__device__ __forceinline__ v8i load_frag(const uint8_t* lds, int row0, int lane) {
    const int r = row0 + (lane & 15);
    const int g = lane >> 4;
    const v4i lo = *reinterpret_cast<const v4i*>(lds + swz(r, 2 * g));
    const v4i hi = *reinterpret_cast<const v4i*>(lds + swz(r, 2 * g + 1));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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

// LDS DMA: every active lane copies 16 (or 4) bytes from base + off to LDS at dst + lane * size (dst and
// base wave-uniform, off per lane).  Inline asm: the waits for these writes are placed by hand
// (wait_stage_barrier); the compiler, which cannot tell the three stages apart, would otherwise drain
// every DMA in flight before each LDS read.  M0 is set in the same statement.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(lds_ptr)const_cast<void*>(p);
}
// A wave-uniform pointer placed in scalar registers (the DMA takes its base there).
__device__ __forceinline__ const void* sgpr_ptr(const void* ptr) {
    const uint64_t v = (uint64_t)(uintptr_t)ptr;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const void* base, uint32_t off, const void* dst) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds_addr(dst)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, const void* dst) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(off), "s"(base), "s"(lds_addr(dst)) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding, then barrier.  The
// compiler's __syncthreads would drain every LDS DMA in flight; this keeps the younger stage loading.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_all_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int V>
using ic = std::integral_constant<int, V>;

// Work-group: NW waves in a 2 x NW/2 grid over the BM x 256 tile.
template <int BM, int NW, bool kGemm1>
__global__ __launch_bounds__(NW * 64, 1) void grouped_gemm_kernel(Params p) {
    constexpr int NWN = NW / 2;                 // compute waves along the weight (N) side
    constexpr int TM = BM / 32;                 // 16-token subtiles per wave (wave covers BM/2 tokens)
    constexpr int WROWS = 256 / NWN;            // weight rows per wave
    constexpr int WN = WROWS / 16;              // 16-row weight subtiles per wave
    constexpr int HC = WROWS / 2;               // GEMM1: output columns per wave (gate + up halves)
    constexpr int NMF = TM * WN;                // MFMAs per wave and K step
    constexpr int A_INS = BM / (8 * NW);        // 1 KB A DMA instructions per wave and step
    constexpr int B_INS = 32 / NW;              // 1 KB B DMA instructions per wave and step
    constexpr int SA_LANES = BM / NW;           // token scales per wave and step
    constexpr int META_PER_WAVE = BM * 3 / NW;  // metadata dwords per wave and step (GEMM2)
    constexpr int META_INS = (META_PER_WAVE + 63) / 64;
    constexpr int DMA_PER_STEP = A_INS + B_INS + 2 + (kGemm1 ? 0 : META_INS);
    static_assert(A_INS >= 1 && B_INS >= 1 && SA_LANES <= 64, "tile shape");
    static_assert(TM * 32 == BM && WN * 16 == WROWS, "tile shape");

    __shared__ __attribute__((aligned(1024))) uint8_t sA[kStages][BM * 128];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[kStages][256 * 128];
    __shared__ __attribute__((aligned(16))) float sSA[kStages][BM];
    __shared__ __attribute__((aligned(16))) float sSW[kStages][NW][4];
    __shared__ __attribute__((aligned(16))) uint32_t sMeta[kStages][kGemm1 ? 4 : META_INS * 64 * NW];
    __shared__ float sRed[BM][NWN];
    __shared__ int sOff[MEGA_MOE_MAX_LOCAL_EXPERTS + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave / NWN) & 1, wn = wave % NWN;
    const int rr = lane & 15, g = lane >> 4;
    const int Kdim = kGemm1 ? p.H : p.I;
    const int KB = Kdim >> 7;
    const int NT = kGemm1 ? (p.I >> 7) : (p.H >> 8);
    const int nblocks = min((int)p.status[1], p.max_blocks);
    const int ntiles = nblocks * NT;
    const int G = gridDim.x;                    // a multiple of 8
    const int logical = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    if (logical >= ntiles) return;
    const int my_tiles = (ntiles - 1 - logical) / G + 1;
    const int nsteps = my_tiles * KB;
    const int full = (nblocks / kGroupBlocks) * kGroupBlocks * NT;
    const int tail = nblocks % kGroupBlocks;

    // expert offsets of the pool in LDS: the expert of a block is found there, so the pipeline never
    // waits on a global load of its own
    for (int i = tid; i <= p.El; i += NW * 64) sOff[i] = p.pool_off[i];
    __syncthreads();

    // tile j of this work-group -> pool block, n tile and local expert (no holes: the last group of
    // blocks may be short)
    auto tile_of = [&](int j, int& b, int& nt, int& le) {
        const int t = logical + j * G;
        if (t < full) {
            const int grp = t / (kGroupBlocks * NT);
            const int rem = t - grp * (kGroupBlocks * NT);
            nt = rem / kGroupBlocks;
            b = grp * kGroupBlocks + (rem - nt * kGroupBlocks);
        } else {
            const int rem = t - full;
            nt = rem / tail;
            b = full / NT + (rem - nt * tail);
        }
        int lo = 0, hi = p.El;              // last expert whose first block is <= b
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sOff[mid] <= b) lo = mid; else hi = mid;
        }
        le = lo;
    };
    // weight row (relative to the tile's first weight row) of B tile row r
    auto b_row = [&](int r) { return kGemm1 ? (r < 128 ? r : p.I - 128 + r) : r; };
    auto a_base = [&](int b) { return (kGemm1 ? p.pool_x : p.l2_x) + (size_t)b * BM * Kdim; };
    auto w_base = [&](int le, int nt) {
        return kGemm1 ? p.w1 + ((size_t)le * (2 * p.I) + nt * 128) * p.H : p.w2 + ((size_t)le * p.H + nt * 256) * p.I;
    };

    // per-lane DMA offsets (fixed for the whole kernel)
    uint32_t a_off[A_INS], b_off[B_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int r = (i * NW + wave) * 8 + (lane >> 3), c = swz_chunk(r, lane & 7);
        a_off[i] = r * Kdim + c * 16;
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int r = (i * NW + wave) * 8 + (lane >> 3), c = swz_chunk(r, lane & 7);
        b_off[i] = b_row(r) * Kdim + c * 16;
    }
    const uint32_t sa_off = (wave * SA_LANES + (lane < SA_LANES ? lane : 0)) * KB * 4;
    uint32_t meta_off[META_INS];
#pragma unroll
    for (int i = 0; i < META_INS; ++i) {
        const int d = wave * META_PER_WAVE + i * 64 + lane;
        meta_off[i] = (uint32_t)(lane + i * 64 < META_PER_WAVE ? d : 0) * 4;
    }

    // issue side: the next step to load, tile ij and K step ikb; per-tile base pointers advance by one
    // K step per issue
    int ij = 0, ikb = 0;
    const uint8_t* iA;
    const uint8_t* iW;
    const uint8_t* iAsf;
    const uint8_t* iWsf;
    const uint8_t* iMeta;
    uint32_t sw_off = 0;
    auto set_issue_tile = [&]() {
        int b, nt, le;
        tile_of(ij, b, nt, le);
        const size_t row0 = (size_t)b * BM;
        iA = a_base(b);
        iW = w_base(le, nt);
        iAsf = reinterpret_cast<const uint8_t*>((kGemm1 ? p.pool_sf : p.l2_sf) + row0 * KB);
        iWsf = reinterpret_cast<const uint8_t*>(kGemm1 ? p.w1_sf + (size_t)le * ((2 * p.I) >> 7) * KB
                                                       : p.w2_sf + (size_t)le * (p.H >> 7) * KB);
        iMeta = reinterpret_cast<const uint8_t*>(p.pool_meta + row0 * 3);
        int blk;
        if (kGemm1) blk = lane == 0 ? nt : (p.I >> 7) + nt;          // gate block, up block
        else blk = nt * 2 + (wn * WROWS) / 128;
        sw_off = (uint32_t)(blk * KB) * 4;
    };
    set_issue_tile();
    auto issue = [&](auto bufc) {
        constexpr int buf = decltype(bufc)::value;
#pragma unroll
        for (int i = 0; i < A_INS; ++i) dma16(iA, a_off[i], &sA[buf][(i * NW + wave) * 1024]);
#pragma unroll
        for (int i = 0; i < B_INS; ++i) dma16(iW, b_off[i], &sB[buf][(i * NW + wave) * 1024]);
        if (lane < SA_LANES) dma4(iAsf, sa_off, &sSA[buf][wave * SA_LANES]);
        if (lane < 2) dma4(iWsf, sw_off, &sSW[buf][wave][0]);
        if (!kGemm1) {
#pragma unroll
            for (int i = 0; i < META_INS; ++i)
                if (lane + i * 64 < META_PER_WAVE)
                    dma4(iMeta, meta_off[i], &sMeta[buf][wave * META_PER_WAVE + i * 64]);
        }
        // advance; past the last step the last step is loaded again (constant DMA count per step)
        if (ikb + 1 < KB) {
            ++ikb;
            iA += 128;
            iW += 128;
            iAsf += 4;
            iWsf += 4;
        } else if (ij + 1 < my_tiles) {
            ikb = 0;
            ++ij;
            set_issue_tile();
        }
    };

    // LDS row of this wave's weight subtile a (GEMM1: the first WN/2 are gate rows, the rest the
    // matching up rows, so gate and up of one output column sit in the same lane)
    int wrow0[WN];
#pragma unroll
    for (int a = 0; a < WN; ++a) {
        if (kGemm1) wrow0[a] = (a < WN / 2 ? 0 : 128) + wn * HC + (a % (WN / 2)) * 16;
        else wrow0[a] = wn * WROWS + a * 16;
    }

    v4f acc[WN][TM];
#pragma unroll
    for (int a = 0; a < WN; ++a)
#pragma unroll
        for (int t = 0; t < TM; ++t) acc[a][t] = v4f{0.f, 0.f, 0.f, 0.f};

    int cj = 0, ckb = 0;      // compute side: tile and K step

    auto epilogue = [&](auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        // lane holds acc[a][t][i]: weight row wrow0[a] + 4g + i, token wm*BM/2 + 16t + rr
        int b, nt, le_unused;
        tile_of(cj, b, nt, le_unused);
        (void)le_unused;
        const size_t row0 = (size_t)b * BM;
        if (kGemm1) {
            constexpr int HA = WN / 2;
            float h[HA][TM][4];
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                float m = 0.f;
#pragma unroll
                for (int a = 0; a < HA; ++a)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float gt = acc[a][t][i], up = acc[a + HA][t][i];
                        const float v = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
                        h[a][t][i] = v;
                        m = fmaxf(m, fabsf(v));
                    }
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                if (g == 0) sRed[wm * (BM / 2) + t * 16 + rr][wn] = m;
            }
            lds_barrier();
            const int I = p.I;
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const int tok = wm * (BM / 2) + t * 16 + rr;
                float am = sRed[tok][0];
#pragma unroll
                for (int w = 1; w < NWN; ++w) am = fmaxf(am, sRed[tok][w]);
                const float sc = fmaxf(am, 1e-4f) / 448.0f;
                const size_t row = row0 + tok;
#pragma unroll
                for (int a = 0; a < HA; ++a) {
                    const int col = nt * 128 + wn * HC + a * 16 + 4 * g;
                    const uint32_t q = cvt_fp8x4(h[a][t][0] / sc, h[a][t][1] / sc, h[a][t][2] / sc,
                                                 h[a][t][3] / sc);
                    *reinterpret_cast<uint32_t*>(p.l2_x + row * I + col) = q;
                    if (p.gemm1_out) {
                        float* go = p.gemm1_out + row * (size_t)(2 * I);
                        *reinterpret_cast<v4f*>(go + col) = acc[a][t];
                        *reinterpret_cast<v4f*>(go + I + col) = acc[a + HA][t];
                    }
                }
                if (wn == 0 && g == 0) p.l2_sf[row * (size_t)(I >> 7) + nt] = sc;
            }
            lds_barrier();      // sRed is rewritten by the next tile
        } else {
            const size_t plane = (size_t)p.S * p.T_max;
            const uint32_t* meta = sMeta[buf];
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const int tok = wm * (BM / 2) + t * 16 + rr;
                const uint32_t ms = meta[tok * 3], mt = meta[tok * 3 + 1], mk = meta[tok * 3 + 2];
                if (ms >= (uint32_t)p.S || mt >= (uint32_t)p.T_max || mk >= (uint32_t)p.K) continue;  // padding
                uint16_t* dst = p.comb + ((size_t)mk * plane + (size_t)ms * p.T_max + mt) * p.H;
#pragma unroll
                for (int a = 0; a < WN; ++a) {
                    const int col = nt * 256 + wn * WROWS + a * 16 + 4 * g;
                    uint2 v;
                    v.x = (uint32_t)f32_to_bf16(acc[a][t][0]) | ((uint32_t)f32_to_bf16(acc[a][t][1]) << 16);
                    v.y = (uint32_t)f32_to_bf16(acc[a][t][2]) | ((uint32_t)f32_to_bf16(acc[a][t][3]) << 16);
                    *reinterpret_cast<uint2*>(dst + col) = v;
                }
            }
        }
#pragma unroll
        for (int a = 0; a < WN; ++a)
#pragma unroll
            for (int t = 0; t < TM; ++t) acc[a][t] = v4f{0.f, 0.f, 0.f, 0.f};
    };

    // one K step on stage buf: wait for it, refill the stage two steps ahead, MFMAs with the
    // promotion pipelined two MFMAs behind, and the epilogue after a tile's last step
    auto step = [&](auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        wait_vm_barrier<DMA_PER_STEP>();        // this stage landed in every wave; stage buf-1 is free
        issue(ic<(buf + 2) % kStages>{});
        // promotion factors: token scale x the wave's weight-block scale (GEMM1: gate and up blocks)
        constexpr int NSW = kGemm1 ? 2 : 1;
        float sc[NSW][TM];
        {
            const float sw0 = sSW[buf][wave][0], sw1 = sSW[buf][wave][1];
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const float sa = sSA[buf][wm * (BM / 2) + t * 16 + rr];
                sc[0][t] = sa * sw0;
                if (kGemm1) sc[NSW - 1][t] = sa * sw1;
            }
        }
        v8i xf[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) xf[t] = load_frag(sA[buf], wm * (BM / 2) + t * 16, lane);
        v8i wf[2];
        wf[0] = load_frag(sB[buf], wrow0[0], lane);
        v4f pr[3];
#pragma unroll
        for (int i = 0; i < NMF + 2; ++i) {
            if (i < NMF) {
                const int a = i / TM, t = i % TM;
                if (t == 0 && a + 1 < WN) wf[(a + 1) & 1] = load_frag(sB[buf], wrow0[a + 1], lane);
                pr[i % 3] = mfma_fp8(wf[a & 1], xf[t], v4f{0.f, 0.f, 0.f, 0.f});
            }
            if (i >= 2) {
                const int k = i - 2, a = k / TM, t = k % TM;
                const int si = (kGemm1 && a >= WN / 2) ? NSW - 1 : 0;
                acc[a][t] += sc[si][t] * pr[k % 3];
            }
        }
        if (++ckb == KB) {
            epilogue(bufc);
            ckb = 0;
            ++cj;
        }
    };

    issue(ic<0>{});
    issue(ic<1>{});
    for (int s = 0; s < nsteps; s += kStages) {
        step(ic<0>{});
        if (s + 1 >= nsteps) break;
        step(ic<1>{});
        if (s + 2 >= nsteps) break;
        step(ic<2>{});
    }
    wait_all_vm();      // no LDS DMA may still be landing when the work-group ends
}

template <int BM, bool kGemm1>
hipError_t launch(const Params& p, int num_cus, hipStream_t stream) {
    int grid = (num_cus + 7) / 8 * 8;
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, kWaves, kGemm1>), dim3(grid), dim3(kWaves * 64), 0, stream, p);
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
